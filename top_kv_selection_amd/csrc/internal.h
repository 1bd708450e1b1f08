// internal.h -- host-side declarations shared by the CSA2 translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace csa2 {

// ---- kernel launches
// Every kernel of the library is launched through launch(), which carries the
// measurement hook of csa2_profile_begin: while it is armed, launches whose
// name matches are given HIP start/stop events (hipExtLaunchKernel records
// the kernel's own execution interval in them).  Launches into a stream that
// is capturing a graph are never timed.
bool profile_events(const char *name, hipStream_t st, hipEvent_t &start, hipEvent_t &stop);

// Errors of the launch itself are left for the caller's hipGetLastError().
template <typename... KArgs, typename... Args>
inline void launch(const char *name, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t st,
                   Args &&...args)
{
    std::tuple<KArgs...> held(static_cast<KArgs>(args)...);
    void *argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    std::apply([&](auto &...a) {
        int k = 0;
        ((argv[k++] = (void *)&a), ...);
    }, held);
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (profile_events(name, st, e0, e1))
        (void)hipExtLaunchKernel((const void *)kernel, grid, block, argv, 0, st, e0, e1, 0);
    else
        (void)hipLaunchKernel((const void *)kernel, grid, block, argv, 0, st);
}

constexpr int kSelectThreads = 512;     // threads of a scoring or many-query selection workgroup
constexpr int kSelectWideThreads = 1024; // threads of a one-query-per-workgroup select launch (16 keys each)
constexpr int kTargetWorkgroups = 512;  // ~2 per CU on a 256-CU MI355X
constexpr int kMaxCandidates = 16384;   // P*B cap: candidates one query may score
constexpr int kMaxRatio = 256;          // largest csa2_cfg.ratio (tokens per main-KV entry)
constexpr int kTailExclude = 1;         // csa2_tail values the kernels test
constexpr int kTailWhole = 2;

// Last main-KV entry a query at token position t sees.  With `ratio` tokens
// compressed into one entry (the "CSA2(ratio, mode)" of the V4.1 Flash
// page's architecture figure), entry j stands for tokens j*ratio ..
// j*ratio + ratio - 1 and exists once the last of them has arrived, so the
// visible entries are 0 .. (t + 1) / ratio - 1; -1 when none is complete yet.
// Ratio 1 (or 0, the default) is one entry per token.  Token positions are
// >= 0 and may reach INT32_MAX with large ratios, so t + 1 is taken unsigned.
__host__ __device__ inline int main_pos(int t, int ratio)
{
    return ratio > 1 ? (int)(((uint32_t)t + 1u) / (uint32_t)ratio) - 1 : t;
}

// Blocks eligible for a query whose last visible entry is t: every block
// holding a visible entry, or only the complete ones when a partial own block
// is excluded; none when no entry is visible (t < 0).
__host__ __device__ inline int eligible_blocks(int t, int B, int tail)
{
    if (t < 0) return 0;
    return tail == kTailExclude ? (t + 1) / B : t / B + 1;
}

struct BlockKeysParams {
    const int8_t *k_idx;
    int8_t *k_blk;
    int T, B, nblk, blk_begin, blk_end;
};

// New tokens written into the caches (row i: sequence seq[i], position pos[i]).
struct AppendParams {
    const int32_t *seq, *pos;
    const int8_t *new_k_idx;
    const void *new_k, *new_v;
    int8_t *k_idx;
    void *k_main, *v_main;
    int8_t *k_blk;                 // nullptr: no block keys
    int n_new, T, B, nblk, d_idx, row_bytes;
};

struct IndexParams {
    const int8_t *q_idx;
    const int32_t *q_seq, *q_pos;
    const int8_t *k_idx, *k_blk;
    int8_t *k_blk_store;    // non-null: store each query's own block key when the query completes it
    uint32_t *tok_hist_clear;   // non-null (fused layer group): zero [n_q][2048] token histograms
    int T, B, P, n_q, G, chunk, nblk;
    int tail;               // csa2_tail reading of a partial own block
    int ratio;              // tokens per main-KV entry: q_pos are tokens, the caches entries
    uint32_t *ws_keys;
    int64_t ws_stride;
    uint32_t *ws_hist;      // [n_q][2048] top-11-bit histograms (split launches)
    int32_t *blk_ids, *blk_cnt;
};

struct TopkParams {
    const int8_t *q_idx;
    const int32_t *q_seq, *q_pos;
    const int8_t *k_idx;
    const int32_t *blk_ids, *blk_cnt;
    int T, B, P, K, n_q, G, chunk;
    int tail;               // csa2_tail reading of a partial own block
    int ratio;              // tokens per main-KV entry (see main_pos)
    uint32_t *ws_keys;
    int64_t ws_stride;
    uint32_t *ws_hist;
    int32_t *topk, *topk_cnt;
    // dense token Top-K of a prompt whose pools are whole prefixes and whose
    // pool ids are not stored: the kernel also writes the pool counts and
    // (Full layer) the key of every block a query completes, in place of the
    // block pass (non-null only there)
    int32_t *pool_cnt_out;
    int8_t *k_blk_store;
    int nblk;
};

struct AttendParams {
    const void *q;
    const int32_t *q_seq, *q_pos;
    const void *k_main, *v_main;
    int n_seq, T;
    const void *k_swa, *v_swa;
    int swa_first, swa_len;
    const int32_t *topk, *topk_cnt;
    int K, W, n_q, n_layers, H;
    float scale_log2;       // logit scale times log2(e)
    void *out;
    float *lse;
    float *ws_part;         // chunk records [L][n_q][H/16][n_splits] (chunk kernel)
    int row_blocks;         // row kernel: items in blocks per workgroup (1) or strided over the grid (0)
    // fused token selection (layer-group decode path): the key list comes from
    // the token keys instead of topk, and topk/topk_cnt are written
    const uint32_t *sel_keys;   // [n_q][sel_stride] token keys
    int64_t sel_stride;
    const uint32_t *sel_hist;   // [n_q][2048] their top-11-bit histogram
    const int32_t *sel_pool;    // [n_q][sel_P] pooled block ids
    const int32_t *sel_pool_cnt;
    int sel_B, sel_P;
    int32_t *topk_out, *topk_cnt_out;
    uint32_t *blk_hist_clear;   // optional: [n_q][2048] histograms to zero once read
    int n_splits;           // chunk kernel: records per item (main chunks + window chunks)
    int keys_per_split;     // MFMA kernel: key-list slots staged (whole steps)
    int n_q_pad;            // n_q rounded up to a multiple of 8 (XCD-aware numbering)
    int n_mc, n_wc;         // chunk kernel: main-list chunks per query, window chunks per (query, layer)
};

// Work split of one selection launch: G workgroups per query, `chunk` items each.
struct SelectPlan {
    int G, chunk;
    bool split;       // scores go through the workspace (G > 1 or too many for LDS)
    size_t key_bytes; // workspace bytes for the scores
    bool dense = false;   // token Top-K: every pool is the whole prefix (MFMA tile kernel)
    bool all = false;     // block pass: every pool is the whole prefix (no scoring)
};

struct AttendPlan {
    bool mfma;    // bf16, D = 128, H a multiple of 16: an MFMA kernel; else the generic one
    bool rows;    // many items: one wave per (query, layer, head group), no splits
    int n_splits, keys_per_split;   // as in AttendParams
    size_t part_bytes;
    int kpw;      // keys per wave and step of the MFMA kernel
    bool chunks;  // few items: key lists cut into chunks (k_attend_chunks + k_attend_combine)
    int n_mc, n_wc;   // main-list chunks per query, window chunks per (query, layer)
};

// Workspace head bytes of a selection launch: one 2048-bin histogram per
// query (split launches only); zero between calls.
size_t select_head_bytes(int n_q, bool split);

SelectPlan plan_index(int n_q, int T, int B, int P, int d_idx);
SelectPlan plan_topk(int n_q, int T, int B, int P, int K, int d_idx);
AttendPlan plan_attend(int n_q, int n_layers, int H, int D, int K, int W, int dtype);

hipError_t launch_block_keys(const BlockKeysParams &p, int n_seq, int d_idx, hipStream_t st);
hipError_t launch_append(const AppendParams &p, hipStream_t st);
hipError_t launch_index_blocks(const IndexParams &p, const SelectPlan &plan, int d_idx,
                               hipStream_t st, bool with_select = true);
hipError_t launch_topk_tokens(const TopkParams &p, const SelectPlan &plan, int d_idx, hipStream_t st);
hipError_t launch_attend(const AttendParams &p, const AttendPlan &plan, int D, int dtype,
                         hipStream_t st, bool fused_select = false);

// (query, layer, head group) items that take the row kernel: more than one
// round of the one-workgroup-per-item MFMA kernel (a workgroup per CU), whose
// second round doubles its time (384 items: 310.9 against 222.9 us per replay
// step; at 256 items the MFMA kernel is 1.5-3 % faster)
constexpr int kRowItemsMin = kTargetWorkgroups / 2 + 1;
constexpr int kWinItemsMin = 1024;      // window-only items that take the shared-window kernel (32 queries a workgroup)
constexpr int kDenseMaxT = 16384;       // longest context of the dense (MFMA tile) token Top-K
constexpr int kDenseMinQueries = 256;   // queries per call below which the per-query kernels run
constexpr int kAttendRowChunk = 2048;   // key-list entries one attention workgroup stages at once
constexpr int kFusedPoolLds = 2048;     // pooled block ids the fused attention keeps in LDS
constexpr int kFusedEligMax = 32768;    // eligible blocks per query the fused layer group takes (256K tokens at B = 8)
hipError_t launch_fill_zero(void *ws, size_t bytes, hipStream_t st);
// Layer-group decode: pool selection (from a split block pass's keys and
// histogram) and token scoring in one launch; ceil(P / pool_tokens_slots)
// workgroups per query.  Requires n_elig_max <= kFusedEligMax and P <= kFusedPoolLds.
int pool_tokens_slots(int n_q, int P, int B);
// The fused decode layer group as one launch (single.hip): its four phases in
// one kernel, handing over per query through counters `ctr` (single_ctr_bytes
// of zeroed workspace, left zeroed).  Needs an attention plan with chunks.
size_t single_ctr_bytes(int n_q);
hipError_t launch_decode_single(const IndexParams &ip, const TopkParams &tp, const AttendParams &ap,
                                const AttendPlan &pl, int d_idx, uint32_t *ctr, hipStream_t st);
hipError_t launch_pool_tokens(const IndexParams &ip, const TopkParams &tp, int d_idx, hipStream_t st);

}  // namespace csa2
