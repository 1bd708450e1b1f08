// api.hip -- the C ABI declared in include/csa2.h: argument checks, workspace
// layout and the mode dispatch of a CSA2 layer group.
//
// Workspace layout: state that must be zero between calls (the selection
// histograms) at the head, scratch (scores, split records) at the tail.  The
// kernels leave the head zeroed again, so a zero-filled workspace sized by
// csa2_workspace_bytes for the largest call serves every call in stream order.
#include <math.h>
#include <string.h>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "csa2.h"
#include "device_common.h"
#include "internal.h"

using namespace csa2;

// ---- measurement hook of csa2_profile_begin / csa2_profile_end: a bounded
// list of HIP event pairs handed to matching launches (see launch() in
// internal.h), in launch order.
namespace csa2 {
namespace {
struct ProfRec {
    char name[32];
    hipEvent_t start, stop;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_armed{false};
char g_prof_filter[64];
std::vector<ProfRec> g_prof;
size_t g_prof_used = 0;

void prof_release()
{
    for (ProfRec &r : g_prof) {
        hipEventDestroy(r.start);
        hipEventDestroy(r.stop);
    }
    g_prof.clear();
    g_prof_used = 0;
}
}  // namespace

bool profile_events(const char *name, hipStream_t st, hipEvent_t &start, hipEvent_t &stop)
{
    if (!g_prof_armed.load(std::memory_order_relaxed)) return false;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_armed.load(std::memory_order_relaxed) || g_prof_used >= g_prof.size()) return false;
    if (g_prof_filter[0] && !strstr(name, g_prof_filter)) return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
    ProfRec &r = g_prof[g_prof_used++];
    strncpy(r.name, name, sizeof(r.name) - 1);
    r.name[sizeof(r.name) - 1] = 0;
    start = r.start;
    stop = r.stop;
    return true;
}
}  // namespace csa2

// ---- scratch of csa2_layer_group_static: a file-scope device array (each
// GPU the library runs on holds its own copy until the process ends).  Host
// code never uses the array's name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device with that
// device current, and is what the kernels receive.
static constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array.
int32_t static_scratch(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return CSA2_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return CSA2_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA2_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return CSA2_OK;
}
}  // namespace

namespace {

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int32_t check_cfg(const csa2_cfg *c)
{
    if (!c) return CSA2_E_NULL;
    if (c->dtype != CSA2_F32 && c->dtype != CSA2_BF16) return CSA2_E_DTYPE;
    if (c->block < 1 || c->block > 16 || c->pool < 1 || c->top_k < 0 || c->window < 0 ||
        c->window > 1024 || c->n_heads < 1 || c->n_heads > 128)
        return CSA2_E_SHAPE;
    if ((long long)c->pool * c->block > kMaxCandidates || c->top_k > c->pool * c->block) return CSA2_E_SHAPE;
    if (c->top_k + c->window < 1) return CSA2_E_SHAPE;
    if (c->d_idx != 32 && c->d_idx != 64) return CSA2_E_UNSUPPORTED;
    if (c->head_dim != 64 && c->head_dim != 128) return CSA2_E_UNSUPPORTED;
    if (!(c->scale >= 0.f) || !isfinite(c->scale)) return CSA2_E_SHAPE;
    if (c->tail != CSA2_TAIL_VISIBLE && c->tail != CSA2_TAIL_EXCLUDE && c->tail != CSA2_TAIL_WHOLE)
        return CSA2_E_SHAPE;
    // compressed main-KV: a query before the first complete entry attends to
    // its window alone, so a window is required
    if (c->ratio < 0 || c->ratio > kMaxRatio || (c->ratio > 1 && c->window < 1)) return CSA2_E_SHAPE;
    return CSA2_OK;
}

int32_t check_sizes(int32_t n_q, int32_t n_seq, int32_t T)
{
    if (n_q < 0 || n_seq < 1 || T < 1 || T > (1 << 24)) return CSA2_E_SHAPE;
    return CSA2_OK;
}



// Workspace layout.  Every call keeps the state that must be zero between
// calls at the head of the workspace and its scratch at the tail end, and
// leaves its head zero again:
//   head: [0, hist_bytes(n_q)), per-query 2048-bin selection histograms (split
//         selections and the fused layer group);
//   tail: the last round_up(scratch) bytes (keys, token histograms, chunk
//         records).
// csa2_workspace_bytes(N, T, L) is an upper bound of every head plus an upper
// bound of every scratch that a call with n_q <= N, T' <= T and n_layers <= L
// may use, so that no call's scratch reaches into another call's head.
size_t hist_bytes(int n_q) { return round_up((size_t)n_q * kRadixBins * sizeof(uint32_t)); }

struct Region {
    uint32_t *ctr;     // head: zero between calls
    void *data;        // tail: scratch
};

// `ctr_bytes` at the head, `data_bytes` at the tail of the workspace.
int32_t carve(void *ws, size_t ws_bytes, size_t ctr_bytes, size_t data_bytes, Region &r)
{
    r = {nullptr, nullptr};
    if (ctr_bytes == 0 && data_bytes == 0) return CSA2_OK;
    if (!ws) return CSA2_E_WORKSPACE;
    if (!aligned16(ws)) return CSA2_E_ALIGN;
    const size_t head = round_up(ctr_bytes), tail = round_up(data_bytes);
    if (ws_bytes < head + tail) return CSA2_E_WORKSPACE;
    r.ctr = (uint32_t *)ws;
    r.data = (char *)ws + ((ws_bytes - tail) / kAlign) * kAlign;
    return CSA2_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_E_HIP; }

float scale_log2_of(const csa2_cfg *c)
{
    const float scale = (c->scale > 0.f) ? c->scale : 1.0f / sqrtf((float)c->head_dim);
    return scale * 1.4426950408889634f;
}

int32_t do_index(const csa2_cfg *c, int32_t n_q, const int8_t *q_idx, const int32_t *q_seq,
                 const int32_t *q_pos, const int8_t *k_idx, const int8_t *k_blk, int32_t n_seq,
                 int32_t T, int32_t *blk_ids, int32_t *blk_cnt, void *ws, size_t ws_bytes,
                 hipStream_t st, bool launch, int8_t *k_blk_store = nullptr)
{
    const SelectPlan pl = plan_index(n_q, T, c->block, c->pool, c->d_idx);
    // the ids may be left unstored only where every pool is the whole prefix
    // with no complete block (T < B) k_blk is empty and may be NULL: no kernel reads or writes it
    if (!q_idx || !q_seq || !q_pos || !k_idx || (!k_blk && T / c->block > 0) || !blk_cnt || (!blk_ids && !pl.all))
        return CSA2_E_NULL;
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(k_blk) || !aligned4(q_seq) ||
        !aligned4(q_pos) || !aligned4(blk_ids) || !aligned4(blk_cnt))
        return CSA2_E_ALIGN;
    Region r;
    if (int32_t e = carve(ws, ws_bytes, select_head_bytes(n_q, pl.split), pl.key_bytes, r)) return e;
    if (!launch) return CSA2_OK;
    IndexParams p{};
    p.q_idx = q_idx; p.q_seq = q_seq; p.q_pos = q_pos; p.k_idx = k_idx; p.k_blk = k_blk;
    p.k_blk_store = k_blk_store;
    p.T = T; p.B = c->block; p.P = c->pool; p.n_q = n_q; p.G = pl.G; p.chunk = pl.chunk; p.tail = c->tail;
    p.ratio = c->ratio;
    p.nblk = T / c->block;
    p.ws_keys = (uint32_t *)r.data;
    p.ws_stride = ((long long)(T - 1) / c->block + 1 + 3) / 4 * 4;   // rows 16-byte aligned
    p.ws_hist = r.ctr;
    p.blk_ids = blk_ids; p.blk_cnt = blk_cnt;
    return hip_status(launch_index_blocks(p, pl, c->d_idx, st));
}

int32_t do_topk(const csa2_cfg *c, int32_t n_q, const int8_t *q_idx, const int32_t *q_seq,
                const int32_t *q_pos, const int8_t *k_idx, int32_t T, const int32_t *blk_ids,
                const int32_t *blk_cnt, int32_t *topk, int32_t *topk_cnt, void *ws,
                size_t ws_bytes, hipStream_t st, bool launch, int32_t *pool_cnt_out = nullptr,
                int8_t *k_blk_store = nullptr)
{
    if (c->top_k < 1) return CSA2_E_SHAPE;
    const bool whole_prefix = (long long)(T - 1) / c->block + 1 <= c->pool;
    if (!q_idx || !q_seq || !q_pos || !k_idx || !blk_cnt || !topk || !topk_cnt || (!blk_ids && !whole_prefix))
        return CSA2_E_NULL;
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned4(q_seq) || !aligned4(q_pos) ||
        !aligned4(blk_ids) || !aligned4(blk_cnt) || !aligned4(topk) || !aligned4(topk_cnt))
        return CSA2_E_ALIGN;
    const SelectPlan pl = plan_topk(n_q, T, c->block, c->pool, c->top_k, c->d_idx);
    Region r;
    if (int32_t e = carve(ws, ws_bytes, select_head_bytes(n_q, pl.split), pl.key_bytes, r)) return e;
    if (!launch) return CSA2_OK;
    TopkParams p{};
    p.q_idx = q_idx; p.q_seq = q_seq; p.q_pos = q_pos; p.k_idx = k_idx;
    p.blk_ids = blk_ids; p.blk_cnt = blk_cnt;
    p.T = T; p.B = c->block; p.P = c->pool; p.K = c->top_k; p.n_q = n_q; p.G = pl.G; p.tail = c->tail;
    p.ratio = c->ratio;
    p.chunk = pl.chunk;
    p.ws_keys = (uint32_t *)r.data;
    p.ws_stride = ((long long)c->pool * c->block + 3) / 4 * 4;
    p.ws_hist = r.ctr;
    p.topk = topk; p.topk_cnt = topk_cnt;
    if (pool_cnt_out) {   // only the dense kernel stands in for the block pass
        if (!pl.dense || blk_ids) return CSA2_E_SHAPE;
        p.pool_cnt_out = pool_cnt_out;
        p.k_blk_store = k_blk_store;
        p.nblk = T / c->block;
    }
    return hip_status(launch_topk_tokens(p, pl, c->d_idx, st));
}

int32_t do_attend(const csa2_cfg *c, int32_t n_layers, int32_t n_q, const void *q,
                  const int32_t *q_seq, const int32_t *q_pos, const void *k_main,
                  const void *v_main, int32_t n_seq, int32_t T, const void *k_swa,
                  const void *v_swa, int32_t swa_first, int32_t swa_len, const int32_t *topk,
                  const int32_t *topk_cnt, void *out, float *lse, void *ws, size_t ws_bytes,
                  hipStream_t st, bool launch)
{
    if (n_layers < 1) return CSA2_E_SHAPE;
    if (!q || !q_seq || !q_pos || !out) return CSA2_E_NULL;
    const bool has_main = topk != nullptr;
    if (has_main != (topk_cnt != nullptr)) return CSA2_E_NULL;
    if (has_main && c->top_k < 1) return CSA2_E_SHAPE;
    if (has_main && (!k_main || !v_main)) return CSA2_E_NULL;
    if (c->window > 0 && (!k_swa || !v_swa)) return CSA2_E_NULL;
    if (!has_main && c->window < 1) return CSA2_E_SHAPE;
    // tokens a sequence may hold: T, or with compressed main-KV the tokens of
    // its T entries plus an incomplete group
    const int per_entry = std::max(c->ratio, 1);
    const long long n_tok = (long long)T * per_entry + (per_entry - 1);
    if (c->window > 0 && (swa_len < 1 || swa_first < 0 || swa_first >= n_tok || swa_len > n_tok))
        return CSA2_E_SHAPE;
    const void *dev16[] = {q, out, k_main, v_main, k_swa, v_swa};
    for (const void *ptr : dev16)
        if (ptr && !aligned16(ptr)) return CSA2_E_ALIGN;
    if (!aligned4(q_seq) || !aligned4(q_pos) || (topk && !aligned4(topk)) ||
        (topk_cnt && !aligned4(topk_cnt)) || (lse && !aligned4(lse)))
        return CSA2_E_ALIGN;
    const int W = c->window;
    const int K = has_main ? c->top_k : 0;
    const AttendPlan pl = plan_attend(n_q, n_layers, c->n_heads, c->head_dim, K, W, c->dtype);
    Region r;
    if (int32_t e = carve(ws, ws_bytes, 0, pl.part_bytes, r))
        return e;
    if (!launch) return CSA2_OK;
    AttendParams p{};
    p.q = q; p.q_seq = q_seq; p.q_pos = q_pos;
    // a window-only call reads no main rows; point them at valid memory anyway
    p.k_main = k_main ? k_main : q;
    p.v_main = v_main ? v_main : q;
    p.n_seq = n_seq; p.T = T;
    p.k_swa = k_swa; p.v_swa = v_swa; p.swa_first = swa_first; p.swa_len = std::max(swa_len, 1);
    p.topk = topk; p.topk_cnt = topk_cnt; p.K = c->top_k; p.W = W;
    p.n_q = n_q; p.n_layers = n_layers; p.H = c->n_heads;
    p.scale_log2 = scale_log2_of(c);
    p.out = out; p.lse = lse;
    p.ws_part = (float *)r.data;
    return hip_status(launch_attend(p, pl, c->head_dim, c->dtype, st));
}

// ---- fused decode layer group: block scoring -> pool selection and token
// scoring in one launch -> token Top-K inside the attention launch ->
// combine (4 launches instead of 6).  Used when the selections are split over
// workgroups (few queries), the keys of a query fit one workgroup's
// registers, and the attention takes the MFMA path.
struct FusedPlan {
    bool ok;
    SelectPlan idx, tok;
    AttendPlan att;
    int64_t blk_stride, tok_stride;
    size_t head;                                    // block histograms
    size_t blk_off, tok_off, tok_hist_off, part_off, tail;   // scratch (at the tail end)
};

FusedPlan plan_fused(const csa2_cfg *c, int n_q, int T, int n_layers)
{
    FusedPlan f{};
    const long long n_elig_max = (long long)(T - 1) / c->block + 1;
    f.idx = plan_index(n_q, T, c->block, c->pool, c->d_idx);
    f.tok = plan_topk(n_q, T, c->block, c->pool, c->top_k, c->d_idx);
    f.att = plan_attend(n_q, n_layers, c->n_heads, c->head_dim, c->top_k, c->window, c->dtype);
    f.ok = c->top_k >= 1 && f.idx.split && f.tok.split && n_elig_max <= kFusedEligMax && f.att.mfma && !f.att.rows &&
           (f.att.chunks || f.att.keys_per_split <= kAttendRowChunk) && c->pool <= kFusedPoolLds;
    f.blk_stride = (n_elig_max + 3) / 4 * 4;
    f.tok_stride = ((long long)c->pool * c->block + 3) / 4 * 4;
    f.head = hist_bytes(n_q) + single_ctr_bytes(n_q);   // block histograms, then the single launch's counters
    size_t off = 0;
    f.blk_off = off;      off += round_up((size_t)n_q * f.blk_stride * 4);
    f.tok_off = off;      off += round_up((size_t)n_q * f.tok_stride * 4);
    f.tok_hist_off = off; off += round_up((size_t)n_q * 2048 * 4);
    f.part_off = off;     off += round_up(f.att.part_bytes);
    f.tail = off;
    return f;
}

int32_t do_block_keys(const csa2_cfg *c, const int8_t *k_idx, int32_t n_seq, int32_t T,
                      int32_t blk_begin, int32_t blk_end, int8_t *k_blk, hipStream_t st, bool launch)
{
    const int nblk = T / c->block;   // no complete block: k_blk is empty and may be NULL
    if (!k_idx || (!k_blk && nblk > 0)) return CSA2_E_NULL;
    if (!aligned16(k_idx) || !aligned16(k_blk)) return CSA2_E_ALIGN;
    blk_begin = std::max(blk_begin, 0);
    blk_end = std::min(blk_end, nblk);
    if (!launch || blk_begin >= blk_end) return CSA2_OK;
    BlockKeysParams p{k_idx, k_blk, T, c->block, nblk, blk_begin, blk_end};
    return hip_status(launch_block_keys(p, n_seq, c->d_idx, st));
}

// Whether some call at a context of at most T positions may take the fused
// decode path (its other conditions only narrow it further).
bool fused_possible(const csa2_cfg *c, int T)
{
    const AttendPlan one = plan_attend(1, 1, c->n_heads, c->head_dim, c->top_k, c->window, c->dtype);
    const long long n_elig_max = (long long)(T - 1) / c->block + 1;
    return one.chunks && c->top_k >= 1 && c->pool <= kFusedPoolLds && n_elig_max > c->pool;
}

// Upper bound of the scratch of every call with n_q' <= n_q, T' <= T and
// n_layers' <= n_layers (each term is monotone in the sizes within the regime
// that uses it):
//  * split selections: keys of n_q' queries; a launch splits only below
//    kTargetWorkgroups queries, or (block pass) beyond kLdsKeys eligible blocks,
//    and the token Top-K of kDenseMinQueries or more prompt queries whose pools
//    are whole prefixes keeps no keys;
//  * chunked attention: records of fewer than kTargetWorkgroups / 2 items;
//  * fused layer group: block and token keys, token histograms and records of
//    fewer than kTargetWorkgroups / 2 items, at contexts up to kFusedEligMax
//    blocks.
size_t scratch_bound(const csa2_cfg *c, int n_q, int T, int n_layers)
{
    const int n_items = kTargetWorkgroups / 2 - 1;
    size_t b = 0;
    // the regimes change at kDenseMinQueries (dense token Top-K) and at
    // kTargetWorkgroups (no split below it)
    for (int n : {n_q, std::min(n_q, kTargetWorkgroups - 1), std::min(n_q, kDenseMinQueries - 1)}) {
        b = std::max(b, plan_index(n, T, c->block, c->pool, c->d_idx).key_bytes);
        b = std::max(b, plan_topk(n, T, c->block, c->pool, c->top_k, c->d_idx).key_bytes);
    }
    const AttendPlan one = plan_attend(1, 1, c->n_heads, c->head_dim, c->top_k, c->window, c->dtype);
    const int HG = std::max(1, c->n_heads / 16);
    const long long att_items = std::min<long long>((long long)n_q * n_layers * HG, n_items);
    const size_t records = one.chunks ? round_up(one.part_bytes / HG * (size_t)att_items) : 0;
    b = std::max(b, records);
    const long long n_elig_max = (long long)(T - 1) / c->block + 1;
    if (fused_possible(c, T)) {
        const int n_f = std::min(n_q, n_items);
        const long long blk_stride = (std::min<long long>(n_elig_max, kFusedEligMax) + 3) / 4 * 4;
        const long long tok_stride = ((long long)c->pool * c->block + 3) / 4 * 4;
        const size_t fused = round_up((size_t)n_f * blk_stride * 4) + round_up((size_t)n_f * tok_stride * 4) +
                             round_up((size_t)n_f * kRadixBins * 4) + records;
        b = std::max(b, fused);
    }
    return round_up(b);
}

// Upper bound of the head of every call with n_q' <= n_q, T' <= T and
// n_layers' <= n_layers: the histograms of the queries of a split selection
// (splits happen below kTargetWorkgroups queries -- for the token Top-K of a
// prompt whose pools are whole prefixes, only below kDenseMinQueries -- or at
// any count beyond kLdsKeys eligible blocks, and less often at smaller T'),
// and of a fused layer group (fewer than kTargetWorkgroups / 2 queries).
size_t head_bound(const csa2_cfg *c, int n_q, int T)
{
    size_t b = 0;
    for (int n : {n_q, std::min(n_q, kTargetWorkgroups - 1), std::min(n_q, kDenseMinQueries - 1)})
        if (plan_index(n, T, c->block, c->pool, c->d_idx).split ||
            plan_topk(n, T, c->block, c->pool, c->top_k, c->d_idx).split)
            b = std::max(b, hist_bytes(n));
    if (fused_possible(c, T)) {
        const int n_f = std::min(n_q, kTargetWorkgroups / 2 - 1);
        b = std::max(b, hist_bytes(n_f) + single_ctr_bytes(n_f));
    }
    return b;
}

int32_t fused_layer_group(const csa2_cfg *c, int32_t mode, int32_t n_layers, int32_t n_q,
                          const int8_t *q_idx, const int32_t *q_seq, const int32_t *q_pos,
                          const int8_t *k_idx, int8_t *k_blk, int32_t blk_update_begin,
                          int32_t n_seq, int32_t T, const void *q, const void *k_main,
                          const void *v_main, const void *k_swa, const void *v_swa,
                          int32_t swa_first, int32_t swa_len, int32_t *blk_ids, int32_t *blk_cnt,
                          int32_t *topk, int32_t *topk_cnt, void *out, float *lse, void *ws,
                          size_t ws_bytes, hipStream_t st, const FusedPlan &f, bool launch, bool single)
{
    if (single && !f.att.chunks) return CSA2_E_UNSUPPORTED;
    // the argument checks of the separate stages (nothing launched)
    if (int32_t e = do_index(c, n_q, q_idx, q_seq, q_pos, k_idx, k_blk, n_seq, T, blk_ids, blk_cnt,
                             ws, ws_bytes, st, false))
        return e;
    if (int32_t e = do_topk(c, n_q, q_idx, q_seq, q_pos, k_idx, T, blk_ids, blk_cnt, topk, topk_cnt,
                            ws, ws_bytes, st, false))
        return e;
    if (int32_t e = do_attend(c, n_layers, n_q, q, q_seq, q_pos, k_main, v_main, n_seq, T, k_swa, v_swa,
                              swa_first, swa_len, topk, topk_cnt, out, lse, ws, ws_bytes, st, false))
        return e;
    if (mode == CSA2_FULL)
        if (int32_t e = do_block_keys(c, k_idx, n_seq, T, blk_update_begin, T / c->block, k_blk, st, false))
            return e;
    Region r;
    if (int32_t e = carve(ws, ws_bytes, f.head, f.tail, r)) return e;
    if (!launch) return CSA2_OK;
    uint32_t *head = r.ctr;
    char *tail = (char *)r.data;
    uint32_t *blk_keys = (uint32_t *)(tail + f.blk_off);
    uint32_t *tok_keys = (uint32_t *)(tail + f.tok_off);
    uint32_t *tok_hist = (uint32_t *)(tail + f.tok_hist_off);
    float *part = (float *)(tail + f.part_off);

    if (mode == CSA2_FULL)
        if (int32_t e = do_block_keys(c, k_idx, n_seq, T, blk_update_begin, T / c->block, k_blk, st, true))
            return e;
    IndexParams ip{};
    ip.q_idx = q_idx; ip.q_seq = q_seq; ip.q_pos = q_pos; ip.k_idx = k_idx; ip.k_blk = k_blk;
    ip.k_blk_store = mode == CSA2_FULL ? k_blk : nullptr;
    ip.tok_hist_clear = tok_hist;
    ip.T = T; ip.B = c->block; ip.P = c->pool; ip.n_q = n_q; ip.G = f.idx.G; ip.chunk = f.idx.chunk;
    ip.tail = c->tail;
    ip.ratio = c->ratio;
    ip.nblk = T / c->block;
    ip.ws_keys = blk_keys; ip.ws_stride = f.blk_stride; ip.ws_hist = head;
    ip.blk_ids = blk_ids; ip.blk_cnt = blk_cnt;

    TopkParams tp{};
    tp.q_idx = q_idx; tp.q_seq = q_seq; tp.q_pos = q_pos; tp.k_idx = k_idx;
    tp.blk_ids = blk_ids; tp.blk_cnt = blk_cnt;
    tp.T = T; tp.B = c->block; tp.P = c->pool; tp.K = c->top_k; tp.n_q = n_q; tp.tail = c->tail;
    tp.ratio = c->ratio;
    tp.G = f.tok.G; tp.chunk = f.tok.chunk;
    tp.ws_keys = tok_keys; tp.ws_stride = f.tok_stride; tp.ws_hist = tok_hist;
    tp.topk = topk; tp.topk_cnt = topk_cnt;

    AttendParams ap{};
    ap.q = q; ap.q_seq = q_seq; ap.q_pos = q_pos; ap.k_main = k_main; ap.v_main = v_main;
    ap.n_seq = n_seq; ap.T = T;
    ap.k_swa = k_swa; ap.v_swa = v_swa; ap.swa_first = swa_first; ap.swa_len = std::max(swa_len, 1);
    ap.topk = topk; ap.topk_cnt = topk_cnt; ap.K = c->top_k; ap.W = c->window;
    ap.n_q = n_q; ap.n_layers = n_layers; ap.H = c->n_heads;
    ap.scale_log2 = scale_log2_of(c);
    ap.out = out; ap.lse = lse; ap.ws_part = part;
    ap.sel_keys = tok_keys; ap.sel_stride = f.tok_stride; ap.sel_hist = tok_hist;
    ap.sel_pool = blk_ids; ap.sel_pool_cnt = blk_cnt; ap.sel_B = c->block; ap.sel_P = c->pool;
    ap.topk_out = topk; ap.topk_cnt_out = topk_cnt; ap.blk_hist_clear = head;
    if (single)
        return hip_status(launch_decode_single(ip, tp, ap, f.att, c->d_idx,
                                               (uint32_t *)((char *)head + hist_bytes(n_q)), st));
    // block scoring (keys and histogram to the workspace)
    if (int32_t e = hip_status(launch_index_blocks(ip, f.idx, c->d_idx, st, false))) return e;
    // pool selection + token scoring in one launch (each scoring workgroup
    // redoes the pool selection); the Top-K is taken inside the attention
    // launch, whose writer also zeroes the block histogram
    if (int32_t e = hip_status(launch_pool_tokens(ip, tp, c->d_idx, st))) return e;
    return hip_status(launch_attend(ap, f.att, c->head_dim, c->dtype, st, true));
}

// csa2_layer_group with the stream given; launch = false only checks every
// argument and the workspace of every stage (nothing is launched).
int32_t layer_group(const csa2_cfg *c, int32_t mode, int32_t n_layers, int32_t n_q, const int8_t *q_idx,
                    const int32_t *q_seq, const int32_t *q_pos, const int8_t *k_idx, int8_t *k_blk,
                    int32_t blk_update_begin, int32_t n_seq, int32_t T, const void *q, const void *k_main,
                    const void *v_main, const void *k_swa, const void *v_swa, int32_t swa_first,
                    int32_t swa_len, int32_t *blk_ids, int32_t *blk_cnt, int32_t *topk, int32_t *topk_cnt,
                    void *out, float *lse, void *ws, size_t ws_bytes, hipStream_t st, bool launch_all,
                    bool single = false)
{
    if (int32_t e = check_cfg(c)) return e;
    if (int32_t e = check_sizes(n_q, n_seq, T)) return e;
    if (mode < CSA2_FULL || mode > CSA2_REINDEX_TOKENS) return CSA2_E_MODE;
    if (n_layers < 1) return CSA2_E_SHAPE;
    if (mode != CSA2_SWA && c->top_k < 1) return CSA2_E_MODE;
    if (n_q == 0) return CSA2_OK;
    const bool selects = mode == CSA2_FULL || mode == CSA2_REINDEX;
    const bool tokens_only = mode == CSA2_REINDEX_TOKENS;
    const bool window_only = mode == CSA2_SWA;
    if (mode == CSA2_REUSE && (!topk || !topk_cnt)) return CSA2_E_NULL;
    if (selects) {
        const FusedPlan f = plan_fused(c, n_q, T, n_layers);
        if (f.ok && ws && ws_bytes >= f.head + f.tail)
            return fused_layer_group(c, mode, n_layers, n_q, q_idx, q_seq, q_pos, k_idx, k_blk,
                                     blk_update_begin, n_seq, T, q, k_main, v_main, k_swa, v_swa,
                                     swa_first, swa_len, blk_ids, blk_cnt, topk, topk_cnt, out, lse,
                                     ws, ws_bytes, st, f, launch_all, single);
        if (single && f.ok && ws) return CSA2_E_WORKSPACE;
    }
    if (single) return CSA2_E_UNSUPPORTED;   // only the fused layer group has a single-launch form
    // every stage is checked before the first launch, then all are launched
    for (int pass = 0; pass < (launch_all ? 2 : 1); pass++) {
        const bool launch = pass == 1;
        if (mode == CSA2_FULL) {
            if (int32_t e = do_block_keys(c, k_idx, n_seq, T, blk_update_begin, T / c->block,
                                          k_blk, st, launch))
                return e;
        }
        if (selects) {
            // A prompt whose pools are whole prefixes and whose pool ids are
            // not stored: the block pass would only write the counts and the
            // completed blocks' keys, which the dense token Top-K writes
            // instead (one launch less).
            const bool in_topk = !blk_ids && plan_index(n_q, T, c->block, c->pool, c->d_idx).all &&
                                 plan_topk(n_q, T, c->block, c->pool, c->top_k, c->d_idx).dense;
            int8_t *store = mode == CSA2_FULL ? k_blk : nullptr;
            if (int32_t e = do_index(c, n_q, q_idx, q_seq, q_pos, k_idx, k_blk, n_seq, T, blk_ids,
                                     blk_cnt, ws, ws_bytes, st, launch && !in_topk, store))
                return e;
            if (int32_t e = do_topk(c, n_q, q_idx, q_seq, q_pos, k_idx, T, blk_ids, blk_cnt, topk,
                                    topk_cnt, ws, ws_bytes, st, launch, in_topk ? blk_cnt : nullptr,
                                    in_topk ? store : nullptr))
                return e;
        }
        if (tokens_only) {   // the shared pool is read, only the token Top-K is fresh
            if (int32_t e = do_topk(c, n_q, q_idx, q_seq, q_pos, k_idx, T, blk_ids, blk_cnt, topk,
                                    topk_cnt, ws, ws_bytes, st, launch))
                return e;
        }
        if (int32_t e = do_attend(c, n_layers, n_q, q, q_seq, q_pos, k_main, v_main, n_seq, T,
                                  k_swa, v_swa, swa_first, swa_len, window_only ? nullptr : topk,
                                  window_only ? nullptr : topk_cnt, out, lse, ws, ws_bytes, st,
                                  launch))
            return e;
    }
    return CSA2_OK;
}

}  // namespace

extern "C" {

int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

int32_t csa2_profile_begin(const char *kernel_filter, int32_t max_launches)
{
    if (max_launches < 0 || max_launches > (1 << 16)) return CSA2_E_SHAPE;
    if (kernel_filter && strlen(kernel_filter) >= sizeof(g_prof_filter)) return CSA2_E_SHAPE;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_armed.store(false);
    prof_release();
    strcpy(g_prof_filter, kernel_filter ? kernel_filter : "");
    g_prof.resize((size_t)max_launches);
    for (size_t i = 0; i < g_prof.size(); i++) {
        ProfRec &r = g_prof[i];
        r.name[0] = 0;
        if (hipEventCreate(&r.start) != hipSuccess) {
            g_prof.resize(i);
            prof_release();
            return CSA2_E_HIP;
        }
        if (hipEventCreate(&r.stop) != hipSuccess) {
            hipEventDestroy(r.start);
            g_prof.resize(i);
            prof_release();
            return CSA2_E_HIP;
        }
    }
    g_prof_armed.store(true);
    return CSA2_OK;
}

int32_t csa2_profile_end(int32_t *n_timed)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_armed.store(false);
    for (size_t i = 0; i < g_prof_used; i++)
        if (hipEventSynchronize(g_prof[i].stop) != hipSuccess) return CSA2_E_HIP;
    if (n_timed) *n_timed = (int32_t)g_prof_used;
    return CSA2_OK;
}

int32_t csa2_profile_record(int32_t i, char *name, int32_t name_len, float *ms)
{
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (g_prof_armed.load() || i < 0 || (size_t)i >= g_prof_used) return CSA2_E_SHAPE;
    const ProfRec &r = g_prof[(size_t)i];
    if (name && name_len > 0) {
        strncpy(name, r.name, (size_t)name_len - 1);
        name[name_len - 1] = 0;
    }
    if (ms && hipEventElapsedTime(ms, r.start, r.stop) != hipSuccess) return CSA2_E_HIP;
    return CSA2_OK;
}

const char *csa2_status_str(int32_t s)
{
    switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_E_NULL: return "a required pointer is NULL";
    case CSA2_E_SHAPE: return "a size is out of range or sizes disagree";
    case CSA2_E_DTYPE: return "unknown element type";
    case CSA2_E_UNSUPPORTED: return "unsupported size (d_idx must be 32 or 64, head_dim 64 or 128)";
    case CSA2_E_ALIGN: return "a device pointer is not aligned (16 bytes for data rows, 4 for int32)";
    case CSA2_E_WORKSPACE: return "workspace missing or too small";
    case CSA2_E_HIP: return "a HIP call or kernel launch failed";
    case CSA2_E_MODE: return "unknown layer mode or mode/argument mismatch";
    default: return "unknown status";
    }
}

int32_t csa2_workspace_bytes(const csa2_cfg *c, int32_t n_q, int32_t T, int32_t n_layers, size_t *bytes)
{
    if (!bytes) return CSA2_E_NULL;
    if (int32_t e = check_cfg(c)) return e;
    if (n_q < 0 || T < 1 || T > (1 << 24) || n_layers < 1) return CSA2_E_SHAPE;
    *bytes = head_bound(c, n_q, T) + scratch_bound(c, n_q, T, n_layers);
    return CSA2_OK;
}

int32_t csa2_workspace_init(void *ws, size_t bytes, void *stream)
{
    if (bytes == 0) return CSA2_OK;
    if (!ws) return CSA2_E_NULL;
    if (!aligned4(ws) || (bytes & 3u)) return CSA2_E_ALIGN;
    return hip_status(launch_fill_zero(ws, bytes, (hipStream_t)stream));
}

int32_t csa2_build_block_keys(const csa2_cfg *c, const int8_t *k_idx, int32_t n_seq, int32_t T,
                              int32_t blk_begin, int32_t blk_end, int8_t *k_blk, void *stream)
{
    if (int32_t e = check_cfg(c)) return e;
    if (int32_t e = check_sizes(0, n_seq, T)) return e;
    return do_block_keys(c, k_idx, n_seq, T, blk_begin, blk_end, k_blk, (hipStream_t)stream, true);
}

int32_t csa2_append_tokens(const csa2_cfg *c, int32_t n_new, const int32_t *seq, const int32_t *pos,
                           const int8_t *new_k_idx, const void *new_k, const void *new_v, int8_t *k_idx,
                           void *k_main, void *v_main, int8_t *k_blk, int32_t n_seq, int32_t T, void *stream)
{
    if (int32_t e = check_cfg(c)) return e;
    if (int32_t e = check_sizes(n_new, n_seq, T)) return e;
    if (n_new == 0) return CSA2_OK;          // nothing to write (the arrays may be empty)
    if (!seq || !pos || !new_k_idx || !new_k || !new_v || !k_idx || !k_main || !v_main) return CSA2_E_NULL;
    if (!aligned4(seq) || !aligned4(pos) || !aligned16(new_k_idx) || !aligned16(new_k) || !aligned16(new_v) ||
        !aligned16(k_idx) || !aligned16(k_main) || !aligned16(v_main) || (k_blk && !aligned16(k_blk)))
        return CSA2_E_ALIGN;
    AppendParams p{};
    p.seq = seq; p.pos = pos; p.new_k_idx = new_k_idx; p.new_k = new_k; p.new_v = new_v;
    p.k_idx = k_idx; p.k_main = k_main; p.v_main = v_main; p.k_blk = k_blk;
    p.n_new = n_new; p.T = T; p.B = c->block; p.nblk = T / c->block; p.d_idx = c->d_idx;
    p.row_bytes = c->head_dim * (c->dtype == CSA2_BF16 ? 2 : 4);
    return hip_status(launch_append(p, (hipStream_t)stream));
}


int32_t csa2_index_blocks(const csa2_cfg *c, int32_t n_q, const int8_t *q_idx, const int32_t *q_seq,
                          const int32_t *q_pos, const int8_t *k_idx, const int8_t *k_blk,
                          int32_t n_seq, int32_t T, int32_t *blk_ids, int32_t *blk_cnt, void *ws,
                          size_t ws_bytes, void *stream)
{
    if (int32_t e = check_cfg(c)) return e;
    if (int32_t e = check_sizes(n_q, n_seq, T)) return e;
    if (n_q == 0) return CSA2_OK;
    return do_index(c, n_q, q_idx, q_seq, q_pos, k_idx, k_blk, n_seq, T, blk_ids, blk_cnt, ws,
                    ws_bytes, (hipStream_t)stream, true);
}

int32_t csa2_topk_tokens(const csa2_cfg *c, int32_t n_q, const int8_t *q_idx, const int32_t *q_seq,
                         const int32_t *q_pos, const int8_t *k_idx, int32_t n_seq, int32_t T,
                         const int32_t *blk_ids, const int32_t *blk_cnt, int32_t *topk,
                         int32_t *topk_cnt, void *ws, size_t ws_bytes, void *stream)
{
    if (int32_t e = check_cfg(c)) return e;
    if (int32_t e = check_sizes(n_q, n_seq, T)) return e;
    if (n_q == 0) return CSA2_OK;
    return do_topk(c, n_q, q_idx, q_seq, q_pos, k_idx, T, blk_ids, blk_cnt, topk, topk_cnt, ws,
                   ws_bytes, (hipStream_t)stream, true);
}

int32_t csa2_attend_group(const csa2_cfg *c, int32_t n_layers, int32_t n_q, const void *q,
                          const int32_t *q_seq, const int32_t *q_pos, const void *k_main,
                          const void *v_main, int32_t n_seq, int32_t T, const void *k_swa,
                          const void *v_swa, int32_t swa_first, int32_t swa_len,
                          const int32_t *topk, const int32_t *topk_cnt, void *out, float *lse,
                          void *ws, size_t ws_bytes, void *stream)
{
    if (int32_t e = check_cfg(c)) return e;
    if (int32_t e = check_sizes(n_q, n_seq, T)) return e;
    if (n_q == 0) return CSA2_OK;
    return do_attend(c, n_layers, n_q, q, q_seq, q_pos, k_main, v_main, n_seq, T, k_swa, v_swa,
                     swa_first, swa_len, topk, topk_cnt, out, lse, ws, ws_bytes,
                     (hipStream_t)stream, true);
}

int32_t csa2_attend(const csa2_cfg *c, int32_t n_q, const void *q, const int32_t *q_seq,
                    const int32_t *q_pos, const void *k_main, const void *v_main, int32_t n_seq,
                    int32_t T, const void *k_swa, const void *v_swa, int32_t swa_first,
                    int32_t swa_len, const int32_t *topk, const int32_t *topk_cnt, void *out,
                    float *lse, void *ws, size_t ws_bytes, void *stream)
{
    return csa2_attend_group(c, 1, n_q, q, q_seq, q_pos, k_main, v_main, n_seq, T, k_swa, v_swa,
                             swa_first, swa_len, topk, topk_cnt, out, lse, ws, ws_bytes, stream);
}

int32_t csa2_layer_group(const csa2_cfg *c, int32_t mode, int32_t n_layers, int32_t n_q,
                         const int8_t *q_idx, const int32_t *q_seq, const int32_t *q_pos,
                         const int8_t *k_idx, int8_t *k_blk, int32_t blk_update_begin,
                         int32_t n_seq, int32_t T, const void *q, const void *k_main,
                         const void *v_main, const void *k_swa, const void *v_swa,
                         int32_t swa_first, int32_t swa_len, int32_t *blk_ids, int32_t *blk_cnt,
                         int32_t *topk, int32_t *topk_cnt, void *out, float *lse, void *ws,
                         size_t ws_bytes, void *stream)
{
    return layer_group(c, mode, n_layers, n_q, q_idx, q_seq, q_pos, k_idx, k_blk, blk_update_begin, n_seq, T, q,
                       k_main, v_main, k_swa, v_swa, swa_first, swa_len, blk_ids, blk_cnt, topk, topk_cnt, out,
                       lse, ws, ws_bytes, (hipStream_t)stream, true);
}

int32_t csa2_layer_group_single(const csa2_cfg *c, int32_t mode, int32_t n_layers, int32_t n_q,
                                const int8_t *q_idx, const int32_t *q_seq, const int32_t *q_pos,
                                const int8_t *k_idx, int8_t *k_blk, int32_t blk_update_begin,
                                int32_t n_seq, int32_t T, const void *q, const void *k_main,
                                const void *v_main, const void *k_swa, const void *v_swa,
                                int32_t swa_first, int32_t swa_len, int32_t *blk_ids, int32_t *blk_cnt,
                                int32_t *topk, int32_t *topk_cnt, void *out, float *lse, void *ws,
                                size_t ws_bytes, void *stream)
{
    return layer_group(c, mode, n_layers, n_q, q_idx, q_seq, q_pos, k_idx, k_blk, blk_update_begin, n_seq, T, q,
                       k_main, v_main, k_swa, v_swa, swa_first, swa_len, blk_ids, blk_cnt, topk, topk_cnt, out,
                       lse, ws, ws_bytes, (hipStream_t)stream, true, true);
}

int32_t csa2_layer_group_static(const csa2_cfg *c, int32_t mode, int32_t n_layers, int32_t n_q,
                                const int8_t *q_idx, const int32_t *q_seq, const int32_t *q_pos,
                                const int8_t *k_idx, int8_t *k_blk, int32_t blk_update_begin,
                                int32_t n_seq, int32_t T, const void *q, const void *k_main,
                                const void *v_main, const void *k_swa, const void *v_swa,
                                int32_t swa_first, int32_t swa_len, int32_t *blk_ids, int32_t *blk_cnt,
                                int32_t *topk, int32_t *topk_cnt, void *out, float *lse, void *stream)
{
    hipStream_t st = (hipStream_t)stream;
    void *ws = nullptr;
    if (int32_t e = static_scratch(&ws)) return e;
    // every argument, and every stage's room in the scratch, first
    if (int32_t e = layer_group(c, mode, n_layers, n_q, q_idx, q_seq, q_pos, k_idx, k_blk, blk_update_begin,
                                n_seq, T, q, k_main, v_main, k_swa, v_swa, swa_first, swa_len, blk_ids, blk_cnt,
                                topk, topk_cnt, out, lse, ws, kStaticScratchBytes, st, false))
        return e;
    if (n_q == 0) return CSA2_OK;
    // The array keeps the previous call's contents: the histograms at its
    // head must start at zero, so they are cleared (with a kernel, which a
    // graph capture may record) for the calls whose selections use them.
    const bool selects = mode == CSA2_FULL || mode == CSA2_REINDEX || mode == CSA2_REINDEX_TOKENS;
    if (selects) {
        const FusedPlan f = plan_fused(c, n_q, T, n_layers);
        const bool uses_head = (f.ok && f.head + f.tail <= kStaticScratchBytes) ||
                               plan_index(n_q, T, c->block, c->pool, c->d_idx).split ||
                               plan_topk(n_q, T, c->block, c->pool, c->top_k, c->d_idx).split;
        if (uses_head)
            if (int32_t e = hip_status(launch_fill_zero(ws, std::min(hist_bytes(n_q), kStaticScratchBytes), st)))
                return e;
    }
    return layer_group(c, mode, n_layers, n_q, q_idx, q_seq, q_pos, k_idx, k_blk, blk_update_begin, n_seq, T, q,
                       k_main, v_main, k_swa, v_swa, swa_first, swa_len, blk_ids, blk_cnt, topk, topk_cnt, out,
                       lse, ws, kStaticScratchBytes, st, true);
}

}  // extern "C"
