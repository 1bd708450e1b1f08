// select.hip -- block keys, token append, hierarchical block pass and token
// Top-K (gfx950).
//
// The hierarchical indexer of the DeepSeek V4.1 Flash page (k-a.in,
// "Hierarchical indexer": at most 16,384 candidates are scored whatever the
// context length) as two exact selections:
//   block pass : score every eligible block with <q_idx, kb_j>, keep the best P
//   token Top-K: score the visible tokens of the pooled blocks, keep the best K
// ("Sparse attention": Top-512 main-KV entries per query).  Scores are int8
// dot products summed exactly with v_dot4_i32_i8, so selections are exact.
//
// Decode has one query per sequence, so a query's scan (up to 1 MiB of block
// keys or candidate rows at 128K context) is split over G workgroups that
// write keys and a histogram to the workspace; a second launch with one
// workgroup per query then selects (in the layer group, the workgroups that
// score the tokens each redo the pool selection instead, k_pool_tokens).  (A
// last-arriving-workgroup hand-off was measured at ~6 us on MI355X -- an L2
// writeback plus a device-scope atomic round trip -- against ~2.5 us for a
// kernel boundary.)  With many queries (prefill) each workgroup owns one
// query and keeps its keys in LDS.
// Loads are 16-byte per lane with DIDX/16 lanes per row, so a wave reads
// 1 KiB of consecutive rows per instruction.
#include "device_common.h"
#include "internal.h"

namespace csa2 {

// One lane's 16 dimensions of a block key: the rounded mean of `n` rows that
// start at `rows` (row stride DIDX bytes).
// All (at most kMaxBlock) row loads are issued before the first is summed.
constexpr int kMaxBlock = 16;

template <int DIDX>
__device__ __forceinline__ int4 block_key_part(const int8_t *rows, int n)
{
    int4 v[kMaxBlock];
#pragma unroll
    for (int r = 0; r < kMaxBlock; r++)
        v[r] = (r < n) ? *reinterpret_cast<const int4 *>(rows + (size_t)r * DIDX) : make_int4(0, 0, 0, 0);
    int sum[16];
#pragma unroll
    for (int b = 0; b < 16; b++) sum[b] = 0;
#pragma unroll
    for (int r = 0; r < kMaxBlock; r++) {
        const int w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
        for (int a = 0; a < 4; a++)
#pragma unroll
            for (int b = 0; b < 4; b++) sum[a * 4 + b] += (int)(int8_t)(w[a] >> (8 * b));
    }
    int out[4];
#pragma unroll
    for (int a = 0; a < 4; a++) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; b++)
            packed |= ((uint32_t)round_mean_half_even(sum[a * 4 + b], n) & 0xFFu) << (8 * b);
        out[a] = (int)packed;
    }
    return make_int4(out[0], out[1], out[2], out[3]);
}

// Dimension `lane` (one lane per dimension, lanes >= DIDX give 0) of the key
// of a block whose first row is `rows`: the rounded mean of its n visible
// rows.  One byte load per row and one division per lane, so a single wave
// computes a whole key with little work (the per-thread block_key_part spends
// 16 divisions per lane).
template <int DIDX>
__device__ __forceinline__ int block_key_dim(const int8_t *rows, int n, int lane)
{
    if (lane >= DIDX) return 0;
    int v[kMaxBlock];
#pragma unroll
    for (int r = 0; r < kMaxBlock; r++) v[r] = (r < n) ? (int)rows[(size_t)r * DIDX + lane] : 0;
    int sum = 0;
#pragma unroll
    for (int r = 0; r < kMaxBlock; r++) sum += v[r];
    return round_mean_half_even(sum, n);
}

// Sum over the 64 lanes of a wave (every lane gets the total).
__device__ __forceinline__ int wave_sum_i32(int v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ int dot16_i8(int4 a, int4 b)
{
    int acc = dot4_i8(a.x, b.x, 0);
    acc = dot4_i8(a.y, b.y, acc);
    acc = dot4_i8(a.z, b.z, acc);
    return dot4_i8(a.w, b.w, acc);
}

// Sum over the LPR (2 or 4) consecutive lanes of a row with DPP quad
// permutes (lane ^ 1, then lane ^ 2), which stay in the vector ALU.
template <int LPR>
__device__ __forceinline__ int row_reduce(int v)
{
    static_assert(LPR == 2 || LPR == 4, "rows of 32 or 64 bytes");
    v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, true);        // quad_perm [1,0,3,2]
    if (LPR == 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, true);   // quad_perm [2,3,0,1]
    return v;
}

// ---------------------------------------------------------------- block keys
template <int DIDX>
__global__ __launch_bounds__(256) void k_block_keys(BlockKeysParams p)
{
    constexpr int LPR = DIDX / 16;
    const int s = blockIdx.y;
    const int item = blockIdx.x * 256 + threadIdx.x;
    const int j = p.blk_begin + item / LPR, part = item % LPR;
    if (j >= p.blk_end) return;
    const int8_t *rows = p.k_idx + ((size_t)s * p.T + (size_t)j * p.B) * DIDX + part * 16;
    const int4 key = block_key_part<DIDX>(rows, p.B);
    *reinterpret_cast<int4 *>(p.k_blk + ((size_t)s * p.nblk + j) * DIDX + part * 16) = key;
}

// ---------------------------------------------------------------- token append
// The rows of new tokens go to their cache positions: one workgroup of 64
// threads per token, 16-byte pieces.  A second launch, after every row of the
// call has landed, stores the key of each block a new token completes.
__global__ __launch_bounds__(64) void k_append_rows(AppendParams p)
{
    const int i = blockIdx.x, lane = threadIdx.x;
    const size_t row = (size_t)p.seq[i] * p.T + p.pos[i];
    if (lane < p.d_idx / 16)
        reinterpret_cast<int4 *>(p.k_idx + row * p.d_idx)[lane] =
            reinterpret_cast<const int4 *>(p.new_k_idx + (size_t)i * p.d_idx)[lane];
    const int pieces = p.row_bytes / 16;
    const int4 *nk = reinterpret_cast<const int4 *>((const uint8_t *)p.new_k + (size_t)i * p.row_bytes);
    const int4 *nv = reinterpret_cast<const int4 *>((const uint8_t *)p.new_v + (size_t)i * p.row_bytes);
    int4 *k = reinterpret_cast<int4 *>((uint8_t *)p.k_main + row * p.row_bytes);
    int4 *v = reinterpret_cast<int4 *>((uint8_t *)p.v_main + row * p.row_bytes);
    for (int x = lane; x < pieces; x += 64) {
        k[x] = nk[x];
        v[x] = nv[x];
    }
}

template <int DIDX>
__global__ __launch_bounds__(64) void k_append_block_keys(AppendParams p)
{
    constexpr int LPR = DIDX / 16;
    const int i = blockIdx.x * (64 / LPR) + threadIdx.x / LPR, part = threadIdx.x % LPR;
    if (i >= p.n_new) return;
    const int t = p.pos[i];
    if ((t + 1) % p.B != 0) return;          // the token leaves its block incomplete
    const int s = p.seq[i], j = t / p.B;
    const int8_t *rows = p.k_idx + ((size_t)s * p.T + (size_t)j * p.B) * DIDX + part * 16;
    *reinterpret_cast<int4 *>(p.k_blk + ((size_t)s * p.nblk + j) * DIDX + part * 16) = block_key_part<DIDX>(rows, p.B);
}

// ---------------------------------------------------------------- block pass
// Scoring: thread group (DIDX/16 lanes) per block, U rows in flight per lane.
// Every key also lands in a per-workgroup histogram of its top 11 bits; split
// launches add it into the query's global histogram, so the last workgroup
// starts the selection with pass 1 already done.
constexpr int kUnroll = 4;
constexpr int kPoolLds = 4096;      // pooled block ids staged in LDS for the emit

// (the body takes its workgroup index, so that the single-launch decode
// kernel can run it for any of its virtual workgroups)
template <int NT, int DIDX, bool SPLIT>
__device__ __forceinline__ void index_blocks_body(const IndexParams &p, int bid)
{
    constexpr int LPR = DIDX / 16, RPP = NT / LPR, IPT = kLdsKeys / NT;
    __shared__ uint32_t s_keys[SPLIT ? 4 : kLdsKeysPadded];
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHist2Words];
    __shared__ uint32_t s_sm[NT / 64 + 4];
    const int q = bid / p.G;   // a query's workgroups are consecutive: spread over the XCDs
    const int g = bid % p.G;
    const int tid = threadIdx.x, part = tid % LPR;
    const int s = p.q_seq[q], t = main_pos(p.q_pos[q], p.ratio);   // last visible entry (-1: none)
    const int jt = t / p.B, n_elig = eligible_blocks(t, p.B, p.tail);
    int32_t *ids = p.blk_ids + (size_t)q * p.P;
    // rows averaged into the own block's key: those at positions <= t, or
    // (whole-block reading) every row of the block that exists
    const int own_n = (p.tail == kTailWhole) ? min(p.B, p.T - jt * p.B) : t - jt * p.B + 1;

    // The query's own block (jt; its last eligible one unless a partial own
    // block is excluded, which leaves jt >= n_elig) is scored by wave 0 of the
    // workgroup whose range holds it, one lane per dimension.  A Full layer
    // also stores the key of a block its query has just completed (t is the
    // block's last position).
    const bool store_own = p.k_blk_store != nullptr && t >= 0 && (t + 1) % p.B == 0 && jt < p.nblk;
    int8_t *own_store = store_own ? p.k_blk_store + ((size_t)s * p.nblk + jt) * DIDX : nullptr;
    const int8_t *own_rows = p.k_idx + ((size_t)s * p.T + (size_t)jt * p.B) * DIDX;

    if (p.tok_hist_clear != nullptr && g == 0)
        for (int b = tid; b < kRadixBins; b += NT) p.tok_hist_clear[(size_t)q * kRadixBins + b] = 0u;

    if (n_elig <= p.P) {   // the pool is every eligible block
        for (int j = g * NT + tid; j < p.P; j += p.G * NT) ids[j] = (j < n_elig) ? j : -1;
        if (g == 0 && tid == 0) p.blk_cnt[q] = n_elig;
        if (store_own && g == 0 && tid < DIDX) own_store[tid] = (int8_t)block_key_dim<DIDX>(own_rows, p.B, tid);
        return;
    }
    for (int b = tid; b < kHist2Words; b += NT) s_hist[b] = 0;
    lds_barrier();

    const int4 qv = *reinterpret_cast<const int4 *>(p.q_idx + (size_t)q * DIDX + part * 16);
    const int lo = SPLIT ? min(n_elig, g * p.chunk) : 0;
    const int hi = SPLIT ? min(n_elig, lo + p.chunk) : n_elig;
    uint32_t *gkeys = p.ws_keys + (size_t)q * p.ws_stride;
    uint32_t *ghist = p.ws_hist + (size_t)q * kRadixBins;
    const int8_t *blk_rows = p.k_blk + (size_t)s * p.nblk * DIDX + part * 16;

    // the own block's rows are read after the first batch's block-key loads
    // have been issued
    bool own_pending = jt >= lo && jt < hi && tid < 64;
    for (int base = lo; base < hi; base += RPP * kUnroll) {
        int4 kv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int j = base + u * RPP + tid / LPR;
            kv[u] = make_int4(0, 0, 0, 0);
            if (j < hi && j < jt) kv[u] = *reinterpret_cast<const int4 *>(blk_rows + (size_t)j * DIDX);
        }
        if (own_pending) {
            own_pending = false;
            const int kd = block_key_dim<DIDX>(own_rows, own_n, tid);
            if (store_own && tid < DIDX) own_store[tid] = (int8_t)kd;
            const int qd = (tid < DIDX) ? (int)p.q_idx[(size_t)q * DIDX + tid] : 0;
            const uint32_t key = (uint32_t)(wave_sum_i32(kd * qd) + (int)kKeyBias);
            if (tid == 0) {
                if (SPLIT) gkeys[jt] = key;
                else s_keys[lds_pad(jt)] = key;
                atomicAdd(&s_hist[hist_pad(key >> kRadixBits)], 1u);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int j = base + u * RPP + tid / LPR;
            int acc = (j < hi) ? dot16_i8(kv[u], qv) : 0;
            acc = row_reduce<LPR>(acc);
            if (j < hi && j < jt && part == 0) {
                const uint32_t key = (uint32_t)(acc + (int)kKeyBias);
                if (SPLIT) gkeys[j] = key;
                else s_keys[lds_pad(j)] = key;
                atomicAdd(&s_hist[hist_pad(key >> kRadixBits)], 1u);
            }
        }
    }
    lds_barrier();
    if (SPLIT) {   // the selection runs in k_index_select, after this launch
        flush_hist<NT>(s_hist, ghist);
        return;
    }
    const uint32_t cap = (uint32_t)p.P;
    auto emit = [&](uint32_t slot, int i) { if (slot < cap) ids[slot] = i; };
    uint32_t k[IPT];
    load_keys_lds<IPT>(s_keys, n_elig, k);
    const Threshold th = threshold_regs<NT, IPT>(k, n_elig, cap, s_hist, s_sm);
    const uint32_t chosen = compact_regs<NT, IPT>(k, th, emit, s_sm);
    for (int o = (int)chosen + tid; o < p.P; o += NT) ids[o] = -1;
    if (tid == 0) p.blk_cnt[q] = (int32_t)min(chosen, cap);
}

template <int NT, int DIDX, bool SPLIT>
__global__ __launch_bounds__(NT) void k_index_blocks(IndexParams p)
{
    index_blocks_body<NT, DIDX, SPLIT>(p, (int)blockIdx.x);
}

// Pools when every eligible block of every query fits (n_elig <= P for the
// longest context): the pool of a query is its blocks 0 .. t/B, so no score
// is needed.  A grid-stride kernel writes the ids (then -1 padding), 16 bytes
// per store when the rows allow it, unless the caller stores no ids (the
// count then describes the pool), and the counts; a Full layer also stores
// the key of the block its query completes.
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kPoolAllThreads = 256;
constexpr int kPoolAllBlocks = 2048;

template <int DIDX>
__global__ __launch_bounds__(kPoolAllThreads) void k_pool_all(IndexParams p)
{
    const size_t stride = (size_t)gridDim.x * kPoolAllThreads;
    const size_t id = (size_t)blockIdx.x * kPoolAllThreads + threadIdx.x;
    const bool vec = (p.P % 4 == 0) && ((reinterpret_cast<uintptr_t>(p.blk_ids) & 15) == 0);
    if (p.blk_ids == nullptr) {
        // the pools are not stored: blk_cnt alone describes them
    } else if (vec) {
        const int P4 = p.P / 4;
        const size_t total = (size_t)p.n_q * P4;
        for (size_t k = id; k < total; k += stride) {
            const int q = (int)(k / P4), j = 4 * (int)(k % P4);
            const int n = eligible_blocks(main_pos(p.q_pos[q], p.ratio), p.B, p.tail);
            const int4 v = make_int4(j < n ? j : -1, j + 1 < n ? j + 1 : -1, j + 2 < n ? j + 2 : -1,
                                     j + 3 < n ? j + 3 : -1);
            // nontemporal: the ids are not read again in this step, and
            // streaming them past the caches keeps the keys and K/V rows the
            // following launches read resident
            const i32x4 vn = {v.x, v.y, v.z, v.w};
            __builtin_nontemporal_store(vn, reinterpret_cast<i32x4 *>(p.blk_ids + (size_t)q * p.P + j));
        }
    } else {
        const size_t total = (size_t)p.n_q * p.P;
        for (size_t k = id; k < total; k += stride) {
            const int q = (int)(k / p.P), j = (int)(k % p.P);
            p.blk_ids[k] = (j < eligible_blocks(main_pos(p.q_pos[q], p.ratio), p.B, p.tail)) ? j : -1;
        }
    }
    for (size_t k = id; k < (size_t)p.n_q * DIDX; k += stride) {
        const int q = (int)(k / DIDX), d = (int)(k % DIDX);
        const int s = p.q_seq[q], t = main_pos(p.q_pos[q], p.ratio);
        const int jt = t / p.B;
        if (d == 0) p.blk_cnt[q] = eligible_blocks(t, p.B, p.tail);
        if (p.k_blk_store != nullptr && t >= 0 && (t + 1) % p.B == 0 && jt < p.nblk) {
            const int8_t *own_rows = p.k_idx + ((size_t)s * p.T + (size_t)jt * p.B) * DIDX;
            p.k_blk_store[((size_t)s * p.nblk + jt) * DIDX + d] = (int8_t)block_key_dim<DIDX>(own_rows, p.B, d);
        }
    }
}

// Pool selection of a split launch: one workgroup per query, after every
// scoring workgroup of k_index_blocks<.., true> has finished (kernel order).
// The histogram (pass 1) and the keys are loaded together.
template <int NT>
__global__ __launch_bounds__(NT) void k_index_select(IndexParams p)
{
    constexpr int IPT = kLdsKeys / NT;
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHist2Words];
    __shared__ uint32_t s_sm[NT / 64 + 4];
    const int q = blockIdx.x, tid = threadIdx.x;
    int32_t *ids = p.blk_ids + (size_t)q * p.P;
    uint32_t *gkeys = p.ws_keys + (size_t)q * p.ws_stride;
    uint32_t *ghist = p.ws_hist + (size_t)q * kRadixBins;
    const uint32_t cap = (uint32_t)p.P;
    auto emit = [&](uint32_t slot, int i) { if (slot < cap) ids[slot] = i; };
    // every global load of the selection is issued before the first is used
    HistRegs<NT> hr;
    load_hist<NT>(ghist, hr);
    uint32_t k[IPT];
    const bool fits = p.ws_stride <= NT * IPT;
    if (fits) load_keys_global<IPT>(gkeys, (int)p.ws_stride, k);
    const int t = main_pos(p.q_pos[q], p.ratio);
    const int n_elig = eligible_blocks(t, p.B, p.tail);
    if (n_elig <= p.P) return;   // handled by the scoring launch (nothing was stored)
    store_hist<NT>(hr, ghist, s_hist);
    uint32_t chosen;
    if (fits) {
        mask_keys<IPT>(n_elig, k);
        const Threshold th = threshold_regs<NT, IPT>(k, n_elig, cap, s_hist, s_sm);
        chosen = compact_regs<NT, IPT>(k, th, emit, s_sm);
    } else {   // more blocks than one workgroup holds in registers
        const GlobalKeys keys{gkeys};
        const Threshold th = radix_threshold<NT>(keys, n_elig, cap, s_hist, s_sm, true);
        chosen = ordered_compact<NT>(keys, n_elig, th, emit, s_sm);
    }
    for (int o = (int)chosen + tid; o < p.P; o += NT) ids[o] = -1;
    if (tid == 0) p.blk_cnt[q] = (int32_t)min(chosen, cap);
}

// ---------------------------------------------------------------- token Top-K
// Threshold and ordered emit of a query's Top-K from its keys in registers and
// its pass-1 histogram in LDS; writes topk/topk_cnt.
template <int NT, int IPT>
__device__ void topk_finish(const TopkParams &p, int q, const uint32_t (&k)[IPT], int n_cand,
                            uint32_t *s_hist, int32_t *s_pool, uint32_t *s_sm)
{
    const int tid = threadIdx.x, B = p.B;
    const int n_pool = p.blk_cnt[q];
    // no stored ids: every pool is the whole prefix, slot r holds block r
    const bool implicit = p.blk_ids == nullptr;
    const int32_t *pool = implicit ? nullptr : p.blk_ids + (size_t)q * p.P;
    const bool pool_in_lds = n_pool <= kPoolLds;
    if (pool_in_lds)
        for (int r = tid; r < n_pool; r += NT) s_pool[r] = implicit ? r : pool[r];
    const Threshold th = threshold_regs<NT, IPT>(k, n_cand, (uint32_t)p.K, s_hist, s_sm);
    int32_t *out = p.topk + (size_t)q * p.K;
    const uint32_t cap = (uint32_t)p.K;
    auto emit = [&](uint32_t slot, int i) {
        const int r = i / B;
        const int blk = pool_in_lds ? s_pool[r] : (implicit ? r : pool[r]);
        if (slot < cap) out[slot] = blk * B + (i - r * B);
    };
    const uint32_t chosen = compact_regs<NT, IPT>(k, th, emit, s_sm);
    for (int o = (int)chosen + tid; o < p.K; o += NT) out[o] = -1;
    if (tid == 0) p.topk_cnt[q] = (int32_t)min(chosen, cap);
}

template <int NT, int DIDX, bool SPLIT>
__global__ __launch_bounds__(NT) void k_topk_tokens(TopkParams p)
{
    constexpr int LPR = DIDX / 16, RPP = NT / LPR, IPT = kLdsKeys / NT;
    __shared__ uint32_t s_keys[SPLIT ? 4 : kLdsKeysPadded];
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHist2Words];
    __shared__ int32_t s_pool[SPLIT ? 4 : kPoolLds];
    __shared__ uint32_t s_sm[NT / 64 + 4];
    const int q = blockIdx.x % p.n_q;   // query-fastest: k_topk_select reads a query's keys on its XCD
    const int g = blockIdx.x / p.n_q;
    const int tid = threadIdx.x, part = tid % LPR;
    const int s = p.q_seq[q], t = main_pos(p.q_pos[q], p.ratio);   // last visible entry
    const int B = p.B;
    const int n_pool = p.blk_cnt[q];
    const int n_cand = n_pool * B;                    // <= P*B <= kLdsKeys
    const bool implicit = p.blk_ids == nullptr;       // every pool is the whole prefix
    const int32_t *pool = implicit ? nullptr : p.blk_ids + (size_t)q * p.P;
    // the histogram is cleared now; the barrier that orders the clearing
    // before the first count comes after the first batch's loads are issued
    for (int b = tid; b < kHist2Words; b += NT) s_hist[b] = 0;

    const int4 qv = *reinterpret_cast<const int4 *>(p.q_idx + (size_t)q * DIDX + part * 16);
    uint32_t *gkeys = p.ws_keys + (size_t)q * p.ws_stride;
    uint32_t *ghist = p.ws_hist + (size_t)q * kRadixBins;

    // A split launch walks its whole chunk of pool slots (every slot below P
    // exists, slots past the count are ignored), so the pool entries are
    // loaded together with the count instead of after it.  Loads are
    // unconditional, from clamped slots and rows (row 0 of the sequence for
    // a slot that is not a visible candidate), and masked afterwards: a load
    // under a divergent branch would be waited for before the next is issued.
    const int lo_w = SPLIT ? g * p.chunk : 0;
    const int hi_w = SPLIT ? min(p.P * B, lo_w + p.chunk) : n_cand;
    for (int base = lo_w; base < hi_w; base += RPP * kUnroll) {
        int cl[kUnroll], blk[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            cl[u] = min(base + u * RPP + tid / LPR, hi_w - 1);
            blk[u] = implicit ? cl[u] / B : pool[cl[u] / B];
        }
        // the query's sequence and count are first used here, so the wait for
        // them stays behind the pool loads (the empty asm keeps the compiler
        // from hoisting their uses out of the loop)
        __builtin_amdgcn_sched_barrier(0);
        int np = n_pool, sq = s;
        asm volatile("" : "+s"(np), "+s"(sq));
        const int hi = SPLIT ? min(np * B, lo_w + p.chunk) : n_cand;
        const int8_t *seq_rows = p.k_idx + (size_t)sq * p.T * DIDX + part * 16;
        int pos[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) pos[u] = blk[u] * B + (cl[u] % B);
        bool vis[kUnroll];
        int4 kv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int c = base + u * RPP + tid / LPR;
            vis[u] = c < hi && pos[u] <= t;
            kv[u] = *reinterpret_cast<const int4 *>(seq_rows + (size_t)(vis[u] ? pos[u] : 0) * DIDX);
        }
        if (base == lo_w) lds_barrier();
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int c = base + u * RPP + tid / LPR;
            int acc = dot16_i8(kv[u], qv);
            acc = row_reduce<LPR>(acc);
            if (c < hi && part == 0) {
                const uint32_t key = vis[u] ? (uint32_t)(acc + (int)kKeyBias) : 0u;
                if (SPLIT) gkeys[c] = key;
                else s_keys[lds_pad(c)] = key;
                atomicAdd(&s_hist[hist_pad(key >> kRadixBits)], 1u);
            }
        }
    }
    lds_barrier();
    if (SPLIT) {   // the selection runs in k_topk_select, after this launch
        flush_hist<NT>(s_hist, ghist);
        return;
    }
    uint32_t k[IPT];
    load_keys_lds<IPT>(s_keys, n_cand, k);
    topk_finish<NT, IPT>(p, q, k, n_cand, s_hist, s_pool, s_sm);
}

// Layer-group decode: the pool selection and the token scoring of a query in
// one launch.  Each workgroup takes n_slots consecutive pool slots
// (pool_tokens_slots: kPoolTokCand / B, or more when that many workgroups
// would not all fit on the chip at once); every workgroup of a
// query first redoes the exact pool selection of k_index_select from the
// block keys and histogram that the split k_index_blocks launch wrote, keeps
// the pool slots its candidates come from in LDS
// and writes them to blk_ids (workgroup 0 also writes blk_cnt), and then
// scores its candidates like a split k_topk_tokens launch (token keys and the
// token histogram go to the workspace).  The selection is repeated
// P*B / kPoolTokCand times per query, but the launch boundary and the round
// trip of the pool through global memory are gone.  The block histogram is
// left as read; the caller's next launch zeroes it.  A query's workgroups
// are numbered consecutively, so round-robin dispatch spreads them over the
// XCDs (measured ~0.15 us faster per decode step than keeping a query's
// workgroups on one XCD; the attention launch, whose workgroups share the
// token keys, is the other way round).
constexpr int kPoolTokCand = 512;
constexpr int kPoolTokMaxWorkgroups = 256;   // one 1,024-thread workgroup per CU

// (G workgroups per query; the body takes its workgroup index)
template <int DIDX, int IPT>
__device__ __forceinline__ void pool_tokens_body(const IndexParams &ip, const TopkParams &tp, int n_slots, int G,
                                                 int bid)
{
    constexpr int NT = kSelectWideThreads;
    constexpr int LPR = DIDX / 16, RPP = NT / LPR;
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHist2Words];
    __shared__ int32_t s_pool[kFusedPoolLds];
    __shared__ uint32_t s_sm[NT / 64 + 4];
    const int q = bid / G, g = bid % G;
    const int tid = threadIdx.x, part = tid % LPR;
    const int B = ip.B, P = ip.P;

    // every load of the pool selection (and the indexer query of the
    // scoring) is issued before the first is used
    HistRegs<NT> hr;
    load_hist<NT>(ip.ws_hist + (size_t)q * kRadixBins, hr);
    uint32_t k[IPT];
    load_keys_global<IPT>(ip.ws_keys + (size_t)q * ip.ws_stride, (int)ip.ws_stride, k);
    const int4 qv = *reinterpret_cast<const int4 *>(tp.q_idx + (size_t)q * DIDX + part * 16);
    const int s = ip.q_seq[q], t = main_pos(ip.q_pos[q], ip.ratio);   // last visible entry
    const int n_elig = eligible_blocks(t, B, ip.tail);
    hist_to_lds<NT>(hr, s_hist);
    // this workgroup's pool slots [s0, s0 + n_slots): s_pool[x] holds slot s0 + x
    const int s0 = g * n_slots;
    int n_pool;
    if (n_elig <= P) {   // the pool is every eligible block (k_index_blocks wrote it)
        for (int x = tid; x < n_slots; x += NT) s_pool[x] = s0 + x;
        n_pool = n_elig;
    } else {
        mask_keys<IPT>(n_elig, k);
        const Threshold th = threshold_regs<NT, IPT>(k, n_elig, (uint32_t)P, s_hist, s_sm);
        int32_t *ids = ip.blk_ids + (size_t)q * P;
        auto emit = [&](uint32_t slot, int i) {
            const int x = (int)slot - s0;
            if (x >= 0 && x < n_slots && (int)slot < P) {
                s_pool[x] = i;
                ids[slot] = i;
            }
        };
        const uint32_t chosen = compact_regs<NT, IPT>(k, th, emit, s_sm);
        n_pool = (int)min(chosen, (uint32_t)P);
        for (int o = max(n_pool, s0) + tid; o < min(P, s0 + n_slots); o += NT) ids[o] = -1;
        if (g == 0 && tid == 0) ip.blk_cnt[q] = n_pool;
    }
    // the pool is complete once this barrier is passed; the histogram memory
    // is free again and counts this workgroup's token keys
    lds_barrier();
    for (int b = tid; b < kHistWords; b += NT) s_hist[b] = 0;

    const int n_cand = n_pool * B;
    const int lo = s0 * B, hi = min(n_cand, (s0 + n_slots) * B);
    uint32_t *gkeys = tp.ws_keys + (size_t)q * tp.ws_stride;
    const int8_t *seq_rows = tp.k_idx + (size_t)s * tp.T * DIDX + part * 16;
    for (int base = lo; base < hi; base += RPP * kUnroll) {
        int pos[kUnroll];
        bool vis[kUnroll];
        int4 kv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int c = base + u * RPP + tid / LPR;
            const int cl = min(c, hi - 1);
            pos[u] = s_pool[cl / B - s0] * B + cl % B;
            vis[u] = c < hi && pos[u] <= t;
            kv[u] = *reinterpret_cast<const int4 *>(seq_rows + (size_t)(vis[u] ? pos[u] : 0) * DIDX);
        }
        if (base == lo) lds_barrier();   // the histogram is cleared
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int c = base + u * RPP + tid / LPR;
            int acc = dot16_i8(kv[u], qv);
            acc = row_reduce<LPR>(acc);
            if (c < hi && part == 0) {
                const uint32_t key = vis[u] ? (uint32_t)(acc + (int)kKeyBias) : 0u;
                gkeys[c] = key;
                atomicAdd(&s_hist[hist_pad(key >> kRadixBits)], 1u);
            }
        }
    }
    lds_barrier();
    flush_hist<NT>(s_hist, tp.ws_hist + (size_t)q * kRadixBins);
}

template <int DIDX, int IPT>
__global__ __launch_bounds__(kSelectWideThreads) void k_pool_tokens(IndexParams ip, TopkParams tp, int n_slots)
{
    pool_tokens_body<DIDX, IPT>(ip, tp, n_slots, (int)gridDim.x / ip.n_q, (int)blockIdx.x);
}

template <int NT>
__global__ __launch_bounds__(NT) void k_topk_select(TopkParams p)
{
    constexpr int IPT = kLdsKeys / NT;
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[kHist2Words];
    __shared__ int32_t s_pool[kPoolLds];
    __shared__ uint32_t s_sm[NT / 64 + 4];
    const int q = blockIdx.x;
    uint32_t *ghist = p.ws_hist + (size_t)q * kRadixBins;
    HistRegs<NT> hr;
    load_hist<NT>(ghist, hr);
    uint32_t k[IPT];
    load_keys_global<IPT>(p.ws_keys + (size_t)q * p.ws_stride, (int)p.ws_stride, k);
    const int n_cand = p.blk_cnt[q] * p.B;
    store_hist<NT>(hr, ghist, s_hist);
    mask_keys<IPT>(n_cand, k);
    topk_finish<NT, IPT>(p, q, k, n_cand, s_hist, s_pool, s_sm);
}

// ---------------------------------------------------------------- dense token Top-K
// Prefill-sized calls where every query's pool is its whole prefix (all its
// eligible blocks fit the pool) and the context is at most kDenseMaxT tokens:
// the candidates of a query at position t are then the positions 0..t.  A
// workgroup takes kDenseQ consecutive queries; for the queries of one
// sequence, v_mfma_i32_16x16x64_i8 scores 16 positions x 16 queries per
// instruction (A = k_idx rows, B = q_idx rows; exact int32 sums), and every
// query's exact Top-K is found by a radix select that rescans the prefix
// instead of storing its keys:
//   pass 1: histogram of key >> 11 per query -> threshold bin b1, with gt1
//           keys above it and eq1 keys in it;
//   pass 2: bitmaps of the keys above bin b1 and of the keys in bin b1 (plain
//           compares, no branch per key); the eq1 keys of bin b1 are then
//           scored again from their rows, and a ballot search over their low
//           key bits finds the K-th key: the ones above it join the first
//           bitmap, those equal to it a tie bitmap.
// When some query has more than kDenseList keys in its bin b1 (many equal
// scores), pass 2 instead takes a histogram of the low bits inside bin b1
// (-> exact threshold key tau and the number of ties to take) and a third
// pass builds bitmaps of keys above tau and equal to tau.  An ordered emit
// over the bitmaps writes the positions ascending, ties lowest position
// first, staged in the query's bitmap row and copied out with coalesced
// stores.  The first pass counts one key bin per 32-bit LDS word: scores lie
// in [-2^20, 2^20], so only the 1,025 bins 512 .. 1536 of key >> 11 can hold
// a key, and word w of a row counts bin 512 + w (a count costs a shift, an
// add and the atomic).  The low-bit histogram of the fallback packs two
// 16-bit counts (at most kDenseMaxT) per word.  The bitmaps reuse the
// histogram memory; per-query rows are padded
// so that the 16 queries of a wave instruction fall in different LDS banks,
// and a wave owns whole bitmap words, which it writes with plain stores.
constexpr int kDenseQ = 16;              // queries per workgroup (one MFMA column block)
constexpr int kDenseWaves = 8;
constexpr int kDenseUnroll = 4;          // position tiles per wave per load batch
constexpr int kDenseBatchPos = 16 * kDenseUnroll;
constexpr int kDenseBatchWords = kDenseBatchPos / 32;
static_assert(kDenseBatchPos % 32 == 0, "a batch covers whole bitmap words");
constexpr int kDenseHistWords = kRadixBins / 2 + 8;   // histogram words per query (+ bank pad)
constexpr int kDenseBin0 = 512;          // key >> 11 of the first occupied first-pass bin
static_assert(kDenseHistWords >= 1025, "every occupied first-pass bin has a word");
constexpr int kDenseMapWords = kDenseMaxT / 32 + 4;   // bitmap words per query (+ bank pad)
constexpr int kDenseList = 128;          // bin-b1 keys per query the two-pass select resolves
constexpr int kDenseStage = 512;         // output slots staged in a bitmap row at once
static_assert(kDenseStage <= kDenseMapWords, "a bitmap row holds the output stage");

typedef int v4i32 __attribute__((ext_vector_type(4)));

// Threshold search over one query's packed 2048-bin histogram by one wave:
// the bin b where the count of keys in bins above b is < n <= count in bins
// >= b; `above` gets the count above b and `in_bin` the count in b.
__device__ __forceinline__ void find_bin_packed(const uint32_t *h, uint32_t n, int &bin, uint32_t &above,
                                                uint32_t &in_bin)
{
    const int lane = threadIdx.x & 63;
    uint32_t c[16];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(h + 16 * lane + 4 * k);
        c[4 * k] = v.x; c[4 * k + 1] = v.y; c[4 * k + 2] = v.z; c[4 * k + 3] = v.w;
    }
    uint32_t S = 0;
#pragma unroll
    for (int k = 0; k < 16; k++) S += (c[k] & 0xffffu) + (c[k] >> 16);
    const uint32_t incl = wave_incl_scan(S);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t suf = total - incl;   // keys in the bins above this lane's 32
    const bool here = suf < n && suf + S >= n;
    int b = 0;
    uint32_t run = suf, cb = 0;
    if (here) {
        for (int k = 15; k >= 0; k--) {
            const uint32_t hi = c[k] >> 16, lo = c[k] & 0xffffu;
            if (run + hi >= n) { b = 2 * k + 1; cb = hi; break; }
            run += hi;
            if (run + lo >= n) { b = 2 * k; cb = lo; break; }
            run += lo;
        }
    }
    const uint64_t found = __builtin_amdgcn_ballot_w64(here);   // exactly one lane when n <= total
    const int src = found ? __builtin_ctzll(found) : 0;
    bin = __builtin_amdgcn_readlane(32 * lane + b, src);
    above = (uint32_t)__builtin_amdgcn_readlane((int)run, src);
    in_bin = (uint32_t)__builtin_amdgcn_readlane((int)cb, src);
}

// The same search over one query's first-pass histogram, one bin per word:
// word w counts key bin kDenseBin0 + w for w = 0 .. 1024; lane l covers words
// 16 l .. 16 l + 15, and lane 63 also word 1024 (the top bin, which only a
// score of exactly 2^20 reaches).  `bin` is returned as a key bin (key >> 11).
__device__ __forceinline__ void find_bin_words(const uint32_t *h, uint32_t n, int &bin, uint32_t &above,
                                               uint32_t &in_bin)
{
    const int lane = threadIdx.x & 63;
    uint32_t c[16];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint4 v = *reinterpret_cast<const uint4 *>(h + 16 * lane + 4 * k);
        c[4 * k] = v.x; c[4 * k + 1] = v.y; c[4 * k + 2] = v.z; c[4 * k + 3] = v.w;
    }
    const uint32_t top = (lane == 63) ? h[1024] : 0u;
    uint32_t S = top;
#pragma unroll
    for (int k = 0; k < 16; k++) S += c[k];
    const uint32_t incl = wave_incl_scan(S);
    const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    const uint32_t suf = total - incl;   // keys in the bins above this lane's
    const bool here = suf < n && suf + S >= n;
    int b = 0;
    uint32_t run = suf, cb = 0;
    if (here) {
        if (run + top >= n) {
            b = 16;
            cb = top;
        } else {
            run += top;
            for (int k = 15; k >= 0; k--) {
                if (run + c[k] >= n) { b = k; cb = c[k]; break; }
                run += c[k];
            }
        }
    }
    const uint64_t found = __builtin_amdgcn_ballot_w64(here);   // exactly one lane when n <= total
    const int src = found ? __builtin_ctzll(found) : 0;
    bin = kDenseBin0 + __builtin_amdgcn_readlane(16 * lane + b, src);
    above = (uint32_t)__builtin_amdgcn_readlane((int)run, src);
    in_bin = (uint32_t)__builtin_amdgcn_readlane((int)cb, src);
}

__device__ __forceinline__ uint32_t or_groups(uint32_t x)   // OR over lanes l, l^16, l^32, l^48
{
    auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = r[0] | r[1];
    r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return r[0] | r[1];
}

// Positions of the set bits of one query's bitmap row, in order: lane l
// covers words 8l .. 8l+7; fn(rank, position) for every set bit, rank being
// its index among all set bits of the row.
template <class Fn>
__device__ __forceinline__ void for_set_bits(const uint32_t *row, uint32_t (&m)[8], Fn &&fn)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < 2; k++) {
        const uint4 a = *reinterpret_cast<const uint4 *>(row + 8 * lane + 4 * k);
        m[4 * k] = a.x; m[4 * k + 1] = a.y; m[4 * k + 2] = a.z; m[4 * k + 3] = a.w;
    }
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) c += __builtin_popcount(m[k]);
    uint32_t r = wave_incl_scan(c) - c;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        uint32_t x = m[k];
        while (x) {
            const int b = __builtin_ctz(x);
            x &= x - 1;
            fn(r++, 256 * lane + 32 * k + b);
        }
    }
}

template <int DIDX>
__global__ __launch_bounds__(kDenseWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_topk_dense(TopkParams p)
{
    constexpr int NT = kDenseWaves * 64;
    constexpr int HW = kDenseHistWords, MW = kDenseMapWords;
    static_assert(2 * kDenseQ * MW <= kDenseQ * HW, "bitmaps reuse the histogram memory");
    __shared__ __attribute__((aligned(16))) uint32_t s_buf[kDenseQ * HW];
    __shared__ uint32_t s_list[kDenseQ][kDenseList];   // positions of the keys of bin b1
    __shared__ int s_b1[kDenseQ], s_tau[kDenseQ], s_need[kDenseQ];
    __shared__ uint32_t s_gt1[kDenseQ], s_eq1[kDenseQ];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    // Workgroup b takes query tile b in the first half of the grid and the
    // tiles from the last one down in the second half, so that the two
    // workgroups a CU holds at once scan prefixes of complementary length.
    const int n_wg = (int)gridDim.x, half = n_wg / 2;
    const int tile_q = (int)blockIdx.x < half ? (int)blockIdx.x : n_wg - 1 - ((int)blockIdx.x - half);
    const int q0 = tile_q * kDenseQ;
    const int K = p.K;
    // this lane's query column (sequence, position, q_idx as the B operand)
    const int qi = q0 + r16;
    const bool qvalid = qi < p.n_q;
    const int sq = qvalid ? p.q_seq[qi] : -1;
    // last candidate entry of this lane's query: its last visible entry, or
    // with a partial own block excluded the end of its last complete block
    // (-1: no candidate)
    const int tv = qvalid ? main_pos(p.q_pos[qi], p.ratio) : -1;
    const int tq = p.tail == kTailExclude ? (tv + 1) / p.B * p.B - 1 : tv;
    v4i32 qb = {0, 0, 0, 0};
    if (qvalid && 16 * g < DIDX) qb = *reinterpret_cast<const v4i32 *>(p.q_idx + (size_t)qi * DIDX + 16 * g);
    uint32_t *gt_map = s_buf, *eq_map = s_buf + kDenseQ * MW;

    // the block pass's outputs when it is not launched (see TopkParams)
    if (p.pool_cnt_out != nullptr) {
        for (int x = tid; x < kDenseQ * DIDX; x += NT) {
            const int i = q0 + x / DIDX, dd = x % DIDX;
            if (i >= p.n_q) continue;
            const int t = main_pos(p.q_pos[i], p.ratio), jt = t / p.B;
            if (dd == 0) p.pool_cnt_out[i] = eligible_blocks(t, p.B, p.tail);
            if (p.k_blk_store != nullptr && t >= 0 && (t + 1) % p.B == 0 && jt < p.nblk) {
                const size_t row0 = (size_t)p.q_seq[i] * p.T + (size_t)jt * p.B;
                p.k_blk_store[((size_t)p.q_seq[i] * p.nblk + jt) * DIDX + dd] =
                    (int8_t)block_key_dim<DIDX>(p.k_idx + row0 * DIDX, p.B, dd);
            }
        }
    }

    auto zero_buf = [&] {
        for (int x = tid * 4; x < kDenseQ * HW; x += NT * 4) *reinterpret_cast<uint4 *>(s_buf + x) = make_uint4(0, 0, 0, 0);
    };

    uint32_t remaining = (uint32_t)__builtin_amdgcn_ballot_w64(qvalid && g == 0) & 0xffffu;
    // the tile's queries, one sequence at a time (every wave takes the same groups)
    while (remaining) {
        const int s = __builtin_amdgcn_readlane(sq, __builtin_ctz(remaining));
        const bool in_group = qvalid && sq == s && ((remaining >> r16) & 1);
        const uint32_t gmask = (uint32_t)__builtin_amdgcn_ballot_w64(in_group && g == 0) & 0xffffu;
        remaining &= ~gmask;
        int tmax = 0, tmin = INT32_MAX;
        for (uint32_t m = gmask; m; m &= m - 1) {
            const int t = __builtin_amdgcn_readlane(tq, __builtin_ctz(m));
            tmax = max(tmax, t);
            tmin = min(tmin, t);
        }
        const bool mine = in_group;
        const int8_t *rows = p.k_idx + (size_t)s * p.T * DIDX;

        // Runs fn(u, pos0, d, check) for every position tile of this wave and
        // done(word0) after each batch: batch gi covers positions
        // kDenseBatchPos * gi .. + kDenseBatchPos - 1 (bitmap words
        // kDenseBatchWords * gi ..), tile u of it positions pos0 =
        // kDenseBatchPos * gi + 16 u ..; d[ii] is the score of position
        // pos0 + 4g + ii for query column r16, and `check` is false when every
        // position of the tile precedes every query.  A batch's loads are
        // issued together and unconditionally, as buffer loads over the
        // sequence's rows (a position past the sequence reads zeros and is
        // never counted; the dims a d_idx of 32 lacks meet zeros in q_idx),
        // and a wave issues the loads of its next batch before it works on
        // this one, so that a batch costs its arithmetic rather than a
        // memory round trip.
        const int n_batches = tmax / kDenseBatchPos + 1;
        const auto rows_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(rows), 0, p.T * DIDX, kRsrcWord3);
        auto scan = [&](auto &&fn, auto &&done) {
            const int part = (16 * g < DIDX) ? 16 * g : 16 * (g & 1);
            auto load = [&](int gi, v4i32 (&a)[kDenseUnroll]) {
                const int off = (kDenseBatchPos * gi + r16) * DIDX + part;
#pragma unroll
                for (int u = 0; u < kDenseUnroll; u++)
                    a[u] = __builtin_bit_cast(v4i32, __builtin_amdgcn_raw_buffer_load_b128(rows_rsrc, off + 16 * u * DIDX, 0, 0));
            };
            // every tile of a batch is scored: a tile past the last query
            // takes the checked path, where no position passes (skipping it
            // instead would leave a prefetched register unread on one path,
            // and the compiler then waits for every load at the loop head)
            auto body = [&](int gi, const v4i32 (&a)[kDenseUnroll]) {
#pragma unroll
                for (int u = 0; u < kDenseUnroll; u++) {
                    const int pos0 = kDenseBatchPos * gi + 16 * u;
                    const v4i32 d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u], qb, v4i32{0, 0, 0, 0}, 0, 0, 0);
                    if (pos0 + 15 > tmin) fn(u, pos0, d, true);
                    else fn(u, pos0, d, false);
                }
                done(kDenseBatchWords * gi);
            };
            int gi = w;
            if (gi >= n_batches) return;
            v4i32 a0[kDenseUnroll], a1[kDenseUnroll];
            load(gi, a0);
            for (; gi + kDenseWaves < n_batches; gi += 2 * kDenseWaves) {
                load(gi + kDenseWaves, a1);
                body(gi, a0);
                load(gi + 2 * kDenseWaves, a0);   // past the end: read, never used
                body(gi + kDenseWaves, a1);
            }
            if (gi < n_batches) body(gi, a0);
        };
        auto nothing = [](int) {};
        // bits of this batch for query column r16 (OR over the lane groups),
        // stored by lane group 0 as the batch's bitmap words
        auto store_bits = [&](uint32_t *map, int word0, uint32_t (&bits)[kDenseBatchWords]) {
#pragma unroll
            for (int k = 0; k < kDenseBatchWords; k++) {
                const uint32_t b = or_groups(bits[k]);
                if (g == 0 && mine && word0 + k < MW) map[r16 * MW + word0 + k] = b;
                bits[k] = 0u;
            }
        };

        // every column of the wave is in the group: tiles before every query
        // need no per-lane test at all
        const bool all_mine = __builtin_amdgcn_ballot_w64(mine) == ~0ull;

        // ---- pass 1: top-bit histograms.  With key = score + 2^21, the word
        // of bin key >> 11 is (score >> 11) + 1024 - kDenseBin0.
        zero_buf();
        __syncthreads();
        uint32_t *hrow = s_buf + r16 * HW + ((int)(kKeyBias >> kRadixBits) - kDenseBin0);
        auto hist_add = [&](int sc) { atomicAdd(&hrow[sc >> kRadixBits], 1u); };
        scan([&](int, int pos0, v4i32 d, bool check) {
            if (!check && all_mine) {
#pragma unroll
                for (int ii = 0; ii < 4; ii++) hist_add(d[ii]);
                return;
            }
            if (!mine) return;
#pragma unroll
            for (int ii = 0; ii < 4; ii++)
                if (!check || pos0 + 4 * g + ii <= tq) hist_add(d[ii]);
        }, nothing);
        __syncthreads();
        for (int jq = w; jq < kDenseQ; jq += kDenseWaves) {
            if (!((gmask >> jq) & 1)) continue;
            const uint32_t n = (uint32_t)__builtin_amdgcn_readlane(tq, jq) + 1;
            int b1 = -1;                 // fewer candidates than K: every key is taken
            uint32_t gt1 = 0, eq1 = 0;
            if (n > (uint32_t)K) find_bin_words(s_buf + jq * HW, (uint32_t)K, b1, gt1, eq1);
            if (lane == 0) {
                s_b1[jq] = b1;
                s_gt1[jq] = gt1;
                s_eq1[jq] = eq1;
                s_need[jq] = 0;
            }
        }
        __syncthreads();
        const int b1q = mine ? s_b1[r16] : -1;
        const bool listed = __syncthreads_and(!mine || s_eq1[r16] <= (uint32_t)kDenseList);
        zero_buf();
        __syncthreads();
        if (listed) {
            // ---- pass 2: bitmaps of the keys above bin b1 and of the keys in
            // bin b1 (plain compares, no branch per key).  A lane's thresholds:
            // above bin b1 from thr_gt, in bin b1 from thr_lo (bins as
            // score >> 11: the bias moves every bin by 1024); every key passes
            // thr_gt when the query keeps all its candidates, and none passes
            // for a lane outside the group.
            uint32_t gw[kDenseBatchWords] = {}, bw[kDenseBatchWords] = {};
            const int b1s = b1q - (int)(kKeyBias >> kRadixBits);
            const int thr_gt = !mine ? INT32_MAX : (b1q < 0 ? INT32_MIN : (b1s + 1) * kRadixBins);
            const int thr_lo = (!mine || b1q < 0) ? INT32_MAX : b1s * kRadixBins;
            const uint32_t lane_bit = 1u << (4 * g);    // position 4g of a 16-position tile
            scan([&](int u, int pos0, v4i32 d, bool check) {
#pragma unroll
                for (int ii = 0; ii < 4; ii++) {
                    // pos0 is a multiple of 16, so the bit of position
                    // pos0 + 4g + ii in its word is 16 (u & 1) + 4g + ii
                    const uint32_t bit = lane_bit << (16 * (u & 1) + ii);
                    const bool ok = !check || pos0 + 4 * g + ii <= tq;
                    gw[u >> 1] |= (ok && d[ii] >= thr_gt) ? bit : 0u;
                    bw[u >> 1] |= (ok && d[ii] >= thr_lo && d[ii] < thr_gt) ? bit : 0u;
                }
            }, [&](int word0) {
                store_bits(gt_map, word0, gw);
                store_bits(eq_map, word0, bw);
            });
            __syncthreads();
            // bin b1: its (at most kDenseList) keys are scored again from
            // their rows; the threshold tau2 on their low key bits that keeps
            // need1 = K - gt1 of them is found bit by bit from the top
            // (counting with ballots); keys above tau2 join the first bitmap,
            // keys equal to it go to the tie bitmap (the query's bin-b1 row,
            // cleared once read), from which the emit takes the first ones in
            // position order
            for (int jq = w; jq < kDenseQ; jq += kDenseWaves) {
                if (!((gmask >> jq) & 1) || s_b1[jq] < 0) continue;
                const int n_list = (int)s_eq1[jq];
                const uint32_t need1 = (uint32_t)K - s_gt1[jq];
                uint32_t *erow = eq_map + jq * MW;
                uint32_t m[8];
                for_set_bits(erow, m, [&](uint32_t r, int pos) {
                    if (r < (uint32_t)kDenseList) s_list[jq][r] = (uint32_t)pos;
                });
                *reinterpret_cast<uint4 *>(erow + 8 * lane) = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(erow + 8 * lane + 4) = make_uint4(0, 0, 0, 0);
                wave_lds_order();
                const int8_t *qrow = p.q_idx + (size_t)(q0 + jq) * DIDX;
                int4 qv[DIDX / 16], kv[2][DIDX / 16];
                int pos_e[2];
                bool vl[2];
#pragma unroll
                for (int k = 0; k < DIDX / 16; k++) qv[k] = *reinterpret_cast<const int4 *>(qrow + 16 * k);
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int x = lane + 64 * h;
                    vl[h] = x < n_list;
                    pos_e[h] = vl[h] ? (int)s_list[jq][x] : 0;
#pragma unroll
                    for (int k = 0; k < DIDX / 16; k++)
                        kv[h][k] = *reinterpret_cast<const int4 *>(rows + (size_t)pos_e[h] * DIDX + 16 * k);
                }
                uint32_t lo[2];
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    int acc = 0;
#pragma unroll
                    for (int k = 0; k < DIDX / 16; k++) {
                        acc = dot4_i8(kv[h][k].x, qv[k].x, acc);
                        acc = dot4_i8(kv[h][k].y, qv[k].y, acc);
                        acc = dot4_i8(kv[h][k].z, qv[k].z, acc);
                        acc = dot4_i8(kv[h][k].w, qv[k].w, acc);
                    }
                    lo[h] = ((uint32_t)(acc + (int)kKeyBias)) & kRadixMask;
                }
                uint32_t tau2 = 0, above = 0;
                for (int bit = kRadixBits - 1; bit >= 0; bit--) {
                    const uint32_t want = (tau2 | (1u << bit)) >> bit;
                    const uint32_t cnt =
                        (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(vl[0] && (lo[0] >> bit) == want)) +
                        (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(vl[1] && (lo[1] >> bit) == want));
                    if (above + cnt >= need1) tau2 |= 1u << bit;
                    else above += cnt;
                }
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    if (vl[h] && lo[h] > tau2) atomicOr(&gt_map[jq * MW + (pos_e[h] >> 5)], 1u << (pos_e[h] & 31));
                    if (vl[h] && lo[h] == tau2) atomicOr(&erow[pos_e[h] >> 5], 1u << (pos_e[h] & 31));
                }
                if (lane == 0) s_need[jq] = (int)(need1 - above);
            }
        } else {
            // ---- pass 2': low-bit histograms inside the threshold bin
            scan([&](int, int pos0, v4i32 d, bool check) {
                if (b1q < 0) return;
#pragma unroll
                for (int ii = 0; ii < 4; ii++) {
                    const uint32_t key = (uint32_t)(d[ii] + (int)kKeyBias);
                    if ((!check || pos0 + 4 * g + ii <= tq) && (int)(key >> kRadixBits) == b1q) {
                        const uint32_t b = key & kRadixMask;
                        atomicAdd(&s_buf[r16 * HW + (b >> 1)], 1u << (16 * (b & 1)));
                    }
                }
            }, nothing);
            __syncthreads();
            for (int jq = w; jq < kDenseQ; jq += kDenseWaves) {
                if (!((gmask >> jq) & 1)) continue;
                const int b1 = s_b1[jq];
                int tau = 0, need = 0;   // fewer candidates than K: every key (> 0) is taken
                if (b1 >= 0) {
                    const uint32_t need1 = (uint32_t)K - s_gt1[jq];
                    int b2;
                    uint32_t gt2, eq2;
                    find_bin_packed(s_buf + jq * HW, need1, b2, gt2, eq2);
                    tau = (b1 << kRadixBits) | b2;
                    need = (int)(need1 - gt2);
                }
                if (lane == 0) {
                    s_tau[jq] = tau;
                    s_need[jq] = need;
                }
            }
            __syncthreads();
            // ---- pass 3: bitmaps of keys above tau and equal to tau
            zero_buf();
            __syncthreads();
            const uint32_t tauq = mine ? (uint32_t)s_tau[r16] : 0u;
            uint32_t gw[kDenseBatchWords] = {}, ew[kDenseBatchWords] = {};
            scan([&](int u, int pos0, v4i32 d, bool check) {
                if (!mine) return;
#pragma unroll
                for (int ii = 0; ii < 4; ii++) {
                    const int pos = pos0 + 4 * g + ii;
                    const bool ok = !check || pos <= tq;
                    const uint32_t key = (uint32_t)(d[ii] + (int)kKeyBias);
                    gw[u >> 1] |= (uint32_t)(ok && key > tauq) << (pos & 31);
                    ew[u >> 1] |= (uint32_t)(ok && key == tauq) << (pos & 31);
                }
            }, [&](int word0) {
                store_bits(gt_map, word0, gw);
                store_bits(eq_map, word0, ew);
            });
        }
        __syncthreads();
        // ---- ordered emit.  A wave takes its query's bitmap words into
        // registers (lane l: words 64 r + l), folds in the first `need` tie
        // bits in position order, and writes the positions in slot order into
        // the query's bitmap row, which then serves as the output stage:
        // kDenseStage slots at a time, copied out with coalesced stores.
        for (int jq = w; jq < kDenseQ; jq += kDenseWaves) {
            if (!((gmask >> jq) & 1)) continue;
            uint32_t *row = gt_map + jq * MW;
            const uint32_t *erow = eq_map + jq * MW;
            const int i = q0 + jq;
            const int n = __builtin_amdgcn_readlane(tq, jq) + 1;
            const int cnt = min(n, K);
            const int need = s_need[jq];   // ties to take, in position order
            int32_t *out = p.topk + (size_t)i * K;
            const int n_words = (n + 31) / 32;
            constexpr int R = (kDenseMaxT / 32 + 63) / 64;
            uint32_t x[R];
#pragma unroll
            for (int r = 0; r < R; r++) x[r] = (64 * r + lane < n_words) ? row[64 * r + lane] : 0u;
            if (need > 0) {
                uint32_t ties = 0;
#pragma unroll
                for (int r = 0; r < R; r++) {
                    if (64 * r >= n_words) break;
                    uint32_t e = (64 * r + lane < n_words) ? erow[64 * r + lane] : 0u;
                    const uint32_t ec = __builtin_popcount(e);
                    const uint32_t e_incl = wave_incl_scan(ec);
                    int take = min(max(need - (int)(ties + e_incl - ec), 0), (int)ec);
                    while (take > 0) {
                        const uint32_t lsb = e & (0u - e);
                        x[r] |= lsb;
                        e ^= lsb;
                        take--;
                    }
                    ties += (uint32_t)__builtin_amdgcn_readlane((int)e_incl, 63);
                }
            }
            wave_lds_order();   // the row is in registers: it becomes the stage
            for (int c0 = 0; c0 < K; c0 += kDenseStage) {
                const int len = min(kDenseStage, K - c0);
                uint32_t run = 0;   // kept positions in the rounds before
#pragma unroll
                for (int r = 0; r < R; r++) {
                    if (64 * r >= n_words) break;
                    const uint32_t sc = __builtin_popcount(x[r]);
                    const uint32_t incl = wave_incl_scan(sc);
                    uint32_t xx = x[r], slot = run + incl - sc;
                    run += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
                    const uint32_t pos0 = (uint32_t)(32 * (64 * r + lane));
                    if (K <= kDenseStage) {
                        // one stage holds every slot, and the kept positions
                        // fill exactly slots 0 .. cnt - 1
                        uint32_t *dst = row + slot;
                        while (xx) {
                            *dst++ = pos0 + (uint32_t)__builtin_ctz(xx);
                            xx &= xx - 1;
                        }
                    } else {
                        while (xx) {
                            const int b = __builtin_ctz(xx);
                            xx &= xx - 1;
                            if (slot >= (uint32_t)c0 && slot < (uint32_t)(c0 + len)) row[slot - c0] = pos0 + (uint32_t)b;
                            slot++;
                        }
                    }
                }
                for (int o = max(cnt, c0) - c0 + lane; o < len; o += 64) row[o] = 0xffffffffu;   // -1: no entry
                wave_lds_order();
                if ((K & 3) == 0 && (len & 3) == 0 && ((uintptr_t)p.topk & 15) == 0) {
                    // 16 bytes a lane, nontemporal: the ids are read once, by
                    // the attention, and need no room in L2 meanwhile
                    for (int o = 4 * lane; o < len; o += 256)
                        __builtin_nontemporal_store(*reinterpret_cast<const v4i32 *>(row + o),
                                                    reinterpret_cast<v4i32 *>(out + c0 + o));
                } else {
                    for (int o = lane; o < len; o += 64) out[c0 + o] = (int32_t)row[o];
                }
                wave_lds_order();   // the stage is read before the next slots are written
            }
            if (lane == 0) p.topk_cnt[i] = cnt;
        }
        __syncthreads();
    }
}

__global__ void k_fill_zero(uint32_t *p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------- planning
static int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

static SelectPlan plan_scan(int n_q, long long n_items, int d_idx, bool must_split)
{
    const int rows_per_iter = kSelectThreads / (d_idx / 16);
    SelectPlan pl{1, (int)n_items, false, 0};
    int G = 1;
    if (n_q < kTargetWorkgroups) G = ceil_div(kTargetWorkgroups, n_q);
    G = std::min(G, ceil_div(n_items, rows_per_iter));
    G = std::max(G, 1);
    if (G > 1 || must_split) {
        int chunk = ceil_div(ceil_div(n_items, G), rows_per_iter) * rows_per_iter;
        pl.G = ceil_div(n_items, chunk);
        pl.chunk = chunk;
        pl.split = true;
        pl.key_bytes = (size_t)n_q * (size_t)((n_items + 3) / 4 * 4) * sizeof(uint32_t);
    }
    return pl;
}

size_t select_head_bytes(int n_q, bool split)
{
    return split ? (size_t)n_q * kRadixBins * sizeof(uint32_t) : 0;
}

SelectPlan plan_index(int n_q, int T, int B, int P, int d_idx)
{
    const long long n_elig_max = (long long)(T - 1) / B + 1;
    if (n_elig_max <= P) {
        SelectPlan pl{1, (int)n_elig_max, false, 0};
        pl.all = true;
        return pl;
    }
    return plan_scan(n_q, n_elig_max, d_idx, n_elig_max > kLdsKeys);
}

SelectPlan plan_topk(int n_q, int T, int B, int P, int K, int d_idx)
{
    (void)K;
    const long long n_elig_max = (long long)(T - 1) / B + 1;
    if (n_elig_max <= P && T <= kDenseMaxT && n_q >= kDenseMinQueries) {
        SelectPlan pl{1, 0, false, 0};
        pl.dense = true;
        return pl;
    }
    return plan_scan(n_q, (long long)P * B, d_idx, false);
}

// ---------------------------------------------------------------- launches
hipError_t launch_block_keys(const BlockKeysParams &p, int n_seq, int d_idx, hipStream_t st)
{
    const int n = (p.blk_end - p.blk_begin) * (d_idx / 16);
    if (n <= 0 || n_seq <= 0) return hipSuccess;
    dim3 grid(ceil_div(n, 256), n_seq);
    if (d_idx == 64) launch("k_block_keys", k_block_keys<64>, grid, dim3(256), st, p);
    else launch("k_block_keys", k_block_keys<32>, grid, dim3(256), st, p);
    return hipGetLastError();
}

hipError_t launch_append(const AppendParams &p, hipStream_t st)
{
    if (p.n_new <= 0) return hipSuccess;
    launch("k_append_rows", k_append_rows, dim3((unsigned)p.n_new), dim3(64), st, p);
    if (p.k_blk) {
        const unsigned per = 64 / (p.d_idx / 16);   // tokens per workgroup
        const dim3 grid((unsigned)((p.n_new + per - 1) / per));
        if (p.d_idx == 64) launch("k_append_block_keys", k_append_block_keys<64>, grid, dim3(64), st, p);
        else launch("k_append_block_keys", k_append_block_keys<32>, grid, dim3(64), st, p);
    }
    return hipGetLastError();
}

template <int DIDX>
static void launch_index_t(const IndexParams &p, const SelectPlan &pl, hipStream_t st, bool with_select)
{
    if (pl.all) {
        const long long work = (long long)p.n_q * std::max(p.P / 4, 1);
        const unsigned blocks = (unsigned)std::min<long long>((work + kPoolAllThreads - 1) / kPoolAllThreads, kPoolAllBlocks);
        launch("k_pool_all", (k_pool_all<DIDX>), dim3(std::max(blocks, 1u)), dim3(kPoolAllThreads), st, p);
        return;
    }
    dim3 grid((unsigned)(p.n_q * pl.G));
    if (pl.split) {
        launch("k_index_blocks", (k_index_blocks<kSelectThreads, DIDX, true>), grid, dim3(kSelectThreads), st, p);
        if (with_select)
            launch("k_index_select", (k_index_select<kSelectWideThreads>), dim3((unsigned)p.n_q), dim3(kSelectWideThreads), st, p);
    } else {
        launch("k_index_blocks", (k_index_blocks<kSelectThreads, DIDX, false>), grid, dim3(kSelectThreads), st, p);
    }
}

hipError_t launch_index_blocks(const IndexParams &p, const SelectPlan &pl, int d_idx, hipStream_t st,
                               bool with_select)
{
    if (p.n_q <= 0) return hipSuccess;
    if (d_idx == 64) launch_index_t<64>(p, pl, st, with_select);
    else launch_index_t<32>(p, pl, st, with_select);
    return hipGetLastError();
}

template <int DIDX>
static void launch_topk_t(const TopkParams &p, const SelectPlan &pl, hipStream_t st)
{
    if (pl.dense) {
        launch("k_topk_dense", (k_topk_dense<DIDX>), dim3((unsigned)((p.n_q + kDenseQ - 1) / kDenseQ)), dim3(kDenseWaves * 64), st, p);
        return;
    }
    dim3 grid((unsigned)(p.n_q * pl.G));
    if (pl.split) {
        launch("k_topk_tokens", (k_topk_tokens<kSelectThreads, DIDX, true>), grid, dim3(kSelectThreads), st, p);
        launch("k_topk_select", (k_topk_select<kSelectWideThreads>), dim3((unsigned)p.n_q), dim3(kSelectWideThreads), st, p);
    } else {
        launch("k_topk_tokens", (k_topk_tokens<kSelectThreads, DIDX, false>), grid, dim3(kSelectThreads), st, p);
    }
}

hipError_t launch_topk_tokens(const TopkParams &p, const SelectPlan &pl, int d_idx, hipStream_t st)
{
    if (p.n_q <= 0) return hipSuccess;
    if (d_idx == 64) launch_topk_t<64>(p, pl, st);
    else launch_topk_t<32>(p, pl, st);
    return hipGetLastError();
}

// Pool slots per workgroup of k_pool_tokens: kPoolTokCand candidates' worth,
// or more, so that the launch needs no second round of workgroups.
int pool_tokens_slots(int n_q, int P, int B)
{
    const int per_query = std::max(1, kPoolTokMaxWorkgroups / std::max(n_q, 1));
    return std::max(kPoolTokCand / B, ceil_div(P, per_query));
}

hipError_t launch_pool_tokens(const IndexParams &ip, const TopkParams &tp, int d_idx, hipStream_t st)
{
    if (ip.n_q <= 0) return hipSuccess;
    const int n_slots = pool_tokens_slots(ip.n_q, ip.P, ip.B);
    const dim3 grid((unsigned)(ip.n_q * ceil_div(ip.P, n_slots)));
    // the block keys of a query sit in registers: 16 per thread up to 16,384
    // eligible blocks, 32 per thread up to kFusedEligMax
    const bool wide = (long long)(ip.T - 1) / ip.B + 1 > kLdsKeys;
    constexpr int IPT = kLdsKeys / kSelectWideThreads;
    static_assert(2 * kLdsKeys == kFusedEligMax, "two register key sets cover the fused limit");
    if (d_idx == 64) {
        if (wide) launch("k_pool_tokens", k_pool_tokens<64, 2 * IPT>, grid, dim3(kSelectWideThreads), st, ip, tp, n_slots);
        else launch("k_pool_tokens", k_pool_tokens<64, IPT>, grid, dim3(kSelectWideThreads), st, ip, tp, n_slots);
    } else {
        if (wide) launch("k_pool_tokens", k_pool_tokens<32, 2 * IPT>, grid, dim3(kSelectWideThreads), st, ip, tp, n_slots);
        else launch("k_pool_tokens", k_pool_tokens<32, IPT>, grid, dim3(kSelectWideThreads), st, ip, tp, n_slots);
    }
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *ws, size_t bytes, hipStream_t st)
{
    const size_t n = bytes / sizeof(uint32_t);
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    launch("k_fill_zero", k_fill_zero, dim3(blocks), dim3(256), st, (uint32_t *)ws, n);
    return hipGetLastError();
}

}  // namespace csa2
