// select.hip -- block keys, hierarchical block pass and token Top-K (gfx950).
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
// write keys to the workspace; the last workgroup to arrive selects.  With many
// queries (prefill) each workgroup owns one query and keeps its keys in LDS.
// Loads are 16-byte per lane with DIDX/16 lanes per row, so a wave reads
// 1 KiB of consecutive rows per instruction.
#include "device_common.h"
#include "internal.h"

namespace csa2 {

// One lane's 16 dimensions of a block key: the rounded mean of `n` rows that
// start at `rows` (row stride DIDX bytes).
template <int DIDX>
__device__ __forceinline__ int4 block_key_part(const int8_t *rows, int n)
{
    int sum[16];
#pragma unroll
    for (int b = 0; b < 16; b++) sum[b] = 0;
    for (int r = 0; r < n; r++) {
        const int4 v = *reinterpret_cast<const int4 *>(rows + (size_t)r * DIDX);
        const int w[4] = {v.x, v.y, v.z, v.w};
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

__device__ __forceinline__ int dot16_i8(int4 a, int4 b)
{
    int acc = dot4_i8(a.x, b.x, 0);
    acc = dot4_i8(a.y, b.y, acc);
    acc = dot4_i8(a.z, b.z, acc);
    return dot4_i8(a.w, b.w, acc);
}

template <int LPR>
__device__ __forceinline__ int row_reduce(int v)
{
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) v += __shfl_xor(v, o, 64);
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

// ---------------------------------------------------------------- block pass
template <int NT, int DIDX, bool SPLIT>
__global__ __launch_bounds__(NT) void k_index_blocks(IndexParams p)
{
    __shared__ uint32_t s_keys[kLdsKeysPadded];
    __shared__ uint32_t s_hist[kRadixBins];
    __shared__ uint32_t s_sm[NT / 64 + 4];
    constexpr int LPR = DIDX / 16;
    const int q = blockIdx.x % p.n_q;
    const int g = blockIdx.x / p.n_q;
    const int tid = threadIdx.x, part = tid % LPR;
    const int s = p.q_seq[q], t = p.q_pos[q];
    const int jt = t / p.B, n_elig = jt + 1;
    int32_t *ids = p.blk_ids + (size_t)q * p.P;

    if (n_elig <= p.P) {   // the pool is every eligible block
        for (int j = g * NT + tid; j < p.P; j += p.G * NT) ids[j] = (j < n_elig) ? j : -1;
        if (g == 0 && tid == 0) p.blk_cnt[q] = n_elig;
        return;
    }

    const int4 qv = *reinterpret_cast<const int4 *>(p.q_idx + (size_t)q * DIDX + part * 16);
    const int lo = SPLIT ? min(n_elig, g * p.chunk) : 0;
    const int hi = SPLIT ? min(n_elig, lo + p.chunk) : n_elig;
    uint32_t *gkeys = p.ws_keys + (size_t)q * p.ws_stride;
    const int8_t *blk_rows = p.k_blk + (size_t)s * p.nblk * DIDX + part * 16;
    const int8_t *own_rows = p.k_idx + ((size_t)s * p.T + (size_t)jt * p.B) * DIDX + part * 16;

    for (int base = lo; base < hi; base += NT / LPR) {
        const int j = base + tid / LPR;
        int acc = 0;
        if (j < hi) {
            const int4 kv = (j < jt) ? *reinterpret_cast<const int4 *>(blk_rows + (size_t)j * DIDX)
                                     : block_key_part<DIDX>(own_rows, t - jt * p.B + 1);
            acc = dot16_i8(kv, qv);
        }
        acc = row_reduce<LPR>(acc);
        if (j < hi && part == 0) {
            const uint32_t key = (uint32_t)(acc + (int)kKeyBias);
            if (SPLIT) gkeys[j] = key;
            else s_keys[lds_pad(j)] = key;
        }
    }

    bool in_lds = true;
    if (SPLIT) {
        if (!last_arrival(p.ws_cnt + q, (uint32_t)p.G, &s_sm[NT / 64 + 3])) return;
        in_lds = n_elig <= kLdsKeys;
        if (in_lds) {
            const GlobalKeys src{gkeys};
            for (int i = tid; i < n_elig; i += NT) s_keys[lds_pad(i)] = src(i);
        }
    }
    __syncthreads();

    const uint32_t cap = (uint32_t)p.P;
    auto emit = [&](uint32_t slot, int i) { if (slot < cap) ids[slot] = i; };
    uint32_t chosen;
    if (in_lds) {
        const LdsKeys keys{s_keys};
        const Threshold th = radix_threshold<NT>(keys, n_elig, (uint32_t)p.P, s_hist, s_sm);
        chosen = ordered_compact<NT>(keys, n_elig, th, emit, s_sm);
    } else {
        const GlobalKeys keys{gkeys};
        const Threshold th = radix_threshold<NT>(keys, n_elig, (uint32_t)p.P, s_hist, s_sm);
        chosen = ordered_compact<NT>(keys, n_elig, th, emit, s_sm);
    }
    for (int o = (int)chosen + tid; o < p.P; o += NT) ids[o] = -1;
    if (tid == 0) p.blk_cnt[q] = (int32_t)min(chosen, cap);
}

// ---------------------------------------------------------------- token Top-K
template <int NT, int DIDX, bool SPLIT>
__global__ __launch_bounds__(NT) void k_topk_tokens(TopkParams p)
{
    __shared__ uint32_t s_keys[kLdsKeysPadded];
    __shared__ uint32_t s_hist[kRadixBins];
    __shared__ uint32_t s_sm[NT / 64 + 4];
    constexpr int LPR = DIDX / 16;
    const int q = blockIdx.x % p.n_q;
    const int g = blockIdx.x / p.n_q;
    const int tid = threadIdx.x, part = tid % LPR;
    const int s = p.q_seq[q], t = p.q_pos[q];
    const int n_cand = p.blk_cnt[q] * p.B;            // <= P*B <= kLdsKeys
    const int32_t *pool = p.blk_ids + (size_t)q * p.P;

    const int4 qv = *reinterpret_cast<const int4 *>(p.q_idx + (size_t)q * DIDX + part * 16);
    const int lo = SPLIT ? min(n_cand, g * p.chunk) : 0;
    const int hi = SPLIT ? min(n_cand, lo + p.chunk) : n_cand;
    uint32_t *gkeys = p.ws_keys + (size_t)q * p.ws_stride;
    const int8_t *seq_rows = p.k_idx + (size_t)s * p.T * DIDX + part * 16;

    for (int base = lo; base < hi; base += NT / LPR) {
        const int c = base + tid / LPR;
        int acc = 0;
        bool valid = false;
        if (c < hi) {
            const int r = c / p.B;
            const int pos = pool[r] * p.B + (c - r * p.B);
            valid = pos <= t;
            if (valid) acc = dot16_i8(*reinterpret_cast<const int4 *>(seq_rows + (size_t)pos * DIDX), qv);
        }
        acc = row_reduce<LPR>(acc);
        if (c < hi && part == 0) {
            const uint32_t key = valid ? (uint32_t)(acc + (int)kKeyBias) : 0u;
            if (SPLIT) gkeys[c] = key;
            else s_keys[lds_pad(c)] = key;
        }
    }

    if (SPLIT) {
        if (!last_arrival(p.ws_cnt + q, (uint32_t)p.G, &s_sm[NT / 64 + 3])) return;
        const GlobalKeys src{gkeys};
        for (int i = tid; i < n_cand; i += NT) s_keys[lds_pad(i)] = src(i);
    }
    __syncthreads();

    int32_t *out = p.topk + (size_t)q * p.K;
    const int B = p.B;
    const uint32_t cap = (uint32_t)p.K;
    auto emit = [&](uint32_t slot, int i) {
        const int r = i / B;
        if (slot < cap) out[slot] = pool[r] * B + (i - r * B);
    };
    const LdsKeys keys{s_keys};
    const Threshold th = radix_threshold<NT>(keys, n_cand, (uint32_t)p.K, s_hist, s_sm);
    const uint32_t chosen = ordered_compact<NT>(keys, n_cand, th, emit, s_sm);
    for (int o = (int)chosen + tid; o < p.K; o += NT) out[o] = -1;
    if (tid == 0) p.topk_cnt[q] = (int32_t)min(chosen, cap);
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
        pl.key_bytes = (size_t)n_q * (size_t)n_items * sizeof(uint32_t);
    }
    return pl;
}

SelectPlan plan_index(int n_q, int T, int B, int P, int d_idx)
{
    const long long n_elig_max = (long long)(T - 1) / B + 1;
    if (n_elig_max <= P) return SelectPlan{1, (int)n_elig_max, false, 0};
    return plan_scan(n_q, n_elig_max, d_idx, n_elig_max > kLdsKeys);
}

SelectPlan plan_topk(int n_q, int B, int P, int K, int d_idx)
{
    (void)K;
    return plan_scan(n_q, (long long)P * B, d_idx, false);
}

// ---------------------------------------------------------------- launches
hipError_t launch_block_keys(const BlockKeysParams &p, int n_seq, int d_idx, hipStream_t st)
{
    const int n = (p.blk_end - p.blk_begin) * (d_idx / 16);
    if (n <= 0 || n_seq <= 0) return hipSuccess;
    dim3 grid(ceil_div(n, 256), n_seq);
    if (d_idx == 64) hipLaunchKernelGGL(k_block_keys<64>, grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_block_keys<32>, grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

template <int DIDX>
static void launch_index_t(const IndexParams &p, const SelectPlan &pl, hipStream_t st)
{
    dim3 grid((unsigned)(p.n_q * pl.G));
    if (pl.split) hipLaunchKernelGGL((k_index_blocks<kSelectThreads, DIDX, true>), grid, dim3(kSelectThreads), 0, st, p);
    else hipLaunchKernelGGL((k_index_blocks<kSelectThreads, DIDX, false>), grid, dim3(kSelectThreads), 0, st, p);
}

hipError_t launch_index_blocks(const IndexParams &p, const SelectPlan &pl, int d_idx, hipStream_t st)
{
    if (p.n_q <= 0) return hipSuccess;
    if (d_idx == 64) launch_index_t<64>(p, pl, st);
    else launch_index_t<32>(p, pl, st);
    return hipGetLastError();
}

template <int DIDX>
static void launch_topk_t(const TopkParams &p, const SelectPlan &pl, hipStream_t st)
{
    dim3 grid((unsigned)(p.n_q * pl.G));
    if (pl.split) hipLaunchKernelGGL((k_topk_tokens<kSelectThreads, DIDX, true>), grid, dim3(kSelectThreads), 0, st, p);
    else hipLaunchKernelGGL((k_topk_tokens<kSelectThreads, DIDX, false>), grid, dim3(kSelectThreads), 0, st, p);
}

hipError_t launch_topk_tokens(const TopkParams &p, const SelectPlan &pl, int d_idx, hipStream_t st)
{
    if (p.n_q <= 0) return hipSuccess;
    if (d_idx == 64) launch_topk_t<64>(p, pl, st);
    else launch_topk_t<32>(p, pl, st);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *ws, size_t bytes, hipStream_t st)
{
    const size_t n = bytes / sizeof(uint32_t);
    if (n == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(k_fill_zero, dim3(blocks), dim3(256), 0, st, (uint32_t *)ws, n);
    return hipGetLastError();
}

}  // namespace csa2
