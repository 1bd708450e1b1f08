// device_common.h -- device helpers shared by the CSA2 kernels (gfx950, wave64).
//
// Exact Top-N without sorting.  Every selection in CSA2 ranks items by an
// integer score, higher first, ties to the lower item index, and returns the
// chosen items in ascending index order.  That set is found in three steps:
//   1. a two-pass radix histogram (11 + 11 bits) over biased keys finds the
//      N-th largest key `thr` and how many of the keys equal to `thr` belong to
//      the set (`quota`);
//   2. every item with key > thr is in, and so are the first `quota` items
//      (in index order) with key == thr;
//   3. an ordered compaction (block-wide exclusive scans over contiguous
//      per-thread ranges) writes the chosen indices in ascending order.
// Keys are score + 2^21; with |score| <= 64 * 128 * 128 = 2^20 every valid key
// lies in [2^20, 3 * 2^20], and key 0 marks "not a candidate".
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kRadixBits = 11;
constexpr int kRadixBins = 1 << kRadixBits;
constexpr uint32_t kRadixMask = kRadixBins - 1;
constexpr uint32_t kKeyBias = 1u << 21;
constexpr int kLdsKeys = 16384;            // keys held in LDS by one workgroup
constexpr int kLdsKeysPadded = kLdsKeys + kLdsKeys / 32;

// LDS index with one pad word per 32 keys: thread-contiguous ranges of 32
// keys then fall into different banks.
__device__ __forceinline__ int lds_pad(int i) { return i + (i >> 5); }

struct LdsKeys {
    const uint32_t *p;
    __device__ __forceinline__ uint32_t operator()(int i) const { return p[lds_pad(i)]; }
};

// Keys written by other workgroups: loaded at device scope so that no stale
// cache line of this CU can be returned.
struct GlobalKeys {
    const uint32_t *p;
    __device__ __forceinline__ uint32_t operator()(int i) const {
        return __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

// Exclusive prefix sum of one value per thread over a workgroup of NT threads
// (NT a multiple of 64).  `sm` holds NT/64 + 1 words; the workgroup total is
// returned in `total`.  Must be reached by every thread.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t &total, uint32_t *sm)
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) sm[wid] = x;
    __syncthreads();
    if (wid == 0) {
        uint32_t w = (lane < NW) ? sm[lane] : 0u;
        uint32_t s = w;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            uint32_t y = __shfl_up(s, o, 64);
            if (lane >= o) s += y;
        }
        if (lane < NW) sm[lane] = s - w;
        if (lane == NW - 1) sm[NW] = s;
    }
    __syncthreads();
    const uint32_t r = sm[wid] + x - v;
    total = sm[NW];
    __syncthreads();
    return r;
}

// Finds the bin b with  base + count(bins > b) < n  <=  base + count(bins >= b).
// Such a bin exists whenever base < n <= base + total count.  Returns b and
// base + count(bins > b).  `sm` holds NT/64 + 3 words.
template <int NT>
__device__ __forceinline__ void find_bin(const uint32_t *hist, uint32_t n, uint32_t base,
                                         uint32_t &bin, uint32_t &above, uint32_t *sm)
{
    constexpr int BPT = kRadixBins / NT;   // bins per thread, walked from the top
    static_assert(BPT >= 1 && kRadixBins % NT == 0, "NT must divide the bin count");
    const int tid = threadIdx.x;
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < BPT; j++) local += hist[kRadixBins - 1 - (tid * BPT + j)];
    uint32_t total;
    uint32_t a = base + block_excl_scan<NT>(local, total, sm);
#pragma unroll
    for (int j = 0; j < BPT; j++) {
        const int b = kRadixBins - 1 - (tid * BPT + j);
        const uint32_t h = hist[b];
        if (a < n && a + h >= n) {
            sm[NT / 64 + 1] = (uint32_t)b;
            sm[NT / 64 + 2] = a;
        }
        a += h;
    }
    __syncthreads();
    bin = sm[NT / 64 + 1];
    above = sm[NT / 64 + 2];
    __syncthreads();
}

// Selection rule: take key > thr, and keys == thr while their rank among the
// equal keys (in index order) is below quota.
struct Threshold {
    uint32_t thr;
    uint32_t quota;
};

// Threshold of the Top-n over keys(0..count-1) (key 0 = not a candidate).
// With at most n candidates every candidate is taken (thr = 0, quota = 0).
template <int NT, class Keys>
__device__ Threshold radix_threshold(const Keys &keys, int count, uint32_t n, uint32_t *hist,
                                     uint32_t *sm)
{
    const int tid = threadIdx.x;
    for (int b = tid; b < kRadixBins; b += NT) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < count; i += NT) atomicAdd(&hist[keys(i) >> kRadixBits], 1u);
    __syncthreads();
    // bin 0 holds only the zero keys (valid keys are >= 2^20)
    const uint32_t n_valid = (uint32_t)count - hist[0];
    if (n_valid <= n) {
        __syncthreads();
        return {0u, 0u};
    }
    uint32_t b1, above1;
    find_bin<NT>(hist, n, 0u, b1, above1, sm);
    for (int b = tid; b < kRadixBins; b += NT) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < count; i += NT) {
        const uint32_t k = keys(i);
        if ((k >> kRadixBits) == b1) atomicAdd(&hist[k & kRadixMask], 1u);
    }
    __syncthreads();
    uint32_t b2, above2;
    find_bin<NT>(hist, n, above1, b2, above2, sm);
    return {(b1 << kRadixBits) | b2, n - above2};
}

// Writes the chosen indices, ascending, through emit(slot, index); returns the
// number chosen.  Thread t owns the contiguous index range [t*ipt, (t+1)*ipt).
template <int NT, class Keys, class Emit>
__device__ uint32_t ordered_compact(const Keys &keys, int count, Threshold th, Emit emit,
                                    uint32_t *sm)
{
    const int ipt = (count + NT - 1) / NT;
    const int lo = min(count, (int)threadIdx.x * ipt);
    const int hi = min(count, lo + ipt);
    uint32_t ties = 0;
    for (int i = lo; i < hi; i++) ties += (keys(i) == th.thr);
    uint32_t unused;
    const uint32_t tie0 = block_excl_scan<NT>(ties, unused, sm);
    uint32_t taken = 0;
    {
        uint32_t r = tie0;
        for (int i = lo; i < hi; i++) {
            const uint32_t k = keys(i);
            taken += (k > th.thr) || (k == th.thr && r < th.quota);
            r += (k == th.thr);
        }
    }
    uint32_t total;
    uint32_t slot = block_excl_scan<NT>(taken, total, sm);
    {
        uint32_t r = tie0;
        for (int i = lo; i < hi; i++) {
            const uint32_t k = keys(i);
            if ((k > th.thr) || (k == th.thr && r < th.quota)) emit(slot++, i);
            r += (k == th.thr);
        }
    }
    return total;
}

// Nearest integer to sum / n (n >= 1), exact ties to the even integer:
// floor(sum/n + 1/2) computed as a floor division of 2*sum + n by 2n; an exact
// tie leaves no remainder and then lands on the odd neighbour, which is moved
// down by one.
__device__ __forceinline__ int round_mean_half_even(int sum, int n)
{
    const int num = 2 * sum + n, den = 2 * n;
    int q = num / den, r = num - q * den;
    if (r < 0) { q -= 1; r += den; }
    if (r == 0 && (q & 1)) q -= 1;
    return q;
}

// Sum of the 4 signed byte products of a and b, plus c.
__device__ __forceinline__ int dot4_i8(int a, int b, int c)
{
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

// Device-scope "last one in" counter: each of `parties` workgroups calls this
// once after its results are written; exactly one gets true, after all the
// others have arrived, and the counter returns to zero.  Must be reached by
// every thread of the workgroup.  `flag` is one LDS word.
__device__ __forceinline__ bool last_arrival(uint32_t *counter, uint32_t parties, uint32_t *flag)
{
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = atomicInc(counter, parties - 1);
        *flag = (prev == parties - 1) ? 1u : 0u;
    }
    __syncthreads();
    const bool last = *flag != 0;
    if (last) __threadfence();
    return last;
}

}  // namespace csa2
