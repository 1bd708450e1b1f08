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
constexpr int kRsrcWord3 = 0x00020000;   // buffer resource word 3: raw buffer, 32-bit data format
constexpr int kLdsKeys = 16384;            // keys held in LDS by one workgroup
constexpr int kLdsKeysPadded = kLdsKeys + kLdsKeys / 32;
// Histograms in LDS also carry one pad word per 32 bins, so that the wave that
// walks them (32 consecutive bins per lane) reads without bank conflicts.  A
// pass-2 histogram is followed by 64 trash words (see threshold_regs); LDS
// arrays holding two histograms are 2 * kHistWords + 64 words.
constexpr int kHistWords = kRadixBins + kRadixBins / 32;
constexpr int kHist2Words = 2 * kHistWords + 64;
__device__ __forceinline__ int hist_pad(int b) { return b + (b >> 5); }

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also waits
// for every outstanding global store of the wave (a full memory round trip);
// no kernel here has one wave read another wave's global writes within a
// launch (that data goes through LDS), so LDS ordering is all they need.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS index with one pad word per 32 keys: thread-contiguous ranges of 32
// keys then fall into different banks.
__device__ __forceinline__ int lds_pad(int i) { return i + (i >> 5); }

struct LdsKeys {
    const uint32_t *p;
    __device__ __forceinline__ uint32_t operator()(int i) const { return p[lds_pad(i)]; }
};

// Keys in global memory, written by an earlier launch.
struct GlobalKeys {
    const uint32_t *p;
    __device__ __forceinline__ uint32_t operator()(int i) const { return p[i]; }
};

// Orders this wave's LDS accesses in the compiler; the hardware performs one
// wave's LDS instructions in issue order.
__device__ __forceinline__ void wave_lds_order()
{
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Inclusive prefix sum across the 64 lanes of a wave with DPP moves (row
// shifts, then row broadcasts), which stay in the VALU instead of the LDS
// crossbar that __shfl_up uses.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x)
{
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Exclusive prefix sum of one value per thread over a workgroup of NT threads
// (NT a multiple of 64).  `sm` holds NT/64 + 1 words; the workgroup total is
// returned in `total`.  Must be reached by every thread.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t &total, uint32_t *sm)
{
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) sm[wid] = x;
    lds_barrier();
    if (wid == 0) {
        const uint32_t w = (lane < NW) ? sm[lane] : 0u;
        const uint32_t s = wave_incl_scan(w);
        if (lane < NW) sm[lane] = s - w;
        if (lane == NW - 1) sm[NW] = s;
    }
    lds_barrier();
    const uint32_t r = sm[wid] + x - v;
    total = sm[NW];
    lds_barrier();
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
    for (int j = 0; j < BPT; j++) local += hist[hist_pad(kRadixBins - 1 - (tid * BPT + j))];
    uint32_t total;
    uint32_t a = base + block_excl_scan<NT>(local, total, sm);
#pragma unroll
    for (int j = 0; j < BPT; j++) {
        const int b = kRadixBins - 1 - (tid * BPT + j);
        const uint32_t h = hist[hist_pad(b)];
        if (a < n && a + h >= n) {
            sm[NT / 64 + 1] = (uint32_t)b;
            sm[NT / 64 + 2] = a;
        }
        a += h;
    }
    lds_barrier();
    bin = sm[NT / 64 + 1];
    above = sm[NT / 64 + 2];
    lds_barrier();
}

// Selection rule: take key > thr, and keys == thr while their rank among the
// equal keys (in index order) is below quota.
struct Threshold {
    uint32_t thr;
    uint32_t quota;
};

// Threshold of the Top-n over keys(0..count-1) (key 0 = not a candidate).
// With at most n candidates every candidate is taken (thr = 0, quota = 0).
// With have_pass1, `hist` already holds the pass-1 histogram.
template <int NT, class Keys>
__device__ Threshold radix_threshold(const Keys &keys, int count, uint32_t n, uint32_t *hist,
                                     uint32_t *sm, bool have_pass1 = false)
{
    const int tid = threadIdx.x;
    if (!have_pass1) {
        for (int b = tid; b < kHistWords; b += NT) hist[b] = 0;
        lds_barrier();
        for (int i = tid; i < count; i += NT) atomicAdd(&hist[hist_pad(keys(i) >> kRadixBits)], 1u);
    }
    lds_barrier();
    // bin 0 holds only the zero keys (valid keys are >= 2^20)
    const uint32_t n_valid = (uint32_t)count - hist[0];
    if (n_valid <= n) {
        lds_barrier();
        return {0u, 0u};
    }
    uint32_t b1, above1;
    find_bin<NT>(hist, n, 0u, b1, above1, sm);
    for (int b = tid; b < kHistWords; b += NT) hist[b] = 0;
    lds_barrier();
    for (int i = tid; i < count; i += NT) {
        const uint32_t k = keys(i);
        if ((k >> kRadixBits) == b1) atomicAdd(&hist[hist_pad(k & kRadixMask)], 1u);
    }
    lds_barrier();
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

// find_bin done by wave 0 alone, in two levels: lane l sums 32 bins (walked
// from the top), a wave scan and a ballot find the one lane whose bins hold the
// crossing, then that lane's 32 bins are spread over 32 lanes for a second
// scan and ballot.  No per-bin loop; one barrier.  `res` is 2 LDS words.
// Requires base < n <= base + (total count).  Must be reached by every thread.
template <int NT>
__device__ __forceinline__ void find_bin_wave(const uint32_t *hist, uint32_t n, uint32_t base,
                                              uint32_t &bin, uint32_t &above, uint32_t *res)
{
    static_assert(kRadixBins == 64 * 32, "one wave covers the bins, 32 per lane");
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const uint32_t *src = hist + hist_pad(kRadixBins - 32 * (lane + 1));   // conflict-free
        uint32_t local = 0;
#pragma unroll
        for (int j = 0; j < 32; j++) local += src[j];
        const uint32_t a0 = base + wave_incl_scan(local) - local;   // count above this lane's bins
        const unsigned long long hit = __ballot(a0 < n && a0 + local >= n);
        const int L = __builtin_ctzll(hit);
        const uint32_t aL = (uint32_t)__builtin_amdgcn_readlane((int)a0, L);
        // bin of lane j (< 32): 2047 - 32L - j, descending
        const int b = kRadixBins - 1 - 32 * L - lane;
        const uint32_t h = (lane < 32) ? hist[hist_pad(b)] : 0u;
        const uint32_t ab = aL + wave_incl_scan(h) - h;
        const unsigned long long hit2 = __ballot(lane < 32 && ab < n && ab + h >= n);
        if (lane == __builtin_ctzll(hit2)) {
            res[0] = (uint32_t)b;
            res[1] = ab;
        }
    }
    lds_barrier();
    bin = res[0];
    above = res[1];
}

// ---- register-resident selection (at most NT * IPT items) -----------------
// Thread t owns items [t*IPT, t*IPT + IPT) as keys k[0..IPT) (0 past the end).
// The pass-1 histogram (bins of key >> 11 over all items) must already be in
// `hist` (LDS).

template <int NT, int IPT>
__device__ Threshold threshold_regs(const uint32_t (&k)[IPT], int count, uint32_t n, uint32_t *hist,
                                    uint32_t *sm)
{
    const uint32_t n_valid = (uint32_t)count - hist[0];
    if (n_valid <= n) {
        lds_barrier();
        return {0u, 0u};
    }
    uint32_t b1, above1;
    find_bin_wave<NT>(hist, n, 0u, b1, above1, sm + NT / 64 + 1);
    // pass 2 into a second histogram (the barrier in find_bin_wave has
    // ordered every read of the first).  Branch-free: a key outside bin b1
    // counts into a trash word of its own lane (past the histogram), so every
    // key costs one LDS atomic and no divergent branch.
    uint32_t *hist2 = hist + kHistWords;
    const int trash = kHistWords + (threadIdx.x & 63);
#pragma unroll
    for (int j = 0; j < IPT; j++) {
        const int slot = ((k[j] >> kRadixBits) == b1) ? hist_pad(k[j] & kRadixMask) : trash;
        atomicAdd(&hist2[slot], 1u);
    }
    lds_barrier();
    uint32_t b2, above2;
    find_bin_wave<NT>(hist2, n, above1, b2, above2, sm + NT / 64 + 1);
    return {(b1 << kRadixBits) | b2, n - above2};
}

// One scan of packed (ties << 16 | greater) counts gives both the rank of a
// thread's first tie and the number of greater items before it; the slot of a
// chosen item is (greater items before it) + min(quota, ties before it).
template <int NT, int IPT, class Emit>
__device__ uint32_t compact_regs(const uint32_t (&k)[IPT], Threshold th, Emit emit, uint32_t *sm)
{
    static_assert(NT * IPT < 65536, "packed counts are 16-bit");
    const int lo = (int)threadIdx.x * IPT;
    uint32_t ties = 0, gt = 0;
#pragma unroll
    for (int j = 0; j < IPT; j++) {
        ties += (k[j] == th.thr);
        gt += (k[j] > th.thr);
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan<NT>((ties << 16) | gt, tot, sm);
    const uint32_t tie0 = pre >> 16, gt0 = pre & 0xffffu;
    const uint32_t total = (tot & 0xffffu) + min(tot >> 16, th.quota);
    static_assert(IPT <= 32, "one bit per item");
    uint32_t gt_mask = 0, tie_mask = 0;
#pragma unroll
    for (int j = 0; j < IPT; j++) {
        gt_mask |= (uint32_t)(k[j] > th.thr) << j;
        tie_mask |= (uint32_t)(k[j] == th.thr) << j;
    }
    // ties whose rank is at least quota are dropped
    uint32_t take = gt_mask;
    if (tie0 < th.quota) {
        uint32_t tm = tie_mask;
        for (uint32_t r = tie0; tm && r < th.quota; r++) {
            take |= tm & (0u - tm);      // lowest remaining tie
            tm &= tm - 1;
        }
    }
    while (take) {
        const int j = __builtin_ctz(take);
        take &= take - 1;
        const uint32_t below = (1u << j) - 1u;
        emit(gt0 + __builtin_popcount(gt_mask & below) + min(tie0 + __builtin_popcount(tie_mask & below), th.quota),
             lo + j);
    }
    return total;
}

// Adds a workgroup's LDS histogram into a global one (non-zero bins only).
template <int NT>
__device__ __forceinline__ void flush_hist(const uint32_t *hist, uint32_t *ghist)
{
    for (int b = threadIdx.x; b < kRadixBins; b += NT) {
        const uint32_t c = hist[hist_pad(b)];
        if (c) atomicAdd(&ghist[b], c);
    }
}

// Global histogram -> registers (issue only; pair with store_hist after other
// loads have been issued), so its round trip overlaps the key loads.
template <int NT>
struct HistRegs {
    uint32_t v[kRadixBins / NT];
};
template <int NT>
__device__ __forceinline__ void load_hist(const uint32_t *ghist, HistRegs<NT> &h)
{
#pragma unroll
    for (int u = 0; u < kRadixBins / NT; u++) h.v[u] = ghist[u * NT + threadIdx.x];
}
// Writes the loaded counts into LDS hist[0..) (padded) and clears the pass-2
// histogram, leaving the global one as it is (other workgroups still read it);
// ends with a barrier.
template <int NT>
__device__ __forceinline__ void hist_to_lds(const HistRegs<NT> &h, uint32_t *hist)
{
#pragma unroll
    for (int u = 0; u < kRadixBins / NT; u++) hist[hist_pad(u * NT + threadIdx.x)] = h.v[u];
    for (int b = threadIdx.x; b < kHistWords; b += NT) hist[kHistWords + b] = 0u;
    lds_barrier();
}

// Writes the loaded counts into LDS hist[0..) (padded), clears the pass-2
// histogram, leaves the global one zeroed, and ends with a barrier.
template <int NT>
__device__ __forceinline__ void store_hist(const HistRegs<NT> &h, uint32_t *ghist, uint32_t *hist)
{
#pragma unroll
    for (int u = 0; u < kRadixBins / NT; u++) {
        const int b = u * NT + threadIdx.x;
        hist[hist_pad(b)] = h.v[u];
        ghist[b] = 0u;
    }
    for (int b = threadIdx.x; b < kHistWords; b += NT) hist[kHistWords + b] = 0u;
    lds_barrier();
}

// Issues the loads of this thread's IPT keys of a global key row that holds
// `row_len` words (a multiple of 4, at least 4, 16-byte aligned); entries past
// the row are 0.  The count of valid keys is applied later by mask_keys, so
// the loads do not wait for it.  Every load is issued (from a slot clamped
// into the row) and its value masked afterwards: a load under a divergent
// branch can make the compiler wait for it before issuing the next.
template <int IPT>
__device__ __forceinline__ void load_keys_global(const uint32_t *g, int row_len, uint32_t (&k)[IPT])
{
    const int lo = (int)threadIdx.x * IPT;
#pragma unroll
    for (int u = 0; u < IPT / 4; u++) {
        const int i = lo + 4 * u;
        const uint4 v = *reinterpret_cast<const uint4 *>(g + min(i, row_len - 4));
        const bool in = i < row_len;
        k[4 * u] = in ? v.x : 0u;
        k[4 * u + 1] = in ? v.y : 0u;
        k[4 * u + 2] = in ? v.z : 0u;
        k[4 * u + 3] = in ? v.w : 0u;
    }
}
template <int IPT>
__device__ __forceinline__ void mask_keys(int count, uint32_t (&k)[IPT])
{
    const int lo = (int)threadIdx.x * IPT;
#pragma unroll
    for (int j = 0; j < IPT; j++)
        if (lo + j >= count) k[j] = 0u;
}

template <int IPT>
__device__ __forceinline__ void load_keys_lds(const uint32_t *lds, int count, uint32_t (&k)[IPT])
{
    const int lo = (int)threadIdx.x * IPT;
#pragma unroll
    for (int j = 0; j < IPT; j++) k[j] = (lo + j < count) ? lds[lds_pad(lo + j)] : 0u;
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

}  // namespace csa2
