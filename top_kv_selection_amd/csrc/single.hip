// single.hip -- the fused decode layer group as one launch (opt-in entry
// point csa2_layer_group_single).
//
// The fused layer group of a few decode queries is four launches: block
// scoring, pool selection with token scoring, token Top-K with chunked
// attention, and the merge of the chunk records.  Here they are four phases
// of one kernel.  Every workgroup takes, phase by phase, the workgroups of
// the separate launches ("virtual workgroups") by index and runs the same
// kernel bodies on them.  A virtual workgroup waits only for what its own
// query needs from the previous phase: the workgroups that produce it count
// themselves into a per-query counter after an agent-scope release (their
// stores written back from the L2 of their XCD), and the consumer polls the
// counter and then acquires at agent scope (its caches invalidated).  Window
// chunks need nothing from the selection and run at once; queries do not wait
// for one another.  Each counter starts at zero (workspace head); the last
// workgroup to finish, when every workgroup is past every wait, clears them.
//
// Residency: every workgroup must be resident, since consumers spin.  The
// launch is cooperative when the stream is not capturing a graph; inside a
// capture it is an ordinary launch (stream order leaves the device to it) of
// at most as many workgroups as the device holds at once.  Every wait is
// bounded (kSinglePolls polls), so a broken assumption gives wrong output,
// never a hang.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace csa2 {

constexpr int kSingleThreads = 1024;       // one 16-wave workgroup per CU
constexpr int kSinglePolls = 1 << 20;      // polls of one wait before it gives up (~1 s)
constexpr int kSingleMergesPerWg = kSingleThreads / (32 * kCombineHeads);   // one 64-thread merge per wave
static_assert(kSelectWideThreads == kSingleThreads && kCkWaves * 64 == kSingleThreads,
              "the pool-scoring and chunk bodies run on a whole workgroup");
static_assert(kSingleMergesPerWg <= 64, "the merge waits are polled by wave 0");

struct SingleParams {
    uint32_t *ctr;        // [3 n_q + 1]: per-query counts of phases 1, 2 and 3, then the done count
    int n_q;
    int idx_G, n_idx;     // phase 1: block-scoring workgroups per query, in all
    int pool_G, n_pool, n_slots;   // phase 2: pool-scoring workgroups per query, in all; pool slots each
    int n_att, att_need;  // phase 3: chunk workgroups in all, per query
    int n_merge;          // phase 4: 64-thread merges
};

// This workgroup's global stores are done and visible at agent scope; then
// it counts itself.  Every wave waits for its own stores to reach the L2 of
// its XCD (all waves of a workgroup share one CU, hence one L2); one wave
// then writes that L2 back (one release fence, not one per wave: each is a
// writeback of the whole L2) and counts the workgroup.
__device__ __forceinline__ void single_arrive(uint32_t *c)
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The threads with `poll` set (all in wave 0) poll their counter *c until it
// reaches `need` (bounded); wave 0 then acquires at agent scope, which
// invalidates the caches of the workgroup's CU and XCD, before the barrier
// lets the other waves read.
__device__ __forceinline__ void single_wait(uint32_t *c, bool poll, uint32_t need)
{
    if (threadIdx.x < 64) {
        if (poll)
            for (int it = 0; it < kSinglePolls && __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need;
                 it++)
                __builtin_amdgcn_s_sleep(2);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
}

template <int DIDX, int IPT>
__global__ __launch_bounds__(kSingleThreads) void k_decode_single(IndexParams ip, TopkParams tp, AttendParams ap,
                                                                  SingleParams sp)
{
    uint32_t *c1 = sp.ctr, *c2 = sp.ctr + sp.n_q, *c3 = sp.ctr + 2 * sp.n_q, *done = sp.ctr + 3 * sp.n_q;
    const int tid = threadIdx.x;

    // phase 1: block scoring (each query's keys and histogram to the workspace)
    for (int b = blockIdx.x; b < sp.n_idx; b += gridDim.x) {
        index_blocks_body<kSingleThreads, DIDX, true>(ip, b);
        single_arrive(&c1[b / sp.idx_G]);
    }
    // phase 2: pool selection and token scoring, once every block key of the query is in
    for (int b = blockIdx.x; b < sp.n_pool; b += gridDim.x) {
        const int q = b / sp.pool_G;
        single_wait(&c1[q], tid == 0, (uint32_t)sp.idx_G);
        pool_tokens_body<DIDX, IPT>(ip, tp, sp.n_slots, sp.pool_G, b);
        single_arrive(&c2[q]);
    }
    // phase 3: token Top-K and the main chunks once every token key of the
    // query is in; window chunks at once
    const int n_main = ap.n_q_pad * ap.n_mc;
    for (int b = blockIdx.x; b < sp.n_att; b += gridDim.x) {
        const int i = (b < n_main ? b : b - n_main) % ap.n_q_pad;
        if (i >= ap.n_q) continue;   // a padding slot of the numbering (uniform over the workgroup)
        if (b < n_main) single_wait(&c2[i], tid == 0, (uint32_t)sp.pool_G);
        attend_chunks_body<true>(ap, b);   // (each iteration ends at a barrier, so LDS is free)
        single_arrive(&c3[i]);
    }
    // phase 4: the merges, one per wave, once every record of the wave's query is in
    const int wave = tid >> 6, lane = tid & 63;
    for (int b0 = blockIdx.x * kSingleMergesPerWg; b0 < sp.n_merge; b0 += gridDim.x * kSingleMergesPerWg) {
        const int bt = b0 + tid, it = bt % ap.n_q_pad;
        single_wait(&c3[it < ap.n_q ? it : 0], tid < kSingleMergesPerWg && bt < sp.n_merge && it < ap.n_q,
                    (uint32_t)sp.att_need);
        const int b = b0 + wave;
        if (b < sp.n_merge) combine_body(ap, b, lane);
    }
    // the last workgroup out clears the counters for the next call
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (prev == gridDim.x - 1) {
            for (int x = 0; x < 3 * sp.n_q; x++) __hip_atomic_store(&sp.ctr[x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

size_t single_ctr_bytes(int n_q)
{
    return ((size_t)(3 * n_q + 1) * sizeof(uint32_t) + 255) / 256 * 256;
}

template <int DIDX, int IPT>
static hipError_t launch_single_t(IndexParams ip, const TopkParams &tp, const AttendParams &ap, SingleParams sp,
                                  long long n_elig_max, hipStream_t st)
{
    auto kernel = k_decode_single<DIDX, IPT>;
    int dev = 0, n_cu = 0, per_cu = 0;
    if (hipError_t e = hipGetDevice(&dev)) return e;
    if (hipError_t e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) return e;
    if (hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kSingleThreads, 0)) return e;
    const int capacity = n_cu * per_cu;
    if (capacity < 1) return hipErrorInvalidConfiguration;
    // phase 1: as many block-scoring workgroups per query as fill the grid
    sp.idx_G = (int)std::max<long long>(1, std::min<long long>(capacity / sp.n_q, n_elig_max));
    sp.n_idx = sp.n_q * sp.idx_G;
    ip.G = sp.idx_G;
    ip.chunk = (int)((n_elig_max + sp.idx_G - 1) / sp.idx_G);
    const int n_phys = (int)std::min<long long>(
        capacity, std::max<long long>({sp.n_idx, sp.n_pool, sp.n_att,
                                       (sp.n_merge + kSingleMergesPerWg - 1) / kSingleMergesPerWg}));
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipError_t e = hipStreamIsCapturing(st, &cs)) return e;
    if (cs != hipStreamCaptureStatusNone) {
        launch("k_decode_single", kernel, dim3((unsigned)n_phys), dim3(kSingleThreads), st, ip, tp, ap, sp);
        return hipGetLastError();
    }
    void *argv[] = {&ip, (void *)&tp, (void *)&ap, &sp};
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const bool timed = profile_events("k_decode_single", st, e0, e1);
    if (timed) (void)hipEventRecord(e0, st);
    const hipError_t e = hipLaunchCooperativeKernel((const void *)kernel, dim3((unsigned)n_phys), dim3(kSingleThreads),
                                                    argv, 0, st);
    if (timed) (void)hipEventRecord(e1, st);
    return e;
}

hipError_t launch_decode_single(const IndexParams &ip, const TopkParams &tp, const AttendParams &ap0,
                                const AttendPlan &pl, int d_idx, uint32_t *ctr, hipStream_t st)
{
    if (ip.n_q <= 0) return hipSuccess;
    if (!pl.chunks) return hipErrorInvalidValue;
    AttendParams ap = ap0;
    ap.n_q_pad = (ap.n_q + 7) / 8 * 8;
    ap.n_mc = pl.n_mc;
    ap.n_wc = pl.n_wc;
    ap.n_splits = ap.n_mc + ap.n_wc;
    SingleParams sp{};
    sp.ctr = ctr;
    sp.n_q = ip.n_q;
    sp.n_slots = pool_tokens_slots(ip.n_q, ip.P, ip.B);
    sp.pool_G = (ip.P + sp.n_slots - 1) / sp.n_slots;
    sp.n_pool = ip.n_q * sp.pool_G;
    sp.n_att = ap.n_q_pad * (ap.n_mc + ap.n_layers * ap.n_wc);
    sp.att_need = ap.n_mc + ap.n_layers * ap.n_wc;
    sp.n_merge = ap.n_q_pad * (ap.H / 16) * ap.n_layers * (16 / kCombineHeads);
    const long long n_elig_max = (long long)(ip.T - 1) / ip.B + 1;
    // the block keys of a query sit in registers: 16 per thread up to 16,384
    // eligible blocks, 32 per thread up to kFusedEligMax (as k_pool_tokens)
    const bool wide = n_elig_max > kLdsKeys;
    constexpr int IPT = kLdsKeys / kSingleThreads;
    if (d_idx == 64)
        return wide ? launch_single_t<64, 2 * IPT>(ip, tp, ap, sp, n_elig_max, st)
                    : launch_single_t<64, IPT>(ip, tp, ap, sp, n_elig_max, st);
    return wide ? launch_single_t<32, 2 * IPT>(ip, tp, ap, sp, n_elig_max, st)
                : launch_single_t<32, IPT>(ip, tp, ap, sp, n_elig_max, st);
}

}  // namespace csa2
