// attend.hip -- sparse + sliding-window attention (gfx950).
//
// "Sparse attention" on the DeepSeek V4.1 Flash page (k-a.in): a query reads
// its Top-K main-KV entries plus a window of the most recent tokens.  Per head,
// one softmax runs over both sets together; the window K/V are the layer's own
// ("CSA2 with cross-layer reuse": every mode computes its own main Q and
// window K/V) while the main K/V and the indices may be shared by a group of
// layers.
//
// Kernels, chosen by how many (query, layer, head group of 16) items a call
// has (bf16, D = 128); all of them run S^T = K Q^T and O^T += V^T P^T on
// v_mfma_f32_16x16x32_bf16 with 16 heads as the MFMA N dimension and an fp32
// online softmax (one head per lane column):
//  * k_attend_chunks + k_attend_combine (fewer than 256 items, as in
//    decode): the key lists are cut into 64-key chunks taken by different
//    workgroups; a main chunk's rows are brought into LDS once for every
//    layer of a group; each (item, chunk) writes a (max, sum, acc) record and
//    a second launch merges an item's records;
//  * k_attend_mfma (256 items, one round of a workgroup per CU): one
//    workgroup of 8 waves per item;
//  * k_attend_rows (more items, as in prefill): one wave per item at a time,
//    each wave walking up to four items;
//  * k_attend_window (window-only layers of 1,024 items or more): the windows
//    of 32 neighbouring queries staged in LDS once;
//  * k_attend_generic (fp32, or any H and D in {64, 128}): one wave per head,
//    keys in sequence, fp32 online softmax on the vector ALU.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace csa2 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr float kLn2 = 0.69314718055994530942f;

// A 16-byte load that streams past the caches: the many-query kernels read
// each query row once, and keeping those rows out of L2 and the MALL leaves
// room for the K/V rows that other workgroups gather again.
typedef int i32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t load_nt_bf16x8(const uint16_t *src)
{
    return __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(reinterpret_cast<const i32x4_nt *>(src)));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// round to nearest even (gfx950's v_cvt_pk_bf16_f32; a NaN stays a NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return f32_to_bf16(v); }

// Window of query position t: [w0, w0 + nw), clipped to the rows supplied.
struct Window {
    int w0, nw;
};
__device__ __forceinline__ Window window_of(int t, int W, int swa_first, int swa_len)
{
    int w0 = max(0, t - W + 1);
    w0 = max(w0, swa_first);
    const int w1 = min(t, swa_first + swa_len - 1);
    return {w0, (W > 0 && w1 >= w0) ? w1 - w0 + 1 : 0};
}

// ============================================================ generic kernel
template <typename T, int D>
__global__ __launch_bounds__(256) void k_attend_generic(AttendParams p)
{
    constexpr int E = D / 64;   // elements per lane
    const int i = blockIdx.x, l = blockIdx.y;
    const int h = blockIdx.z * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= p.H) return;
    const int s = p.q_seq[i], t = p.q_pos[i];
    const int cnt = p.topk ? p.topk_cnt[i] : 0;
    const Window win = window_of(t, p.W, p.swa_first, p.swa_len);
    const T *qrow = (const T *)p.q + (((size_t)l * p.n_q + i) * p.H + h) * D;
    const T *kmain = (const T *)p.k_main + (size_t)s * p.T * D;
    const T *vmain = (const T *)p.v_main + (size_t)s * p.T * D;
    const T *kswa = (const T *)p.k_swa + ((size_t)l * p.n_seq + s) * p.swa_len * D;
    const T *vswa = (const T *)p.v_swa + ((size_t)l * p.n_seq + s) * p.swa_len * D;
    const int32_t *tk = p.topk ? p.topk + (size_t)i * p.K : nullptr;

    float qv[E], acc[E];
#pragma unroll
    for (int e = 0; e < E; e++) {
        qv[e] = to_f32<T>(qrow[lane * E + e]);
        acc[e] = 0.f;
    }
    float m = -INFINITY, lsum = 0.f;
    const int n_keys = cnt + win.nw;
    for (int kk = 0; kk < n_keys; kk++) {
        const T *kr, *vr;
        if (kk < cnt) {
            const size_t off = (size_t)tk[kk] * D;
            kr = kmain + off;
            vr = vmain + off;
        } else {
            const size_t off = (size_t)(win.w0 + (kk - cnt) - p.swa_first) * D;
            kr = kswa + off;
            vr = vswa + off;
        }
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < E; e++) dot += qv[e] * to_f32<T>(kr[lane * E + e]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
        const float logit = dot * p.scale_log2;
        const float m_new = fmaxf(m, logit);
        const float alpha = exp2f(m - m_new);
        const float pw = exp2f(logit - m_new);
        lsum = lsum * alpha + pw;
#pragma unroll
        for (int e = 0; e < E; e++) acc[e] = acc[e] * alpha + pw * to_f32<T>(vr[lane * E + e]);
        m = m_new;
    }
    T *orow = (T *)p.out + (((size_t)l * p.n_q + i) * p.H + h) * D;
    const float inv = 1.f / lsum;
#pragma unroll
    for (int e = 0; e < E; e++) orow[lane * E + e] = from_f32<T>(acc[e] * inv);
    if (p.lse && lane == 0) p.lse[((size_t)l * p.n_q + i) * p.H + h] = (m + log2f(lsum)) * kLn2;
}

// ============================================================ MFMA kernel
constexpr int kWaves = 8;                      // waves per workgroup, 32 keys each per step
constexpr int kStepKeys = kWaves * 32;         // keys per workgroup step (32 keys per wave)
constexpr int kRowChunk = kAttendRowChunk;     // row codes staged in LDS at once
static_assert(kRowChunk % (kWaves * 64) == 0 && kRowChunk % kStepKeys == 0, "whole staging rounds and steps");
constexpr int kVtStride = 40;                  // bf16 per V^T row in LDS (32 keys + pad)
// After the key loop a wave's V^T buffer holds its partial output, 16 heads x
// kObStride floats: with 144 floats per head, the 16-byte writes of a wave
// (lane -> head r16, dims 16m + 4g) cover every bank equally.
constexpr int kObStride = 144;
static_assert(16 * kObStride * 4 <= 128 * kVtStride * 2, "a wave's partial output fits its V^T buffer");
constexpr int kHeadRec = 4 + 128;              // chunk record per head: max, sum, 2 pad, acc[128]
constexpr int kPartFloats = 16 * kHeadRec;     // one chunk record (16 heads), 16-byte aligned
constexpr int kMergeBatch = 16;                // chunk records loaded at once by the merge

// Key slot e (0..7) of lane group g inside a 32-key step: the keys whose
// scores this lane holds after the QK MFMA (rows 4g..4g+3 of tile 0 and of
// tile 1).  Both PV operands use this same order along the contraction.
__device__ __forceinline__ int slot_key(int g, int e) { return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4); }

// One workgroup per (query, head group of 16, layer), walking the whole key
// list.  K rows go straight from memory into the MFMA A operand (16 B per
// lane, each row read once); V rows are written transposed into LDS so that
// the PV operand is two 8-byte LDS reads per lane.  Workgroups are numbered
// query-fastest with the query count padded to a multiple of 8, so with
// round-robin XCD dispatch every layer of a query runs on one XCD and the
// shared main rows are fetched from HBM once and then hit that XCD's L2.
// FUSED: the token Top-K is taken first, from the token keys and histogram
// (layer-group decode).
template <bool FUSED>
__global__ __launch_bounds__(kWaves * 64) void k_attend_mfma(AttendParams p)
{
    constexpr int NT = kWaves * 64, IPT = kLdsKeys / NT;
    constexpr int KPW = 32, NTAU = 2, STEP = kWaves * KPW;   // keys per wave and step: two QK tiles
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[kWaves][128 * kVtStride];
    __shared__ float s_ml[kWaves][16][2];
    __shared__ int s_rows[kRowChunk];
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[FUSED ? kHist2Words : 4];
    __shared__ int32_t s_pool[FUSED ? kFusedPoolLds : 4];
    static_assert(!FUSED || kFusedPoolLds % (kWaves * 64) == 0, "whole pool loads per thread");
    __shared__ uint32_t s_sm[NT / 64 + 4];

    const int HG = p.H / 16;
    const int id = blockIdx.x;
    const int i = id % p.n_q_pad;
    const int rest = id / p.n_q_pad;
    const int hg = rest % HG;
    const int l = rest / HG;
    if (i >= p.n_q) return;

    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
    const int s = p.q_seq[i], t = p.q_pos[i];
    const Window win = window_of(t, p.W, p.swa_first, p.swa_len);
    int cnt;
    if constexpr (FUSED) {
        // Exact token Top-K from the token keys (same selection as the
        // standalone Top-K call); selected slots in this workgroup's share of
        // the key list go straight into s_rows.
        HistRegs<NT> hr;
        load_hist<NT>(p.sel_hist + (size_t)i * kRadixBins, hr);
        uint32_t k[IPT];
        load_keys_global<IPT>(p.sel_keys + (size_t)i * p.sel_stride, (int)p.sel_stride, k);
        // every pool slot is read (slots past the count are never used), so
        // these loads go out with the others instead of waiting for the count
        constexpr int PPT = kFusedPoolLds / NT;
        int32_t pv[PPT];
#pragma unroll
        for (int u = 0; u < PPT; u++) {
            const int r = u * NT + (int)threadIdx.x;
            pv[u] = (r < p.sel_P) ? p.sel_pool[(size_t)i * p.sel_P + r] : -1;
        }
        const int n_pool = p.sel_pool_cnt[i];
        const int B = p.sel_B;
#pragma unroll
        for (int u = 0; u < PPT; u++) s_pool[u * NT + threadIdx.x] = pv[u];
        hist_to_lds<NT>(hr, s_hist);
        const int n_cand = n_pool * B;
        // The selection's size is known from the histogram (bin 0 holds the
        // positions past t), so the window codes, and the padding past the
        // list when it ends with a window key, are written now, off the
        // selection's critical path.
        {
            const int cnt_pre = min(p.K, n_cand - (int)s_hist[0]);
            const int ke = min(cnt_pre + win.nw, p.keys_per_split);
            for (int x = threadIdx.x; x < p.keys_per_split; x += NT) {
                if (x >= cnt_pre && x < ke) s_rows[x] = -(win.w0 + (x - cnt_pre) - p.swa_first) - 1;
                else if (x >= ke && ke > 0 && win.nw > 0) s_rows[x] = -(win.w0 + (ke - 1 - cnt_pre) - p.swa_first) - 1;
            }
        }
        mask_keys<IPT>(n_cand, k);
        const Threshold th = threshold_regs<NT, IPT>(k, n_cand, (uint32_t)p.K, s_hist, s_sm);
        const bool writer = (l == 0 && hg == 0);
        int32_t *out_tk = p.topk_out + (size_t)i * p.K;
        auto emit = [&](uint32_t slot, int c) {
            const int r = c / B;
            const int pos = s_pool[r] * B + (c - r * B);
            if ((int)slot < p.keys_per_split) s_rows[slot] = pos;
            if (writer && (int)slot < p.K) out_tk[slot] = pos;
        };
        cnt = (int)compact_regs<NT, IPT>(k, th, emit, s_sm);
        if (writer) {
            for (int o = cnt + (int)threadIdx.x; o < p.K; o += NT) out_tk[o] = -1;
            if (threadIdx.x == 0) p.topk_cnt_out[i] = cnt;
            if (p.blk_hist_clear)
                for (int b = threadIdx.x; b < kRadixBins; b += NT) p.blk_hist_clear[(size_t)i * kRadixBins + b] = 0u;
        }
    } else {
        cnt = p.topk ? p.topk_cnt[i] : 0;
    }
    const int n_keys = cnt + win.nw;
    const int k_begin = 0;
    const int k_end = min(n_keys, p.keys_per_split);

    const uint16_t *qrow = (const uint16_t *)p.q + (((size_t)l * p.n_q + i) * p.H + hg * 16 + r16) * 128;
    const uint16_t *kmain = (const uint16_t *)p.k_main + (size_t)s * p.T * 128;
    const uint16_t *vmain = (const uint16_t *)p.v_main + (size_t)s * p.T * 128;
    const uint16_t *kswa = (const uint16_t *)p.k_swa + ((size_t)l * p.n_seq + s) * p.swa_len * 128;
    const uint16_t *vswa = (const uint16_t *)p.v_swa + ((size_t)l * p.n_seq + s) * p.swa_len * 128;
    const int32_t *tk = p.topk ? p.topk + (size_t)i * p.K : nullptr;

    // Row code of key kk: main row r -> r, window row r -> -(r + 1).  Slots
    // past the last key repeat the last key (read, then masked).  Only the
    // slots the chunk's steps read are staged, and every Top-K id load is
    // issued (from a clamped entry) before any is used, so the loads overlap
    // instead of each waiting under its own branch.
    auto stage_rows = [&](int kc) {
        constexpr int SPT = kRowChunk / (kWaves * 64);
        const int n_stage = min(kRowChunk, (k_end - kc + STEP - 1) / STEP * STEP);
        int id[SPT];
#pragma unroll
        for (int u = 0; u < SPT; u++) {
            const int kk = min(kc + u * kWaves * 64 + (int)threadIdx.x, k_end - 1);
            id[u] = (tk && p.K > 0) ? tk[min(kk, p.K - 1)] : 0;
        }
#pragma unroll
        for (int u = 0; u < SPT; u++) {
            const int x = u * kWaves * 64 + (int)threadIdx.x;
            const int kk = min(kc + x, k_end - 1);
            if (x < n_stage) s_rows[x] = (kk < cnt) ? id[u] : -(win.w0 + (kk - cnt) - p.swa_first) - 1;
        }
        lds_barrier();
    };
    auto row_ptr = [&](int code, const uint16_t *mbase, const uint16_t *wbase) -> const uint16_t * {
        return code >= 0 ? mbase + (size_t)code * 128 : wbase + (size_t)(-code - 1) * 128;
    };

    bf16x8_t qb[4];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) qb[kk] = *reinterpret_cast<const bf16x8_t *>(qrow + kk * 32 + g * 8);

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t acc[8];
#pragma unroll
    for (int m = 0; m < 8; m++) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint16_t *vt = s_vt[w];

    // K operand rows (keys kw + r16 and, with two tiles, kw + 16 + r16) and
    // this lane's V slots (dims r16*8 .. r16*8+7) of one step, all issued
    // back to back.  With one tile the V slots of the absent second tile are
    // zero, so its columns of V^T are zero (and its P terms are zero too).
    auto load_kv = [&](int kb, bf16x8_t (&ka)[2][4], uint4 (&vv)[8]) {
        const int *rows = s_rows + ((kb - k_begin + w * KPW) % kRowChunk);
#pragma unroll
        for (int tau = 0; tau < NTAU; tau++) {
            const uint16_t *kr = row_ptr(rows[16 * tau + r16], kmain, kswa);
#pragma unroll
            for (int kk = 0; kk < 4; kk++) ka[tau][kk] = *reinterpret_cast<const bf16x8_t *>(kr + kk * 32 + g * 8);
        }
#pragma unroll
        for (int e = 0; e < 4 * NTAU; e++)
            vv[e] = *reinterpret_cast<const uint4 *>(row_ptr(rows[slot_key(g, e)], vmain, vswa) + r16 * 8);
#pragma unroll
        for (int e = 4 * NTAU; e < 8; e++) vv[e] = make_uint4(0u, 0u, 0u, 0u);
        __builtin_amdgcn_sched_barrier(0);
    };

    // One step on the registers loaded for it; `next` runs once K and V have
    // left the registers (after QK and the V^T write) and issues the following
    // step's loads into the same registers, overlapping softmax and PV.
    auto compute = [&](int kb, bf16x8_t (&ka)[2][4], uint4 (&vv)[8], auto &&next) {
        const int kw = kb + w * KPW;
        // S^T = K Q^T: lane holds keys 4g+ii (tile 0) and 16+4g+ii (tile 1) of head r16
        f32x4_t st[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int tau = 0; tau < NTAU; tau++) {
#pragma unroll
            for (int kk = 0; kk < 4; kk++)
                st[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tau][kk], qb[kk], st[tau], 0, 0, 0);
        }
        // V^T into LDS: row = dim, 4 consecutive keys per 8-byte write
#pragma unroll
        for (int j = 0; j < 8; j++) {
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const uint32_t dw = (&vv[e].x)[j >> 1];
                h[e] = (j & 1) ? (dw >> 16) : (dw & 0xffffu);
            }
            uint16_t *row = vt + (r16 * 8 + j) * kVtStride;
            *reinterpret_cast<uint2 *>(row + 4 * g) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            *reinterpret_cast<uint2 *>(row + 16 + 4 * g) = make_uint2(h[4] | (h[5] << 16), h[6] | (h[7] << 16));
        }
        next();
        // online softmax over this step's 32 keys (log2 domain)
        float sc[8];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int key = kw + slot_key(g, e);
            sc[e] = (e < 4 * NTAU && key < k_end) ? st[e >> 2][e & 3] * p.scale_log2 : -INFINITY;
            mx = fmaxf(mx, sc[e]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float pr[8], rs = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            pr[e] = exp2f(sc[e] - m_use);
            rs += pr[e];
        }
        rs += __shfl_xor(rs, 16, 64);
        rs += __shfl_xor(rs, 32, 64);
        l_run = l_run * alpha + rs;
        m_run = m_new;
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; e++) pb[e] = __builtin_bit_cast(__bf16, f32_to_bf16(pr[e]));
#pragma unroll
        for (int m = 0; m < 8; m++) acc[m] *= alpha;
        lds_barrier();
        // O^T += V^T P^T over the 8 dim tiles
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const uint16_t *row = vt + (16 * m + r16) * kVtStride;
            const uint2 a0 = *reinterpret_cast<const uint2 *>(row + 4 * g);
            const uint2 a1 = *reinterpret_cast<const uint2 *>(row + 16 + 4 * g);
            const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), pb, acc[m], 0, 0, 0);
        }
        lds_barrier();
    };

    // Software pipeline: the loads of step s+1 are issued into the registers
    // that step s has just consumed.  Row codes are staged per kRowChunk keys;
    // a chunk boundary stages before the loads that need it (the barrier in
    // stage_rows orders it after every wave's earlier reads of s_rows).
    bf16x8_t ka[2][4];
    uint4 vv[8];
    if (k_begin < k_end) {
        if constexpr (FUSED) {
            // main slots were written by the selection, window slots and (if
            // the list ends with a window key) the padding before it; without
            // a window, repeat the last selected key in the slots past the end
            lds_barrier();
            if (win.nw == 0) {
                const int last = s_rows[k_end - 1 - k_begin];
                for (int x = k_end - k_begin + (int)threadIdx.x; x < p.keys_per_split; x += NT) s_rows[x] = last;
                lds_barrier();
            }
        } else {
            stage_rows(k_begin);
        }
        load_kv(k_begin, ka, vv);
        for (int kb = k_begin; kb < k_end; kb += STEP) {
            const int kn = kb + STEP;
            const bool more = kn < k_end;
            const bool restage = more && ((kn - k_begin) % kRowChunk == 0);
            compute(kb, ka, vv, [&] {
                if (more && !restage) load_kv(kn, ka, vv);
            });
            if (restage) {
                stage_rows(kn);
                load_kv(kn, ka, vv);
            }
        }
    }

    // ---- merge the waves (every wave has finished with its V^T buffer: the
    // key loop ends with a workgroup barrier)
    float *ob = reinterpret_cast<float *>(&s_vt[w][0]);   // this wave's [16][kObStride]
#pragma unroll
    for (int m = 0; m < 8; m++)
        *reinterpret_cast<float4 *>(ob + r16 * kObStride + 16 * m + 4 * g) =
            make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
    if (g == 0) {
        s_ml[w][r16][0] = m_run;
        s_ml[w][r16][1] = l_run;
    }
    lds_barrier();
    // thread -> (head hh, dims d0 .. d0+3)
    const int hh = threadIdx.x >> 5, d0 = (threadIdx.x & 31) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ww++) M = fmaxf(M, s_ml[ww][hh][0]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < kWaves; ww++) {
        const float f = exp2f(s_ml[ww][hh][0] - Mu);
        L += f * s_ml[ww][hh][1];
        const float4 v = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(&s_vt[ww][0]) + hh * kObStride + d0);
        o[0] += f * v.x; o[1] += f * v.y; o[2] += f * v.z; o[3] += f * v.w;
    }
    const size_t row_id = ((size_t)l * p.n_q + i) * p.H + hg * 16 + hh;
    const float inv = 1.f / L;
    const uint32_t lo = (uint32_t)f32_to_bf16(o[0] * inv) | ((uint32_t)f32_to_bf16(o[1] * inv) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(o[2] * inv) | ((uint32_t)f32_to_bf16(o[3] * inv) << 16);
    *reinterpret_cast<uint2 *>((uint16_t *)p.out + row_id * 128 + d0) = make_uint2(lo, hi);
    if (p.lse && (threadIdx.x & 31) == 0) p.lse[row_id] = (M + log2f(L)) * kLn2;
}

// Merge of the chunk records of one (query, layer, head group): one
// workgroup per pair of heads, thread -> (head, 4 dims), so that the records
// (16 heads x 132 floats each) are read by many CUs at once; every record's
// loads of a batch are issued before use.  Workgroups are numbered
// query-fastest over the query count padded to 8, as in k_attend_chunks, so
// a query's records are read on the XCD that wrote them.
constexpr int kCombineHeads = 2;   // heads per combine workgroup
// (the body takes its workgroup index and its thread index 0 .. 63)
__device__ __forceinline__ void combine_body(const AttendParams &p, int bid, int tid)
{
    const int HG = p.H / 16;
    const int i = bid % p.n_q_pad;
    const int rest = bid / p.n_q_pad;
    const int hq = rest % (16 / kCombineHeads);
    const int hg = (rest / (16 / kCombineHeads)) % HG, l = (rest / (16 / kCombineHeads)) / HG;
    if (i >= p.n_q) return;
    const int hh = hq * kCombineHeads + (tid >> 5), d0 = (tid & 31) * 4;
    const size_t rec0 = (((size_t)l * p.n_q + i) * HG + hg) * p.n_splits;
    float M = -INFINITY, L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < p.n_splits; c0 += kMergeBatch) {
        float mc[kMergeBatch], lc[kMergeBatch];
        float4 a[kMergeBatch];
        // The loads of all records of the batch must be in flight together
        // (one round trip).  In this form the compiler issues all of them
        // before the first wait (checked in the generated assembly); an
        // earlier build of the same loop waited for each record before
        // loading the next, which cost ~1.5 us per merge launch (6.0 against
        // 4.2 us).  Unconditional clamped loads with selects compiled to 20
        // more VGPRs and a 0.6 us slower step.
#pragma unroll
        for (int u = 0; u < kMergeBatch; u++) {
            if (c0 + u < p.n_splits) {
                const float *r = p.ws_part + (rec0 + c0 + u) * kPartFloats + hh * kHeadRec;
                mc[u] = r[0];
                lc[u] = r[1];
                a[u] = *reinterpret_cast<const float4 *>(r + 4 + d0);
            } else {
                mc[u] = -INFINITY;
                lc[u] = 0.f;
                a[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < kMergeBatch; u++) Mn = fmaxf(Mn, mc[u]);
        const float Mu = (Mn == -INFINITY) ? 0.f : Mn;
        const float rescale = exp2f(M - Mu);
        L *= rescale;
        o[0] *= rescale; o[1] *= rescale; o[2] *= rescale; o[3] *= rescale;
#pragma unroll
        for (int u = 0; u < kMergeBatch; u++) {
            const float f = exp2f(mc[u] - Mu);
            L += f * lc[u];
            o[0] += f * a[u].x; o[1] += f * a[u].y; o[2] += f * a[u].z; o[3] += f * a[u].w;
        }
        M = Mn;
    }
    const size_t row_id = ((size_t)l * p.n_q + i) * p.H + hg * 16 + hh;
    const float inv = 1.f / L;
    const uint32_t lo = (uint32_t)f32_to_bf16(o[0] * inv) | ((uint32_t)f32_to_bf16(o[1] * inv) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(o[2] * inv) | ((uint32_t)f32_to_bf16(o[3] * inv) << 16);
    *reinterpret_cast<uint2 *>((uint16_t *)p.out + row_id * 128 + d0) = make_uint2(lo, hi);
    if (p.lse && (tid & 31) == 0) p.lse[row_id] = (M + log2f(L)) * kLn2;
}

__global__ __launch_bounds__(32 * kCombineHeads) void k_attend_combine(AttendParams p)
{
    combine_body(p, (int)blockIdx.x, (int)threadIdx.x);
}

// ============================================================ row kernel
// Many (query, layer, head group) items, as in prefill: one wave owns an item
// and walks its whole key list, 32 keys per step, so no two waves share a
// softmax and no workgroup barrier is needed.
//  * Gather: a step's 32 K rows and 32 V rows go from L2 straight into the
//    wave's LDS tiles (buffer loads with the LDS destination), 16 lanes per
//    256-byte row, so every load instruction reads four whole rows.  The
//    MFMA operands are then read from LDS: K with 16-byte reads in the A
//    layout (key = lane % 16), V^T with the transposing 8-byte read, which
//    hands each lane one dim of four keys.  (Loading K rows straight into the
//    A layout puts 16 different rows on consecutive lanes, which halves the
//    gather rate.)
//  * Phases: the key list is walked as the Top-K rows (row ids staged in
//    LDS) and then the window (contiguous rows), so a step reads one table.
//  * Lazy running max: m moves only when a score exceeds it by more than
//    kLazyLog2 (so P <= 2^kLazyLog2 and every term stays finite); the
//    softmax is invariant to m, so the result is the same function, and a
//    step whose scores all stay under the bound needs no cross-lane
//    reduction and no rescale of the accumulators.  The row sum is kept per
//    lane and reduced across the four lane groups once per item.
// Tile layout: tile row r (0..31) of a step sits at byte
// inst * (r % 8) + 256 * (r / 8): load instruction x writes rows x, x+8,
// x+16, x+24 as one 1 KiB run, and the runs are `inst` bytes apart.  The LDS
// serves 64 banks of 4 bytes per clock, so 256 bytes apart is the same bank:
//  * V^T reads take 32 bytes of 8 rows (runs 0..7) at once: runs 32 bytes
//    apart (kRowVInst) put those rows on disjoint banks;
//  * K reads (A layout) take 16 bytes of 16 rows at once, rows r and r + 8
//    from one run: runs 16 bytes apart (kRowKInst) spread rows 0..7 over 32
//    banks, and the rows of odd slots (r / 8 odd) are stored rotated by
//    128 bytes (chunk c of the row at position (c + 8) % 16 of its slot), so
//    rows 8..15 take the other 32.  The load of such a row simply fetches its
//    chunks in that order.
constexpr int kRowKInst = 1024 + 16;
constexpr int kRowVInst = 1024 + 32;
constexpr int kRowTileBytes = 8 * kRowVInst;
constexpr int kRowWaves = 4;            // waves (items in flight) per workgroup
constexpr int kRowCodes = 512;          // Top-K row ids staged per wave at once (16 steps)
constexpr int kRowItemsPerWave = 4;     // items a wave walks in a one-round call
constexpr int kRowBlockItems = 2;        // items a wave walks in a larger call (blocks in rounds)
constexpr int kTileInst = 1024 + 16;    // bytes per load instruction in a tile
constexpr int kTileBytes = 8 * kTileInst;
constexpr float kLazyLog2 = 8.f;
constexpr int kRowPrefetchLoads = 6;    // last vector loads of the next item's prefetch (2 table + 4 query)

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int v4i32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float max_groups(float x)   // max over lanes l, l^16, l^32, l^48
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_groups(float x)   // sum over lanes l, l^16, l^32, l^48
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t *base, long long n_rows)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0, (int)(n_rows * 256), kRsrcWord3);
}

__global__ __launch_bounds__(kRowWaves * 64) void k_attend_rows(AttendParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_tiles[kRowWaves][2][kRowTileBytes];   // K, V
    __shared__ __attribute__((aligned(16))) int s_codes[kRowWaves][kRowCodes];

    // the wave index is uniform over the wave: keep it (and the item, its
    // pointers and buffer descriptors) in scalar registers
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
    // Each wave walks a few items, wave0, wave0 + stride, ...  Workgroup b
    // runs on XCD b % 8 (round-robin dispatch).
    //  * Calls that fit one round of the grid (the chip's workgroups, each
    //    wave taking up to kRowItemsPerWave items): wave v = 4 b + w takes
    //    items v, v + n_waves, ..., so every wave sees the whole range of
    //    prefix lengths, and the short early prefixes of a prompt are dealt
    //    to every XCD in turn rather than all to the first (whose waves
    //    would then finish early while the others still run).
    //  * Larger calls: workgroup b takes a block of kRowWaves * kRowBlockItems
    //    consecutive items (wave w its items w, w + kRowWaves, ...), the
    //    blocks of an XCD contiguous so that neighbouring queries, whose
    //    windows overlap, share one L2, and the blocks run in rounds that
    //    the hardware dispatch balances over the CUs.
    const int per_xcd = gridDim.x / 8;
    const int slot = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const int n_waves = gridDim.x * kRowWaves;
    const int wave0 = p.row_blocks ? slot * kRowWaves * kRowBlockItems + w : (int)blockIdx.x * kRowWaves + w;
    const int stride = p.row_blocks ? kRowWaves : n_waves;
    const int HG = p.H / 16;
    const int n_items = p.n_q * p.n_layers * HG;
    if (wave0 >= n_items) return;   // whole wave; no barriers follow
    const int item_end = p.row_blocks ? min(n_items, (slot + 1) * kRowWaves * kRowBlockItems) : n_items;

    int *codes = s_codes[w];
    uint8_t *ktile = s_tiles[w][0], *vtile = s_tiles[w][1];

    struct Item {
        int i, hg, l, s, cnt, main_steps, n_steps, wrow0, nw;
    };
    // item index -> (query, head group, layer); the query's sequence,
    // position and Top-K count come from the tables
    auto item_from = [&](int item, int s, int t, int cnt) {
        Item it;
        it.i = item % p.n_q;
        it.hg = (item / p.n_q) % HG;
        it.l = item / (p.n_q * HG);
        it.s = s;
        const Window win = window_of(t, p.W, p.swa_first, p.swa_len);
        it.cnt = cnt;
        it.main_steps = (it.cnt + 31) / 32;
        it.n_steps = it.main_steps + (win.nw + 31) / 32;
        it.wrow0 = win.w0 - p.swa_first;
        it.nw = win.nw;
        return it;
    };
    auto load_q = [&](int item, bf16x8_t (&qb)[4]) {
        const int i = item % p.n_q, hg = (item / p.n_q) % HG, l = item / (p.n_q * HG);
        const uint16_t *qrow = (const uint16_t *)p.q + (((size_t)l * p.n_q + i) * p.H + hg * 16 + r16) * 128;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) qb[kk] = load_nt_bf16x8(qrow + kk * 32 + g * 8);
    };
    // Top-K row ids kc .. kc + kRowCodes - 1 into the list (a synchronous
    // round trip); slots past cnt repeat the last id
    auto stage = [&](const Item &it, int k0) {
        const int32_t *tk = p.topk + (size_t)it.i * p.K;
        wave_lds_order();
        for (int x = lane; x < kRowCodes; x += 64) codes[x] = tk[min(k0 + x, it.cnt - 1)];
        wave_lds_order();
    };
    // the next item's first kRowCodes ids, 8 per lane, as two 16-byte loads
    // (ids past K read as zero; those past cnt are masked keys)
    const bool pf_ids = p.topk != nullptr && p.K % 4 == 0;
    auto load_ids = [&](int i, v4i32 (&cn)[2]) {
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t *>(p.topk + (size_t)i * p.K), 0,
                                                          4 * min(p.K, kRowCodes), kRsrcWord3);
        cn[0] = __builtin_bit_cast(v4i32, __builtin_amdgcn_raw_buffer_load_b128(rs, 32 * lane, 0, 0));
        cn[1] = __builtin_bit_cast(v4i32, __builtin_amdgcn_raw_buffer_load_b128(rs, 32 * lane + 16, 0, 0));
    };
    auto put_ids = [&](const v4i32 (&cn)[2]) {
        wave_lds_order();
        *reinterpret_cast<v4i32 *>(codes + 8 * lane) = cn[0];
        *reinterpret_cast<v4i32 *>(codes + 8 * lane + 4) = cn[1];
        wave_lds_order();
    };
    // The 16 loads of step st of item it (list position kc staged): load x
    // brings tile rows x + 8a (a = lane / 16) of K and of V, lane % 16 taking
    // 16 bytes of the row.
    auto issue_loads = [&](const Item &it, int st, int &kc) {
        int row[8];
        __amdgpu_buffer_rsrc_t rk, rv;
        if (st < it.main_steps) {
            if (32 * st - kc == kRowCodes) {
                kc = 32 * st;
                stage(it, kc);
            }
            const int4 c0 = *reinterpret_cast<const int4 *>(codes + 32 * st - kc + 8 * g);
            const int4 c1 = *reinterpret_cast<const int4 *>(codes + 32 * st - kc + 8 * g + 4);
            row[0] = c0.x; row[1] = c0.y; row[2] = c0.z; row[3] = c0.w;
            row[4] = c1.x; row[5] = c1.y; row[6] = c1.z; row[7] = c1.w;
            const size_t main0 = (size_t)it.s * p.T * 128;
            rk = rows_rsrc((const uint16_t *)p.k_main + main0, p.T);
            rv = rows_rsrc((const uint16_t *)p.v_main + main0, p.T);
        } else {
            const int r0 = it.wrow0 + 32 * (st - it.main_steps) + 8 * g, r_last = it.wrow0 + it.nw - 1;
#pragma unroll
            for (int x = 0; x < 8; x++) row[x] = min(r0 + x, r_last);
            const size_t swa0 = ((size_t)it.l * p.n_seq + it.s) * p.swa_len * 128;
            rk = rows_rsrc((const uint16_t *)p.k_swa + swa0, p.swa_len);
            rv = rows_rsrc((const uint16_t *)p.v_swa + swa0, p.swa_len);
        }
        // lane group g fills slot g of each run: K chunks rotated in odd slots
        const uint32_t koff = (uint32_t)(((r16 + 8 * (g & 1)) & 15) * 16), voff = (uint32_t)r16 * 16u;
#pragma unroll
        for (int x = 0; x < 8; x++) {
            const uint32_t off = (uint32_t)row[x] * 256u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(ktile + kRowKInst * x), 16, off + koff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(vtile + kRowVInst * x), 16, off + voff, 0, 0, 0);
        }
    };

    // operand addresses in the tiles (per lane; tau, m, h are immediates)
    //   K, A layout: tile row 16 tau + r16, row chunk 4 kk + g, which a row
    //   of an odd slot (r16 >= 8) holds 8 chunks further on
    const int krot = 8 * (r16 >> 3);
    const uint8_t *ka_row = ktile + kRowKInst * (r16 & 7) + 256 * (r16 >> 3);
    const uint8_t *ka_at[4];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) ka_at[kk] = ka_row + 16 * ((4 * kk + g + krot) & 15);
    //   V^T via the transposing read: lane r16 of group g addresses tile row
    //   16 h + 4 g + r16 / 4, dims 16 m + 4 (r16 % 4) .. +3
    const int vrow = 4 * g + (r16 >> 2);
    const uint8_t *va_base = vtile + kRowVInst * (vrow & 7) + 256 * (vrow >> 3) + 8 * (r16 & 3);

    // Items one after another.  While an item runs, the next item's table
    // entries, ids and query rows are loaded (issued right after the loads of
    // the item's second step, the query rows last, so that step waits for
    // everything but them), and its first step's rows are requested once the
    // item's last step has read its operands: only the first item of a wave
    // waits for its ids, query rows and first rows in turn.
    auto fence = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    Item cur;
    {
        const int i0 = wave0 % p.n_q;
        cur = item_from(wave0, p.q_seq[i0], p.q_pos[i0], p.topk ? p.topk_cnt[i0] : 0);
    }
    bf16x8_t qb[4];
    load_q(wave0, qb);
    int kc = 0;
    if (cur.main_steps > 0) stage(cur, 0);
    if (cur.n_steps > 0) issue_loads(cur, 0, kc);
    for (int item = wave0;;) {
        const int next_item = item + stride;
        const bool has_next = next_item < item_end;
        const int nx_i = next_item % p.n_q;
        const bool pf = has_next && pf_ids;   // the next item's ids come from the prefetch
        v4i32 cn[2] = {v4i32{0, 0, 0, 0}, v4i32{0, 0, 0, 0}};
        bf16x8_t qn[4] = {qb[0], qb[1], qb[2], qb[3]};
        int nx_s = 0, nx_t = 0, nx_c = 0;
        Item nxt = cur;
        bool next_issued = false;
        auto prefetch = [&]() {
            if (!has_next) return;
            fence();
            if (pf) load_ids(nx_i, cn);
            if (p.topk) nx_c = p.topk_cnt[nx_i];
            fence();
            // exactly kRowPrefetchLoads vector loads, issued last
            nx_s = p.q_seq[nx_i];
            nx_t = p.q_pos[nx_i];
            load_q(next_item, qn);
            fence();
        };
        // the next item's first rows, once this item's ids are no longer read
        auto start_next = [&]() {
            if (!has_next) return;
            nxt = item_from(next_item, __builtin_amdgcn_readfirstlane(nx_s), __builtin_amdgcn_readfirstlane(nx_t),
                            __builtin_amdgcn_readfirstlane(nx_c));
            int kc_next = 0;
            if (nxt.main_steps > 0) {
                if (pf) put_ids(cn);
                else stage(nxt, 0);
            }
            if (nxt.n_steps > 0) issue_loads(nxt, 0, kc_next);
            next_issued = true;
        };
        // the first wait after the prefetch leaves its loads in flight
        const int pf_step = (cur.n_steps < 2) ? 0 : 1;

        float m_run = -INFINITY, l_part = 0.f;
        f32x4_t acc[8];
#pragma unroll
        for (int m = 0; m < 8; m++) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (cur.n_steps < 2) prefetch();
        for (int st = 0; st < cur.n_steps; st++) {
            const int n_valid = (st < cur.main_steps) ? min(32, cur.cnt - 32 * st)
                                                      : min(32, cur.nw - 32 * (st - cur.main_steps));
            // this step's rows are in the tiles once the wave's loads are
            // done; at step 1 the prefetch issued after them may still run
            if (st == pf_step && has_next) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kRowPrefetchLoads) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            bf16x8_t ka[2][4], va[8];
#pragma unroll
            for (int tau = 0; tau < 2; tau++)
#pragma unroll
                for (int kk = 0; kk < 4; kk++)
                    ka[tau][kk] = *reinterpret_cast<const bf16x8_t *>(ka_at[kk] + 512 * tau);
#pragma unroll
            for (int m = 0; m < 8; m++) {
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(va_base + 32 * m));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(va_base + 512 + 32 * m));
                const uint4 u = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                           __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y);
                va[m] = __builtin_bit_cast(bf16x8_t, u);
            }
            // the tiles are free once these reads have returned: the next
            // step's rows (or the next item's first) are fetched during this
            // step's arithmetic
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (st + 1 < cur.n_steps) {
                issue_loads(cur, st + 1, kc);
                if (st == 0) prefetch();
            } else {
                start_next();
            }

            // S^T = K Q^T: lane holds keys 4g+ii (tile 0) and 16+4g+ii (tile 1) of head r16
            f32x4_t sk[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kk = 0; kk < 4; kk++)
#pragma unroll
                for (int tau = 0; tau < 2; tau++)
                    sk[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tau][kk], qb[kk], sk[tau], 0, 0, 0);
            // softmax terms of this step (log2 domain; the scale is positive, so
            // the maximum of the raw scores gives the maximum logit)
            float sc[8];
#pragma unroll
            for (int e = 0; e < 8; e++) sc[e] = sk[e >> 2][e & 3];
            if (n_valid < 32) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    if (slot_key(g, e) >= n_valid) sc[e] = -INFINITY;
            }
            const float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                                   fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7]))) * p.scale_log2;
            if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyLog2)) {
                const float hmax = max_groups(mx);
                const float m_new = (hmax > m_run + kLazyLog2) ? hmax : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first finite max
                l_part *= alpha;
#pragma unroll
                for (int m = 0; m < 8; m++) acc[m] *= alpha;
                m_run = m_new;
            }
            const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
            bf16x8_t pb;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float pr = __builtin_amdgcn_exp2f(fmaf(sc[e], p.scale_log2, -m_use));
                l_part += pr;
                pb[e] = (__bf16)pr;
            }
            // O^T += V^T P^T over the 8 dim tiles
#pragma unroll
            for (int m = 0; m < 8; m++) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[m], pb, acc[m], 0, 0, 0);
        }
        if (!next_issued) start_next();

        // acc[m][ii] = O[head r16][dim 16m + 4g + ii] (unnormalised)
        const float L = sum_groups(l_part);
        const float inv = 1.f / L;
        // nontemporal stores: the output is written once, and keeping it out
        // of L2 leaves room for the K/V rows other waves gather
        const size_t row_id = ((size_t)cur.l * p.n_q + cur.i) * p.H + cur.hg * 16 + r16;
        uint16_t *orow = (uint16_t *)p.out + row_id * 128;
        // Lanes of groups g and g ^ 1 swap halves (v_permlane16_swap swaps the
        // odd 16-lane rows of its first operand with the even rows of its
        // second), so that each lane holds 8 consecutive dims, of dim tile 2j
        // (even g) or 2j + 1 (odd g), and each store writes 64 contiguous
        // bytes of every row.
#pragma unroll
        for (int j = 0; j < 4; j++) {
            uint32_t lo[2], hi[2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int m = 2 * j + h;
                lo[h] = (uint32_t)f32_to_bf16(acc[m][0] * inv) | ((uint32_t)f32_to_bf16(acc[m][1] * inv) << 16);
                hi[h] = (uint32_t)f32_to_bf16(acc[m][2] * inv) | ((uint32_t)f32_to_bf16(acc[m][3] * inv) << 16);
            }
            const auto sl = __builtin_amdgcn_permlane16_swap(lo[0], lo[1], false, false);
            const auto sh = __builtin_amdgcn_permlane16_swap(hi[0], hi[1], false, false);
            const int dim0 = 16 * (2 * j + (g & 1)) + 4 * (g & ~1);
            __builtin_nontemporal_store(i32x4_nt{(int)sl[0], (int)sh[0], (int)sl[1], (int)sh[1]},
                                        reinterpret_cast<i32x4_nt *>(orow + dim0));
        }
        if (p.lse && g == 0) p.lse[row_id] = (m_run + log2f(L)) * kLn2;

        if (!has_next) break;
        item = next_item;
        cur = nxt;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) qb[kk] = qn[kk];
        kc = 0;
    }
}

// ============================================================ chunk kernel
// Few (query, layer, head group) items, as in decode: the key lists are cut
// into chunks of kCkKeys keys taken by different workgroups, so the gather is
// spread over the chip (a CU keeps only a few tens of KB of loads in flight,
// so what one workgroup gathers sets its time).  A chunk of the main (Top-K)
// list serves every layer of the group: its workgroup brings the chunk's K and
// V rows into LDS once, and each wave runs one (layer, head group) item over
// them, with the row kernel's operand reads (K in the A layout, V^T by the
// transposing read).  Window chunks belong to one layer.  Each (item, chunk)
// writes a (max, sum, acc) record; k_attend_combine merges an item's records.
// FUSED (layer-group decode): the main-chunk workgroups first take the token
// Top-K from the token keys and histogram, and each writes its own slots of
// topk (chunk 0 also the count); window-chunk workgroups need no selection and
// start at once.
// Workgroups: main chunks (query fastest, the query count padded to 8, so the
// chunks of a query, which load the same token keys, share one XCD), then
// window chunks.
constexpr int kCkWaves = 16;
constexpr int kCkTiles = 2;                   // 32-key tiles per chunk
constexpr int kCkKeys = 32 * kCkTiles;        // keys per chunk
static_assert(kCkKeys * 16 == kCkWaves * 64, "one 16-byte K piece and one V piece per thread");

// (the body takes its workgroup index)
template <bool FUSED>
__device__ __forceinline__ void attend_chunks_body(const AttendParams &p, int bid)
{
    constexpr int NT = kCkWaves * 64, IPT = kLdsKeys / NT;
    __shared__ __attribute__((aligned(16))) uint8_t s_tiles[kCkTiles][2][kTileBytes];   // K, V
    __shared__ int s_rows[kCkKeys];
    __shared__ __attribute__((aligned(16))) uint32_t s_hist[FUSED ? kHist2Words : 4];
    __shared__ int32_t s_pool[FUSED ? kFusedPoolLds : 4];
    static_assert(!FUSED || kFusedPoolLds % NT == 0, "whole pool loads per thread");
    __shared__ uint32_t s_sm[NT / 64 + 4];

    const int HG = p.H / 16;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
    const int n_main_wg = p.n_q_pad * p.n_mc;
    const bool is_main = bid < n_main_wg;
    int i, c, lw = 0;
    if (is_main) {
        i = bid % p.n_q_pad;
        c = bid / p.n_q_pad;
    } else {
        const int b = bid - n_main_wg;
        i = b % p.n_q_pad;
        c = (b / p.n_q_pad) % p.n_wc;
        lw = (b / p.n_q_pad) / p.n_wc;
    }
    if (i >= p.n_q) return;   // whole workgroup
    const int s = p.q_seq[i], t = p.q_pos[i];
    const Window win = window_of(t, p.W, p.swa_first, p.swa_len);
    const int n_items = is_main ? p.n_layers * HG : HG;
    const int split = is_main ? c : p.n_mc + c;
    // item j: (layer, head group) = (j / HG, j % HG) for a main chunk, (lw, j) for a window chunk
    auto item_q = [&](int j, bf16x8_t (&qb)[4]) {
        const int l = is_main ? j / HG : lw, hg = is_main ? j % HG : j;
        const uint16_t *qrow = (const uint16_t *)p.q + (((size_t)l * p.n_q + i) * p.H + hg * 16 + r16) * 128;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) qb[kk] = *reinterpret_cast<const bf16x8_t *>(qrow + kk * 32 + g * 8);
    };
    // this wave's first item's Q is loaded before anything else waits
    bf16x8_t qb[4];
    if (w < n_items) item_q(w, qb);

    int n_valid;   // keys of this chunk
    if (is_main) {
        int cnt;
        if constexpr (FUSED) {
            HistRegs<NT> hr;
            load_hist<NT>(p.sel_hist + (size_t)i * kRadixBins, hr);
            uint32_t k[IPT];
            load_keys_global<IPT>(p.sel_keys + (size_t)i * p.sel_stride, (int)p.sel_stride, k);
            constexpr int PPT = kFusedPoolLds / NT;
            int32_t pv[PPT];
#pragma unroll
            for (int u = 0; u < PPT; u++) {
                const int r = u * NT + (int)threadIdx.x;
                pv[u] = (r < p.sel_P) ? p.sel_pool[(size_t)i * p.sel_P + r] : -1;
            }
            const int n_pool = p.sel_pool_cnt[i];
            const int B = p.sel_B;
#pragma unroll
            for (int u = 0; u < PPT; u++) s_pool[u * NT + threadIdx.x] = pv[u];
            hist_to_lds<NT>(hr, s_hist);
            const int n_cand = n_pool * B;
            mask_keys<IPT>(n_cand, k);
            const Threshold th = threshold_regs<NT, IPT>(k, n_cand, (uint32_t)p.K, s_hist, s_sm);
            // each main chunk writes its own slots of topk (and their -1
            // padding), so only this chunk's keys look up their positions
            int32_t *out_tk = p.topk_out + (size_t)i * p.K;
            const int kb0 = c * kCkKeys;
            auto emit = [&](uint32_t slot, int cc) {
                const int x = (int)slot - kb0;
                if (x >= 0 && x < kCkKeys) {
                    const int r = cc / B;
                    const int pos = s_pool[r] * B + (cc - r * B);
                    s_rows[x] = pos;
                    out_tk[slot] = pos;
                }
            };
            cnt = (int)compact_regs<NT, IPT>(k, th, emit, s_sm);
            for (int o = max(cnt, kb0) + (int)threadIdx.x; o < min(p.K, kb0 + kCkKeys); o += NT) out_tk[o] = -1;
            if (c == 0) {
                if (threadIdx.x == 0) p.topk_cnt_out[i] = cnt;
                if (p.blk_hist_clear)
                    for (int b = threadIdx.x; b < kRadixBins; b += NT) p.blk_hist_clear[(size_t)i * kRadixBins + b] = 0u;
            }
            n_valid = min(max(cnt - c * kCkKeys, 0), kCkKeys);
            lds_barrier();
        } else {
            cnt = min(p.topk_cnt[i], p.K);
            n_valid = min(max(cnt - c * kCkKeys, 0), kCkKeys);
            if (threadIdx.x < kCkKeys && n_valid > 0)
                s_rows[threadIdx.x] = p.topk[(size_t)i * p.K + c * kCkKeys + min((int)threadIdx.x, n_valid - 1)];
            lds_barrier();
        }
    } else {
        n_valid = min(max(win.nw - c * kCkKeys, 0), kCkKeys);
    }

    // ---- the chunk's K and V rows into the tiles: thread -> (slot, 16-byte
    // piece); slots past the chunk's keys repeat its last key (masked later)
    if (n_valid > 0) {
        const int slot = threadIdx.x >> 4, part = threadIdx.x & 15;
        const int sl = min(slot, n_valid - 1);
        const uint16_t *krow, *vrow;
        if (is_main) {
            const size_t r = (size_t)s * p.T + s_rows[sl];
            krow = (const uint16_t *)p.k_main + r * 128;
            vrow = (const uint16_t *)p.v_main + r * 128;
        } else {
            const size_t r = ((size_t)lw * p.n_seq + s) * p.swa_len + (win.w0 - p.swa_first) + c * kCkKeys + sl;
            krow = (const uint16_t *)p.k_swa + r * 128;
            vrow = (const uint16_t *)p.v_swa + r * 128;
        }
        const uint4 kv = *reinterpret_cast<const uint4 *>(krow + part * 8);
        const uint4 vv = *reinterpret_cast<const uint4 *>(vrow + part * 8);
        const int tau = slot >> 5, rr = slot & 31;
        const int off = kTileInst * (rr & 7) + 256 * (rr >> 3) + 16 * part;
        *reinterpret_cast<uint4 *>(&s_tiles[tau][0][off]) = kv;
        *reinterpret_cast<uint4 *>(&s_tiles[tau][1][off]) = vv;
    }
    lds_barrier();

    // ---- each wave: its items over the chunk's tiles
    //   K, A layout: tile row 16 h + r16, bytes 64 kk + 16 g
    const int ka_off = kTileInst * (r16 & 7) + 256 * (r16 >> 3) + 16 * g;
    //   V^T via the transposing read: lane r16 of group g addresses tile row
    //   16 h + 4 g + r16 / 4, dims 16 m + 4 (r16 % 4) .. +3
    const int vr = 4 * g + (r16 >> 2);
    const int va_off = kTileInst * (vr & 7) + 256 * (vr >> 3) + 8 * (r16 & 3);
    for (int j = w; j < n_items; j += kCkWaves) {
        if (j != w) item_q(j, qb);
        const int l = is_main ? j / HG : lw, hg = is_main ? j % HG : j;
        float m_run = -INFINITY, l_part = 0.f;
        f32x4_t acc[8];
#pragma unroll
        for (int m = 0; m < 8; m++) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tau = 0; tau < kCkTiles; tau++) {
            const int nv = n_valid - 32 * tau;   // keys in this tile (uniform)
            if (nv <= 0) break;
            const uint8_t *kt = s_tiles[tau][0], *vt = s_tiles[tau][1];
            bf16x8_t ka[2][4];
#pragma unroll
            for (int h = 0; h < 2; h++)
#pragma unroll
                for (int kk = 0; kk < 4; kk++)
                    ka[h][kk] = *reinterpret_cast<const bf16x8_t *>(kt + ka_off + 512 * h + 64 * kk);
            f32x4_t sk[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kk = 0; kk < 4; kk++)
#pragma unroll
                for (int h = 0; h < 2; h++)
                    sk[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[h][kk], qb[kk], sk[h], 0, 0, 0);
            // lane holds keys 4g+ii (tile half 0) and 16+4g+ii (half 1) of head r16
            float sc[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                sc[e] = sk[e >> 2][e & 3] * p.scale_log2;
                if (slot_key(g, e) >= nv) sc[e] = -INFINITY;
            }
            const float mx = max_groups(fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                                              fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7]))));
            const float m_new = fmaxf(m_run, mx);      // finite: the tile has a key
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first tile
            l_part *= alpha;
#pragma unroll
            for (int m = 0; m < 8; m++) acc[m] *= alpha;
            m_run = m_new;
            bf16x8_t pb;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float pr = __builtin_amdgcn_exp2f(sc[e] - m_run);
                l_part += pr;
                pb[e] = (__bf16)pr;
            }
#pragma unroll
            for (int m = 0; m < 8; m++) {
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(vt + va_off + 32 * m));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(vt + va_off + 512 + 32 * m));
                const uint4 u = make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                           __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, u), pb, acc[m], 0, 0, 0);
            }
        }
        // the record of (item, chunk): per head max and sum (log2 domain) and
        // the unnormalised acc; an empty chunk writes (-inf, 0, 0)
        const float L = sum_groups(l_part);
        const size_t rec0 = (((size_t)l * p.n_q + i) * HG + hg) * p.n_splits;
        float *rec = p.ws_part + (rec0 + split) * kPartFloats + r16 * kHeadRec;
#pragma unroll
        for (int m = 0; m < 8; m++)
            *reinterpret_cast<float4 *>(rec + 4 + 16 * m + 4 * g) = make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
        if (g == 0) {
            rec[0] = m_run;
            rec[1] = L;
        }
    }
}

template <bool FUSED>
__global__ __launch_bounds__(kCkWaves * 64) void k_attend_chunks(AttendParams p)
{
    attend_chunks_body<FUSED>(p, (int)blockIdx.x);
}

// ============================================================ window kernel
// Window-only layers with many queries (prefill): neighbouring queries share
// most of their windows, so a workgroup takes kWinQ consecutive queries and
// brings the union of their windows into LDS once; its waves then run the row
// kernel's step on one query at a time with both operands read from LDS (K in
// the A layout, V^T by the transposing read).  K rows are padded to 272 bytes
// (the 16 rows of an A-operand read start in different banks) and V rows to
// 288 bytes (the 8 rows of a transposing read pass do).
//  * Fast path: the tile's queries share a sequence and the union of their
//    windows fits kWinRows rows: one staging, each wave takes kWinQPW queries.
//  * Otherwise the tile is done as kWinQPW parts of kWinWaves queries (one per
//    wave), each walking the union of its windows in chunks of kWinRows rows,
//    one sequence at a time; a query's softmax state stays in its wave's
//    registers across chunks.
constexpr int kWinWaves = 16;
constexpr int kWinQPW = 2;               // queries per wave
constexpr int kWinQ = kWinQPW * kWinWaves;   // queries per workgroup
constexpr int kWinRows = 160;            // window rows staged at once (32 queries of a 128 window: 159)
constexpr int kWinKStride = 272;         // bytes per staged K row
constexpr int kWinVStride = 288;         // bytes per staged V row

// Copies window rows [c0, c0 + n_rows) of K and V (256 bytes each) into the
// padded LDS rows of the window kernel; every load is issued before the
// first store (and before `between`), and the stores wait for the workgroup
// to be done with the previous rows unless there are none.
template <typename Between>
__device__ __forceinline__ void win_stage(const uint8_t *ksrc, const uint8_t *vsrc, int c0, int n_rows,
                                          uint8_t *s_k, uint8_t *s_v, bool first_barrier, Between &&between)
{
    constexpr int NT = kWinWaves * 64;
    constexpr int PER = (kWinRows * 16 + NT - 1) / NT;
    const int tid = threadIdx.x;
    static_assert(PER == 3, "staging is written out for three 16-byte pieces per thread");
    auto src = [&](int u) {
        const int x = tid + u * NT;
        return (size_t)(c0 + min(x >> 4, n_rows - 1)) * 256 + 16 * (x & 15);
    };
    const uint4 k0 = *reinterpret_cast<const uint4 *>(ksrc + src(0)), v0 = *reinterpret_cast<const uint4 *>(vsrc + src(0));
    const uint4 k1 = *reinterpret_cast<const uint4 *>(ksrc + src(1)), v1 = *reinterpret_cast<const uint4 *>(vsrc + src(1));
    const uint4 k2 = *reinterpret_cast<const uint4 *>(ksrc + src(2)), v2 = *reinterpret_cast<const uint4 *>(vsrc + src(2));
    between();
    if (first_barrier) __syncthreads();
    auto put = [&](int u, uint4 kv, uint4 vv) {
        const int x = tid + u * NT;
        const int r = x >> 4, c = x & 15;
        if (r < n_rows) {
            *reinterpret_cast<uint4 *>(s_k + r * kWinKStride + 16 * c) = kv;
            *reinterpret_cast<uint4 *>(s_v + r * kWinVStride + 16 * c) = vv;
        }
    };
    put(0, k0, v0);
    put(1, k1, v1);
    put(2, k2, v2);
    __syncthreads();
}

__global__ __launch_bounds__(kWinWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void k_attend_window(AttendParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_k[kWinRows * kWinKStride];
    __shared__ __attribute__((aligned(16))) uint8_t s_v[kWinRows * kWinVStride];
    __shared__ __attribute__((aligned(16))) uint8_t s_q[kWinWaves][16 * 256];   // each wave's first query rows, then its output rows

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int HG = p.H / 16;
    const int tiles_q = (p.n_q + kWinQ - 1) / kWinQ;
    // Workgroup b runs on XCD b % 8 (round-robin dispatch); each XCD takes a
    // contiguous range of tiles, so the window rows it stages stay in its L2.
    const int per_xcd = (int)gridDim.x / 8;
    const int tile = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
    if (tile >= tiles_q * HG * p.n_layers) return;   // whole workgroup
    const int q0 = (tile % tiles_q) * kWinQ;
    const int hg = (tile / tiles_q) % HG;
    const int l = tile / (tiles_q * HG);

    // lane j < kWinQ of every wave holds query q0 + j: its sequence (-1 past
    // n_q), first window row and row count; a query's entries are read with
    // readlane, the tile's union with ballots and wave reductions
    static_assert(kWinQ <= 64, "a tile's queries are held one per lane");
    int ls = -1, lr0 = 0, lnw = 0;
    if (lane < kWinQ && q0 + lane < p.n_q) {
        const Window win = window_of(p.q_pos[q0 + lane], p.W, p.swa_first, p.swa_len);
        ls = p.q_seq[q0 + lane];
        lr0 = win.w0 - p.swa_first;
        lnw = win.nw;
    }
    const bool has_rows = ls >= 0 && lnw > 0;
    auto at = [&](int v, int j) { return __builtin_amdgcn_readlane(v, j); };
    // min of lo and max of hi over the lanes of mask
    auto span_of = [&](uint64_t mask, int &lo, int &hi) {
        const bool in = (mask >> lane) & 1;
        int a = in ? lr0 : INT32_MAX, b = in ? lr0 + lnw : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            a = min(a, __shfl_xor(a, o));
            b = max(b, __shfl_xor(b, o));
        }
        lo = __builtin_amdgcn_readfirstlane(a);
        hi = __builtin_amdgcn_readfirstlane(b);
    };
    // Stages window rows [c0, c0 + n_rows) of sequence s (all loads first).
    auto stage = [&](int s, int c0, int n_rows) {
        const size_t row0 = ((size_t)l * p.n_seq + s) * p.swa_len;
        win_stage((const uint8_t *)p.k_swa + row0 * 256, (const uint8_t *)p.v_swa + row0 * 256, c0, n_rows, s_k, s_v,
                  true, [] {});
    };
    struct State {
        bf16x8_t qb[4];
        f32x4_t acc[8];
        float m_run, l_part;
    };
    auto begin = [&](State &st, int i) {
        const uint16_t *qrow = (const uint16_t *)p.q + (((size_t)l * p.n_q + i) * p.H + hg * 16 + r16) * 128;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) st.qb[kk] = load_nt_bf16x8(qrow + kk * 32 + g * 8);
#pragma unroll
        for (int m = 0; m < 8; m++) st.acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        st.m_run = -INFINITY;
        st.l_part = 0.f;
    };
    // The keys of window rows [a, b), staged from row c0, 32 per step.
    auto attend_rows = [&](State &st, int a, int b, int c0) {
        for (int k0 = a; k0 < b; k0 += 32) {
            const int n_valid = min(32, b - k0);
            bf16x8_t ka[2][4], va[8];
#pragma unroll
            for (int tau = 0; tau < 2; tau++) {
                const int r = min(k0 + 16 * tau + r16, b - 1) - c0;
#pragma unroll
                for (int kk = 0; kk < 4; kk++)
                    ka[tau][kk] = *reinterpret_cast<const bf16x8_t *>(s_k + r * kWinKStride + 64 * kk + 16 * g);
            }
            f32x4_t sk[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kk = 0; kk < 4; kk++)
#pragma unroll
                for (int tau = 0; tau < 2; tau++)
                    sk[tau] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[tau][kk], st.qb[kk], sk[tau], 0, 0, 0);
            // V^T operands after QK, in the registers K has left
            const int rv0 = min(k0 + 4 * g + (r16 >> 2), b - 1) - c0;
            const int rv1 = min(k0 + 16 + 4 * g + (r16 >> 2), b - 1) - c0;
#pragma unroll
            for (int m = 0; m < 8; m++) {
                const v4i16 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(s_v + rv0 * kWinVStride + 32 * m + 8 * (r16 & 3)));
                const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(s_v + rv1 * kWinVStride + 32 * m + 8 * (r16 & 3)));
                const uint4 u = make_uint4(__builtin_bit_cast(uint2, lo4).x, __builtin_bit_cast(uint2, lo4).y,
                                           __builtin_bit_cast(uint2, hi4).x, __builtin_bit_cast(uint2, hi4).y);
                va[m] = __builtin_bit_cast(bf16x8_t, u);
            }
            float sc[8];
#pragma unroll
            for (int e = 0; e < 8; e++) sc[e] = sk[e >> 2][e & 3];
            if (n_valid < 32) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    if (slot_key(g, e) >= n_valid) sc[e] = -INFINITY;
            }
            const float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                                   fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7]))) * p.scale_log2;
            if (__builtin_amdgcn_ballot_w64(mx > st.m_run + kLazyLog2)) {
                const float hmax = max_groups(mx);
                const float m_new = (hmax > st.m_run + kLazyLog2) ? hmax : st.m_run;
                const float alpha = __builtin_amdgcn_exp2f(st.m_run - m_new);
                st.l_part *= alpha;
#pragma unroll
                for (int m = 0; m < 8; m++) st.acc[m] *= alpha;
                st.m_run = m_new;
            }
            const float m_use = (st.m_run == -INFINITY) ? 0.f : st.m_run;
            bf16x8_t pb;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float pr = __builtin_amdgcn_exp2f(fmaf(sc[e], p.scale_log2, -m_use));
                st.l_part += pr;
                pb[e] = (__bf16)pr;
            }
#pragma unroll
            for (int m = 0; m < 8; m++) st.acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[m], pb, st.acc[m], 0, 0, 0);
        }
    };
    // st.acc[m][ii] = O[head r16][dim 16m + 4g + ii] (unnormalised)
    auto finish = [&](State &st, int i) {
        const float L = sum_groups(st.l_part);
        const float inv = 1.f / L;
        // The item's 16 output rows are contiguous (4 KB).  They go through
        // the wave's query-row slot, which the first query's rows have left,
        // so that each store writes four whole rows (1 KB), nontemporally
        // (written once, they need no room in L2; with 32-byte pieces per
        // row, nontemporal stores were slower).
        const size_t row0 = ((size_t)l * p.n_q + i) * p.H + hg * 16;
        uint8_t *so = s_q[w];
        wave_lds_order();
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const uint32_t lo2 = (uint32_t)f32_to_bf16(st.acc[m][0] * inv) | ((uint32_t)f32_to_bf16(st.acc[m][1] * inv) << 16);
            const uint32_t hi2 = (uint32_t)f32_to_bf16(st.acc[m][2] * inv) | ((uint32_t)f32_to_bf16(st.acc[m][3] * inv) << 16);
            *reinterpret_cast<uint2 *>(so + 256 * r16 + 32 * m + 8 * g) = make_uint2(lo2, hi2);
        }
        wave_lds_order();
        uint8_t *obase = (uint8_t *)p.out + row0 * 256;
#pragma unroll
        for (int x = 0; x < 4; x++)
            __builtin_nontemporal_store(*reinterpret_cast<const i32x4_nt *>(so + 1024 * x + 16 * lane),
                                        reinterpret_cast<i32x4_nt *>(obase + 1024 * x + 16 * lane));
        if (p.lse && g == 0) p.lse[row0 + r16] = (st.m_run + log2f(L)) * kLn2;
    };

    // the fast path's condition: one sequence, and the union fits one staging
    const uint64_t with_rows = __builtin_amdgcn_ballot_w64(has_rows);
    int s0 = -1, lo = INT32_MAX, hi = 0;
    bool one_seq = true;
    if (with_rows) {
        s0 = at(ls, __builtin_ctzll(with_rows));
        one_seq = __builtin_amdgcn_ballot_w64(has_rows && ls != s0) == 0;
        span_of(with_rows, lo, hi);
    }
    if (one_seq && (s0 < 0 || hi - lo <= kWinRows)) {
        // One staging (no earlier rows to protect, so no barrier before its
        // stores).  The wave's first query rows go straight into its LDS
        // slot with buffer loads issued after the window loads, so the
        // barrier after the stores waits for both together and the rows are
        // then read from LDS.
        State st;
        const bool first = q0 + w < p.n_q;
        auto q_to_lds = [&]() {
            if (!first) return;
            const uint16_t *qrow0 = (const uint16_t *)p.q + (((size_t)l * p.n_q + q0 + w) * p.H + hg * 16) * 128;
            const auto rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(qrow0), 0, 16 * 256, kRsrcWord3);
#pragma unroll
            for (int x = 0; x < 4; x++)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (__attribute__((address_space(3))) void *)(s_q[w] + 1024 * x),
                                                         16, 1024 * x + 16 * lane, 0, 0, 0);
        };
        if (s0 >= 0) {
            const size_t row0 = ((size_t)l * p.n_seq + s0) * p.swa_len;
            win_stage((const uint8_t *)p.k_swa + row0 * 256, (const uint8_t *)p.v_swa + row0 * 256, lo, hi - lo, s_k,
                      s_v, false, q_to_lds);
        } else {
            q_to_lds();
            __syncthreads();
        }
        if (first) {
#pragma unroll
            for (int kk = 0; kk < 4; kk++)
                st.qb[kk] = *reinterpret_cast<const bf16x8_t *>(s_q[w] + 256 * r16 + 64 * kk + 16 * g);
#pragma unroll
            for (int m = 0; m < 8; m++) st.acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            st.m_run = -INFINITY;
            st.l_part = 0.f;
        }
        // a wave's queries w, w + kWinWaves, ... in turn; the next query's
        // rows are requested before this one's output stores, so waiting for
        // them does not wait for the stores
#pragma unroll
        for (int half = 0; half < kWinQPW; half++) {
            const int j = w + kWinWaves * half, i = q0 + j;
            if (i >= p.n_q) break;
            const int my_r0 = at(lr0, j), my_nw = at(lnw, j);
            if (my_nw > 0) attend_rows(st, my_r0, my_r0 + my_nw, lo);
            const bool next = half + 1 < kWinQPW && i + kWinWaves < p.n_q;
            bf16x8_t qn[4];
            if (next) {
                const uint16_t *qrow = (const uint16_t *)p.q + (((size_t)l * p.n_q + i + kWinWaves) * p.H + hg * 16 + r16) * 128;
#pragma unroll
                for (int kk = 0; kk < 4; kk++) qn[kk] = load_nt_bf16x8(qrow + kk * 32 + g * 8);
            }
            finish(st, i);
            if (next) {
#pragma unroll
                for (int kk = 0; kk < 4; kk++) st.qb[kk] = qn[kk];
#pragma unroll
                for (int m = 0; m < 8; m++) st.acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                st.m_run = -INFINITY;
                st.l_part = 0.f;
            }
        }
        return;
    }
    // general path: parts of kWinWaves queries, chunks of kWinRows rows
#pragma unroll
    for (int half = 0; half < kWinQPW; half++) {
        const int j = w + kWinWaves * half, i = q0 + j;
        const bool valid = i < p.n_q;
        const int my_r0 = at(lr0, j), my_nw = at(lnw, j);
        State st;
        if (valid) begin(st, i);
        // the part's queries with rows, as lane bits
        const uint64_t part = (kWinWaves >= 64 ? ~0ull : ((1ull << kWinWaves) - 1)) << (kWinWaves * half);
        uint64_t remaining = with_rows & part;
        // one sequence at a time; every wave takes the same groups and chunks
        while (remaining) {
            const int s = at(ls, __builtin_ctzll(remaining));
            const uint64_t gmask = __builtin_amdgcn_ballot_w64(has_rows && ls == s) & remaining;
            int glo, ghi;
            span_of(gmask, glo, ghi);
            remaining &= ~gmask;
            const bool mine = valid && ((gmask >> j) & 1);
            for (int c0 = glo; c0 < ghi; c0 += kWinRows) {
                const int n_rows = min(kWinRows, ghi - c0);
                stage(s, c0, n_rows);
                if (!mine) continue;
                const int a = max(my_r0, c0), b = min(my_r0 + my_nw, c0 + n_rows);
                if (a < b) attend_rows(st, a, b, c0);
            }
        }
        if (valid) finish(st, i);
    }
}

// ============================================================ planning / launch
static int ceil_div_i(long long a, long long b) { return (int)((a + b - 1) / b); }

AttendPlan plan_attend(int n_q, int n_layers, int H, int D, int K, int W, int dtype)
{
    AttendPlan pl{(dtype == 1) && (D == 128) && (H % 16 == 0), false, 1, 0, 0, 32, false, 0, 0};
    if (!pl.mfma) return pl;
    const long long base = (long long)n_q * n_layers * (H / 16);
    if (base < kTargetWorkgroups / 2) {
        // too few (query, layer, head group) items to spread the gather over
        // the chip: cut the key lists into chunks, one workgroup each, and
        // merge each item's chunk records
        pl.chunks = true;
        pl.n_mc = (K + kCkKeys - 1) / kCkKeys;
        pl.n_wc = (W + kCkKeys - 1) / kCkKeys;
        pl.n_splits = pl.n_mc + pl.n_wc;
        pl.part_bytes = (size_t)base * pl.n_splits * kPartFloats * sizeof(float);
        return pl;
    }
    const int steps = std::max(1, (K + W + kStepKeys - 1) / kStepKeys);
    pl.keys_per_split = steps * kStepKeys;
    // enough items for one wave each to fill the chip: the row kernel
    pl.rows = base >= kRowItemsMin;
    return pl;
}

hipError_t launch_attend(const AttendParams &p0, const AttendPlan &pl, int D, int dtype, hipStream_t st,
                         bool fused_select)
{
    if (p0.n_q <= 0 || p0.n_layers <= 0) return hipSuccess;
    AttendParams p = p0;
    const bool rows_fit = (long long)p.T * 256 < INT32_MAX && (long long)p.swa_len * 256 < INT32_MAX;
    if (pl.rows && !fused_select && p0.topk == nullptr &&
        (long long)p.n_q * p.n_layers * (p.H / 16) >= kWinItemsMin) {
        // window-only layer with many queries: shared windows in LDS
        const long long n_wg = (long long)((p.n_q + kWinQ - 1) / kWinQ) * (p.H / 16) * p.n_layers;
        launch("k_attend_window", k_attend_window, dim3((unsigned)((n_wg + 7) / 8 * 8)), dim3(kWinWaves * 64), st, p);
        return hipGetLastError();
    }
    if (pl.rows && !fused_select && rows_fit) {
        const long long items = (long long)p.n_q * p.n_layers * (p.H / 16);
        long long n_wg;
        if (items <= (long long)kRowWaves * kRowItemsPerWave * kTargetWorkgroups) {   // one round: waves stride over every item
            p.row_blocks = 0;
            n_wg = std::min<long long>((items + kRowWaves - 1) / kRowWaves, kTargetWorkgroups);
        } else {                                      // blocks of consecutive items, in rounds
            p.row_blocks = 1;
            const long long per_wg = (long long)kRowWaves * kRowBlockItems;
            n_wg = (items + per_wg - 1) / per_wg;
        }
        launch("k_attend_rows", k_attend_rows, dim3((unsigned)((n_wg + 7) / 8 * 8)), dim3(kRowWaves * 64), st, p);
        return hipGetLastError();
    }
    if (pl.chunks) {
        p.n_q_pad = (p.n_q + 7) / 8 * 8;
        p.n_mc = (fused_select || p.topk != nullptr) ? pl.n_mc : 0;
        p.n_wc = pl.n_wc;
        p.n_splits = p.n_mc + p.n_wc;
        const long long n_wg = (long long)p.n_q_pad * (p.n_mc + (long long)p.n_layers * p.n_wc);
        if (fused_select) launch("k_attend_chunks", k_attend_chunks<true>, dim3((unsigned)n_wg), dim3(kCkWaves * 64), st, p);
        else launch("k_attend_chunks", k_attend_chunks<false>, dim3((unsigned)n_wg), dim3(kCkWaves * 64), st, p);
        const long long n_rows = (long long)p.n_q_pad * (p.H / 16) * p.n_layers;
        launch("k_attend_combine", k_attend_combine, dim3((unsigned)(n_rows * (16 / kCombineHeads))), dim3(32 * kCombineHeads), st, p);
        return hipGetLastError();
    }
    if (pl.mfma) {
        p.n_q_pad = (p.n_q + 7) / 8 * 8;
        p.n_splits = 1;
        p.keys_per_split = pl.keys_per_split;
        const long long n_wg = (long long)p.n_q_pad * (p.H / 16) * p.n_layers;
        if (fused_select) launch("k_attend_mfma", k_attend_mfma<true>, dim3((unsigned)n_wg), dim3(kWaves * 64), st, p);
        else launch("k_attend_mfma", k_attend_mfma<false>, dim3((unsigned)n_wg), dim3(kWaves * 64), st, p);
        return hipGetLastError();
    }
    dim3 grid((unsigned)p.n_q, (unsigned)p.n_layers, (unsigned)ceil_div_i(p.H, 4));
    if (dtype == 0) {
        if (D == 64) launch("k_attend_generic", (k_attend_generic<float, 64>), grid, dim3(256), st, p);
        else launch("k_attend_generic", (k_attend_generic<float, 128>), grid, dim3(256), st, p);
    } else {
        if (D == 64) launch("k_attend_generic", (k_attend_generic<uint16_t, 64>), grid, dim3(256), st, p);
        else launch("k_attend_generic", (k_attend_generic<uint16_t, 128>), grid, dim3(256), st, p);
    }
    return hipGetLastError();
}

}  // namespace csa2
