// attend.hip -- sparse + sliding-window attention (gfx950).
//
// "Sparse attention" on the DeepSeek V4.1 Flash page (k-a.in): a query reads
// its Top-K main-KV entries plus a window of the most recent tokens.  Per head,
// one softmax runs over both sets together; the window K/V are the layer's own
// ("CSA2 with cross-layer reuse": every mode computes its own main Q and
// window K/V) while the main K/V and the indices may be shared by a group of
// layers.
//
// Two kernels:
//  * k_attend_mfma (bf16, D = 128, heads in groups of 16).  A wave takes 32
//    keys per step: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (keys x heads),
//    online softmax in fp32 (one head per lane column), then O^T += V^T P^T.
//    K rows go straight from HBM into MFMA operands (16 B per lane, each row
//    read once); V rows are written transposed into LDS so that the PV operand
//    is two 8-byte LDS reads per lane.  Decode splits a query's key list over
//    workgroups; partial (max, sum, acc) records are merged by the last
//    workgroup to arrive.  Workgroups of one query are numbered so that they
//    land on one XCD (round-robin dispatch), so layers that share main rows
//    re-read them from that XCD's L2.
//  * k_attend_generic (fp32 or bf16, any H, D in {64, 128}): one wave per head,
//    keys in sequence, fp32 online softmax on the vector ALU.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace csa2 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);   // keep NaN a NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

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
constexpr int kVtStride = 40;                 // bf16 per V^T row in LDS (32 keys + pad)
constexpr int kPartFloats = 16 * (2 + 128);   // one split record: 16 x (max, sum, acc[128])

// Key slot e (0..7) of lane group g inside a 32-key step: the keys whose
// scores this lane holds after the QK MFMA (rows 4g..4g+3 of tile 0 and of
// tile 1).  Both PV operands use this same order along the contraction.
__device__ __forceinline__ int slot_key(int g, int e) { return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4); }

__global__ __launch_bounds__(256) void k_attend_mfma(AttendParams p)
{
    __shared__ __attribute__((aligned(16))) uint16_t s_vt[4][128 * kVtStride];
    __shared__ float s_ml[4][16][2];
    __shared__ uint32_t s_flag;

    const int HG = p.H / 16;
    const int id = blockIdx.x;
    const int i = id % p.n_q_pad;
    int rest = id / p.n_q_pad;
    const int split = rest % p.n_splits;
    rest /= p.n_splits;
    const int hg = rest % HG;
    const int l = rest / HG;
    if (i >= p.n_q) return;

    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
    const int s = p.q_seq[i], t = p.q_pos[i];
    const int cnt = p.topk ? p.topk_cnt[i] : 0;
    const Window win = window_of(t, p.W, p.swa_first, p.swa_len);
    const int n_keys = cnt + win.nw;

    const uint16_t *qrow = (const uint16_t *)p.q + (((size_t)l * p.n_q + i) * p.H + hg * 16 + r16) * 128;
    const uint16_t *kmain = (const uint16_t *)p.k_main + (size_t)s * p.T * 128;
    const uint16_t *vmain = (const uint16_t *)p.v_main + (size_t)s * p.T * 128;
    const uint16_t *kswa = (const uint16_t *)p.k_swa + ((size_t)l * p.n_seq + s) * p.swa_len * 128;
    const uint16_t *vswa = (const uint16_t *)p.v_swa + ((size_t)l * p.n_seq + s) * p.swa_len * 128;
    const int32_t *tk = p.topk ? p.topk + (size_t)i * p.K : nullptr;

    // element offset of key kk's row and which cache it lives in; slots past
    // the last key re-read the last key's row (always valid inside the loop,
    // where n_keys >= 1) and are masked out of the softmax
    auto key_off = [&](int kk, bool &main) -> size_t {
        kk = min(kk, n_keys - 1);
        main = kk < cnt;
        if (main) return (size_t)tk[kk] * 128;
        return (size_t)(win.w0 + (kk - cnt) - p.swa_first) * 128;
    };

    bf16x8_t qb[4];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) qb[kk] = *reinterpret_cast<const bf16x8_t *>(qrow + kk * 32 + g * 8);

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t acc[8];
#pragma unroll
    for (int m = 0; m < 8; m++) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint16_t *vt = s_vt[w];
    const int k_begin = split * p.keys_per_split;
    const int k_stop = min(n_keys, k_begin + p.keys_per_split);
    for (int kb = k_begin; kb < k_stop; kb += kAttendKeysPerIter) {
        const int kw = kb + w * 32;
        // K operand rows: keys kw + r16 (tile 0) and kw + 16 + r16 (tile 1)
        bf16x8_t ka[2][4];
#pragma unroll
        for (int tau = 0; tau < 2; tau++) {
            bool main;
            const size_t off = key_off(kw + 16 * tau + r16, main);
            const uint16_t *kr = (main ? kmain : kswa) + off;
#pragma unroll
            for (int kk = 0; kk < 4; kk++) ka[tau][kk] = *reinterpret_cast<const bf16x8_t *>(kr + kk * 32 + g * 8);
        }
        // V rows of this lane's 8 key slots, dims r16*8 .. r16*8+7
        uint4 vv[8];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            bool main;
            const size_t off = key_off(kw + slot_key(g, e), main);
            vv[e] = *reinterpret_cast<const uint4 *>((main ? vmain : vswa) + off + r16 * 8);
        }
        // S^T = K Q^T: lane holds keys 4g+ii (tile 0) and 16+4g+ii (tile 1) of head r16
        f32x4_t st[2];
#pragma unroll
        for (int tau = 0; tau < 2; tau++) {
            st[tau] = f32x4_t{0.f, 0.f, 0.f, 0.f};
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
        // online softmax over this step's 32 keys (log2 domain)
        float sc[8];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int key = kw + slot_key(g, e);
            sc[e] = (key < k_stop) ? st[e >> 2][e & 3] * p.scale_log2 : -INFINITY;
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
        __syncthreads();
        // O^T += V^T P^T over the 8 dim tiles
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const uint16_t *row = vt + (16 * m + r16) * kVtStride;
            const uint2 a0 = *reinterpret_cast<const uint2 *>(row + 4 * g);
            const uint2 a1 = *reinterpret_cast<const uint2 *>(row + 16 + 4 * g);
            const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), pb, acc[m], 0, 0, 0);
        }
        __syncthreads();
    }

    // ---- merge the 4 waves (the V^T buffer is free now)
    float *ob = reinterpret_cast<float *>(&s_vt[0][0]);   // [4][16][128]
#pragma unroll
    for (int m = 0; m < 8; m++)
#pragma unroll
        for (int ii = 0; ii < 4; ii++) ob[(w * 16 + r16) * 128 + 16 * m + 4 * g + ii] = acc[m][ii];
    if (g == 0) {
        s_ml[w][r16][0] = m_run;
        s_ml[w][r16][1] = l_run;
    }
    __syncthreads();
    const int hh = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * 8;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ww++) M = fmaxf(M, s_ml[ww][hh][0]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float L = 0.f, o[8];
#pragma unroll
    for (int j = 0; j < 8; j++) o[j] = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ww++) {
        const float f = exp2f(s_ml[ww][hh][0] - Mu);
        L += f * s_ml[ww][hh][1];
#pragma unroll
        for (int j = 0; j < 8; j++) o[j] += f * ob[(ww * 16 + hh) * 128 + d0 + j];
    }

    const size_t row_id = ((size_t)l * p.n_q + i) * p.H + hg * 16 + hh;
    if (p.n_splits > 1) {
        const size_t rec0 = (((size_t)l * p.n_q + i) * HG + hg) * p.n_splits;
        float *rec = p.ws_part + (rec0 + split) * kPartFloats + hh * 130;
        if ((threadIdx.x & 15) == 0) {
            rec[0] = M;
            rec[1] = L;
        }
#pragma unroll
        for (int j = 0; j < 8; j++) rec[2 + d0 + j] = o[j];
        const size_t ctr = ((size_t)l * p.n_q + i) * HG + hg;
        if (!last_arrival(p.ws_cnt + ctr, (uint32_t)p.n_splits, &s_flag)) return;
        // merge the split records of this (layer, query, head group)
        M = -INFINITY;
        for (int c = 0; c < p.n_splits; c++) {
            const float *r = p.ws_part + (rec0 + c) * kPartFloats + hh * 130;
            M = fmaxf(M, __hip_atomic_load(r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
        const float Mu2 = (M == -INFINITY) ? 0.f : M;
        L = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++) o[j] = 0.f;
        for (int c = 0; c < p.n_splits; c++) {
            const float *r = p.ws_part + (rec0 + c) * kPartFloats + hh * 130;
            const float f = exp2f(__hip_atomic_load(r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - Mu2);
            L += f * __hip_atomic_load(r + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int j = 0; j < 8; j++)
                o[j] += f * __hip_atomic_load(r + 2 + d0 + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    const float inv = 1.f / L;
    uint32_t packed[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
        packed[j] = (uint32_t)f32_to_bf16(o[2 * j] * inv) | ((uint32_t)f32_to_bf16(o[2 * j + 1] * inv) << 16);
    *reinterpret_cast<uint4 *>((uint16_t *)p.out + row_id * 128 + d0) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    if (p.lse && (threadIdx.x & 15) == 0) p.lse[row_id] = (M + log2f(L)) * kLn2;
}

// ============================================================ planning / launch
static int ceil_div_i(long long a, long long b) { return (int)((a + b - 1) / b); }

AttendPlan plan_attend(int n_q, int n_layers, int H, int D, int K, int W, int dtype)
{
    AttendPlan pl{false, 1, 0, 0};
    pl.mfma = (dtype == 1) && (D == 128) && (H % 16 == 0);
    if (!pl.mfma) return pl;
    const int n_keys_max = K + W;
    const int steps = std::max(1, ceil_div_i(n_keys_max, kAttendKeysPerIter));
    const long long base = (long long)n_q * n_layers * (H / 16);
    int n_splits = 1;
    if (base < kTargetWorkgroups) n_splits = std::min(steps, ceil_div_i(kTargetWorkgroups, base));
    const int steps_per_split = ceil_div_i(steps, n_splits);
    n_splits = ceil_div_i(steps, steps_per_split);
    pl.n_splits = n_splits;
    pl.keys_per_split = steps_per_split * kAttendKeysPerIter;
    pl.part_bytes = (n_splits > 1) ? (size_t)base * n_splits * kPartFloats * sizeof(float) : 0;
    return pl;
}

hipError_t launch_attend(const AttendParams &p0, const AttendPlan &pl, int D, int dtype, hipStream_t st)
{
    if (p0.n_q <= 0 || p0.n_layers <= 0) return hipSuccess;
    AttendParams p = p0;
    if (pl.mfma) {
        p.n_splits = pl.n_splits;
        p.keys_per_split = pl.keys_per_split;
        p.n_q_pad = (p.n_q + 7) / 8 * 8;
        const long long n_wg = (long long)p.n_q_pad * pl.n_splits * (p.H / 16) * p.n_layers;
        hipLaunchKernelGGL(k_attend_mfma, dim3((unsigned)n_wg), dim3(256), 0, st, p);
        return hipGetLastError();
    }
    dim3 grid((unsigned)p.n_q, (unsigned)p.n_layers, (unsigned)ceil_div_i(p.H, 4));
    if (dtype == 0) {
        if (D == 64) hipLaunchKernelGGL((k_attend_generic<float, 64>), grid, dim3(256), 0, st, p);
        else hipLaunchKernelGGL((k_attend_generic<float, 128>), grid, dim3(256), 0, st, p);
    } else {
        if (D == 64) hipLaunchKernelGGL((k_attend_generic<uint16_t, 64>), grid, dim3(256), 0, st, p);
        else hipLaunchKernelGGL((k_attend_generic<uint16_t, 128>), grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace csa2
