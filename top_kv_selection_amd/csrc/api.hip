// api.hip -- the C ABI declared in include/csa2.h: argument checks, workspace
// layout and the mode dispatch of a CSA2 layer group.
//
// Workspace layout: state that must be zero between calls (the selection
// histograms) at the head, scratch (scores, split records) at the tail.  The
// kernels leave the head zeroed again, so a zero-filled workspace sized by
// csa2_workspace_bytes for the largest call serves every call in stream order.
#include <math.h>
#include <algorithm>

#include "csa2.h"
#include "internal.h"

using namespace csa2;

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
    return CSA2_OK;
}

int32_t check_sizes(int32_t n_q, int32_t n_seq, int32_t T)
{
    if (n_q < 0 || n_seq < 1 || T < 1 || T > (1 << 24)) return CSA2_E_SHAPE;
    return CSA2_OK;
}



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
    if (!q_idx || !q_seq || !q_pos || !k_idx || !k_blk || !blk_ids || !blk_cnt) return CSA2_E_NULL;
    if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(k_blk) || !aligned4(q_seq) ||
        !aligned4(q_pos) || !aligned4(blk_ids) || !aligned4(blk_cnt))
        return CSA2_E_ALIGN;
    const SelectPlan pl = plan_index(n_q, T, c->block, c->pool, c->d_idx);
    Region r;
    if (int32_t e = carve(ws, ws_bytes, select_head_bytes(n_q, pl.split), pl.key_bytes, r)) return e;
    if (!launch) return CSA2_OK;
    IndexParams p{};
    p.q_idx = q_idx; p.q_seq = q_seq; p.q_pos = q_pos; p.k_idx = k_idx; p.k_blk = k_blk;
    p.k_blk_store = k_blk_store;
    p.T = T; p.B = c->block; p.P = c->pool; p.n_q = n_q; p.G = pl.G; p.chunk = pl.chunk; p.tail = c->tail;
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
                size_t ws_bytes, hipStream_t st, bool launch)
{
    if (c->top_k < 1) return CSA2_E_SHAPE;
    if (!q_idx || !q_seq || !q_pos || !k_idx || !blk_ids || !blk_cnt || !topk || !topk_cnt)
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
    p.chunk = pl.chunk;
    p.ws_keys = (uint32_t *)r.data;
    p.ws_stride = ((long long)c->pool * c->block + 3) / 4 * 4;
    p.ws_hist = r.ctr;
    p.topk = topk; p.topk_cnt = topk_cnt;
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
    if (c->window > 0 && (swa_len < 1 || swa_first < 0 || swa_first >= T || swa_len > T)) return CSA2_E_SHAPE;
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
    size_t head, blk_off, tok_off, tok_hist_off, part_off, tail;
};

FusedPlan plan_fused(const csa2_cfg *c, int n_q, int T, int n_layers)
{
    FusedPlan f{};
    const long long n_elig_max = (long long)(T - 1) / c->block + 1;
    f.idx = plan_index(n_q, T, c->block, c->pool, c->d_idx);
    f.tok = plan_topk(n_q, T, c->block, c->pool, c->top_k, c->d_idx);
    f.att = plan_attend(n_q, n_layers, c->n_heads, c->head_dim, c->top_k, c->window, c->dtype);
    f.ok = c->top_k >= 1 && f.idx.split && f.tok.split && n_elig_max <= kMaxCandidates && f.att.mfma && !f.att.rows &&
           (f.att.chunks || f.att.keys_per_split <= kAttendRowChunk) && c->pool <= kFusedPoolLds;
    f.blk_stride = (n_elig_max + 3) / 4 * 4;
    f.tok_stride = ((long long)c->pool * c->block + 3) / 4 * 4;
    f.head = (size_t)n_q * 2048 * sizeof(uint32_t);
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
    if (!k_idx || !k_blk) return CSA2_E_NULL;
    if (!aligned16(k_idx) || !aligned16(k_blk)) return CSA2_E_ALIGN;
    const int nblk = T / c->block;
    blk_begin = std::max(blk_begin, 0);
    blk_end = std::min(blk_end, nblk);
    if (!launch || blk_begin >= blk_end) return CSA2_OK;
    BlockKeysParams p{k_idx, k_blk, T, c->block, nblk, blk_begin, blk_end};
    return hip_status(launch_block_keys(p, n_seq, c->d_idx, st));
}

int32_t fused_layer_group(const csa2_cfg *c, int32_t mode, int32_t n_layers, int32_t n_q,
                          const int8_t *q_idx, const int32_t *q_seq, const int32_t *q_pos,
                          const int8_t *k_idx, int8_t *k_blk, int32_t blk_update_begin,
                          int32_t n_seq, int32_t T, const void *q, const void *k_main,
                          const void *v_main, const void *k_swa, const void *v_swa,
                          int32_t swa_first, int32_t swa_len, int32_t *blk_ids, int32_t *blk_cnt,
                          int32_t *topk, int32_t *topk_cnt, void *out, float *lse, void *ws,
                          size_t ws_bytes, hipStream_t st, const FusedPlan &f)
{
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
    if (!aligned16(ws)) return CSA2_E_ALIGN;
    uint32_t *head = (uint32_t *)ws;
    char *tail = (char *)ws + round_up(f.head);
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
    ip.nblk = T / c->block;
    ip.ws_keys = blk_keys; ip.ws_stride = f.blk_stride; ip.ws_hist = head;
    ip.blk_ids = blk_ids; ip.blk_cnt = blk_cnt;
    // block scoring (keys and histogram to the workspace)
    if (int32_t e = hip_status(launch_index_blocks(ip, f.idx, c->d_idx, st, false))) return e;

    TopkParams tp{};
    tp.q_idx = q_idx; tp.q_seq = q_seq; tp.q_pos = q_pos; tp.k_idx = k_idx;
    tp.blk_ids = blk_ids; tp.blk_cnt = blk_cnt;
    tp.T = T; tp.B = c->block; tp.P = c->pool; tp.K = c->top_k; tp.n_q = n_q; tp.tail = c->tail;
    tp.G = f.tok.G; tp.chunk = f.tok.chunk;
    tp.ws_keys = tok_keys; tp.ws_stride = f.tok_stride; tp.ws_hist = tok_hist;
    tp.topk = topk; tp.topk_cnt = topk_cnt;
    // pool selection + token scoring in one launch (each scoring workgroup
    // redoes the pool selection); the Top-K is taken inside the attention
    // launch, whose writer also zeroes the block histogram
    if (int32_t e = hip_status(launch_pool_tokens(ip, tp, c->d_idx, st))) return e;

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
    return hip_status(launch_attend(ap, f.att, c->head_dim, c->dtype, st, true));
}

}  // namespace

extern "C" {

int32_t csa2_abi_version(void) { return CSA2_ABI_VERSION; }

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
    const SelectPlan pi = plan_index(n_q, T, c->block, c->pool, c->d_idx);
    const SelectPlan pt = plan_topk(n_q, T, c->block, c->pool, c->top_k, c->d_idx);
    const AttendPlan pa = plan_attend(n_q, n_layers, c->n_heads, c->head_dim, c->top_k, c->window, c->dtype);
    const size_t ctr = std::max(select_head_bytes(n_q, pi.split), select_head_bytes(n_q, pt.split));
    const size_t data = std::max({pi.key_bytes, pt.key_bytes, pa.part_bytes});
    size_t need = round_up(ctr) + round_up(data);
    const FusedPlan f = plan_fused(c, n_q, T, n_layers);
    if (f.ok) need = std::max(need, round_up(f.head) + f.tail);
    *bytes = need;
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
    if (int32_t e = check_cfg(c)) return e;
    if (int32_t e = check_sizes(n_q, n_seq, T)) return e;
    if (mode < CSA2_FULL || mode > CSA2_REINDEX_TOKENS) return CSA2_E_MODE;
    if (n_layers < 1) return CSA2_E_SHAPE;
    if (mode != CSA2_SWA && c->top_k < 1) return CSA2_E_MODE;
    if (n_q == 0) return CSA2_OK;
    hipStream_t st = (hipStream_t)stream;
    const bool selects = mode == CSA2_FULL || mode == CSA2_REINDEX;
    const bool tokens_only = mode == CSA2_REINDEX_TOKENS;
    const bool window_only = mode == CSA2_SWA;
    if (mode == CSA2_REUSE && (!topk || !topk_cnt)) return CSA2_E_NULL;
    if (selects) {
        const FusedPlan f = plan_fused(c, n_q, T, n_layers);
        if (f.ok && ws && ws_bytes >= round_up(f.head) + f.tail)
            return fused_layer_group(c, mode, n_layers, n_q, q_idx, q_seq, q_pos, k_idx, k_blk,
                                     blk_update_begin, n_seq, T, q, k_main, v_main, k_swa, v_swa,
                                     swa_first, swa_len, blk_ids, blk_cnt, topk, topk_cnt, out, lse,
                                     ws, ws_bytes, st, f);
    }
    // every stage is checked before the first launch, then all are launched
    for (int pass = 0; pass < 2; pass++) {
        const bool launch = pass == 1;
        if (mode == CSA2_FULL) {
            if (int32_t e = do_block_keys(c, k_idx, n_seq, T, blk_update_begin, T / c->block,
                                          k_blk, st, launch))
                return e;
        }
        if (selects) {
            if (int32_t e = do_index(c, n_q, q_idx, q_seq, q_pos, k_idx, k_blk, n_seq, T, blk_ids,
                                     blk_cnt, ws, ws_bytes, st, launch,
                                     mode == CSA2_FULL ? k_blk : nullptr))
                return e;
            if (int32_t e = do_topk(c, n_q, q_idx, q_seq, q_pos, k_idx, T, blk_ids, blk_cnt, topk,
                                    topk_cnt, ws, ws_bytes, st, launch))
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

}  // extern "C"
