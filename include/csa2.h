/*
 * csa2.h -- C ABI of the CSA2 sparse-attention library for MI355X (gfx950).
 *
 * The method (page "DeepSeek V4.1 Flash", k-a.in, and the forum summary on
 * artofsm.art):
 *   - "Hierarchical indexer" key fact, and the forum summary's description of
 *     a hierarchical sparse indexer that narrows the attention candidates down
 *     to blocks: an indexer first scores blocks of B tokens and keeps a pool of
 *     at most P blocks, so at most P*B candidate tokens are scored;
 *   - "Sparse attention" key fact: each query then attends to its Top-K
 *     main-KV entries plus a sliding window of the W most recent tokens;
 *   - "CSA2 with cross-layer reuse" mode table: a Full layer computes its own
 *     keys and fresh indices, a Reindex layer reuses the keys but selects with
 *     its own indexer query, a Reuse layer reuses keys and indices; every mode
 *     has its own main query and its own sliding-window K/V.
 * The pages leave the scores open; this library fixes them:
 *   - token score  s_p = <q_idx, k_idx[p]>, int8 x int8 summed exactly in int32;
 *   - block score  s_j = <q_idx, kb_j>, where kb_j is the per-dimension mean of
 *     block j's k_idx rows that are visible to the query (positions <= t),
 *     rounded to the nearest integer with ties to even;
 *   - every selection ranks by score, higher first, and breaks ties by the
 *     lower block id / lower position, so the selected set is unique;
 *   - attention is one softmax per head over the selected main entries and the
 *     window entries together, logits scale * <q, k>, scale = 1/sqrt(D) unless
 *     given.
 *
 * Conventions for every entry point:
 *   - Pointers named as device data are device pointers (hipMalloc'd or from a
 *     framework allocator) owned by the caller.  The library allocates nothing
 *     and keeps no pointer after the call returns.
 *   - Arrays are dense, row-major, with the shapes given; int32 indices.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; the call returns after the launches, without waiting.
 *   - Arguments are checked before anything is launched; a bad argument
 *     returns its status code and leaves every buffer untouched.  A failed
 *     launch returns CSA2_E_HIP.  Faults inside a kernel surface at the
 *     caller's next synchronisation.  Nothing is printed, nothing is thrown.
 *   - Positions: sequence s holds positions 0..T-1 in every cache; a query row
 *     i belongs to sequence q_seq[i] at position q_pos[i] (0 <= q_pos[i] < T)
 *     and sees positions <= q_pos[i] only (the pages: both stacks are causal);
 *     with a compression ratio the main caches count entries (see csa2_cfg).
 *     Device-side values of q_seq/q_pos are trusted: out-of-range values are
 *     undefined behaviour, not an error code.
 *   - Workspace: `ws` is device memory of at least csa2_workspace_bytes()
 *     bytes that is zero-filled before its first use (csa2_workspace_init or
 *     any zero fill).  It holds selection histograms that every call leaves
 *     zeroed again, and scratch; one workspace serves any number of calls
 *     issued in order on one stream when it is sized for the largest of them.
 *     Calls that run concurrently need separate workspaces.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 3

typedef enum {
    CSA2_OK = 0,
    CSA2_E_NULL = 1,        /* a required pointer is NULL                        */
    CSA2_E_SHAPE = 2,       /* a size is out of range or sizes disagree          */
    CSA2_E_DTYPE = 3,       /* unknown element type                              */
    CSA2_E_UNSUPPORTED = 4, /* valid but not built (e.g. head_dim not 64 or 128) */
    CSA2_E_ALIGN = 5,       /* a device pointer is not 16-byte aligned           */
    CSA2_E_WORKSPACE = 6,   /* workspace missing or smaller than required        */
    CSA2_E_HIP = 7,         /* a HIP runtime call or kernel launch failed        */
    CSA2_E_MODE = 8         /* unknown layer mode, or a mode/argument mismatch   */
} csa2_status;

typedef enum {
    CSA2_FULL = 0,      /* own keys: update block keys, fresh pool + Top-K, attend */
    CSA2_REINDEX = 1,   /* shared keys, own q_idx: fresh pool + Top-K, attend      */
    CSA2_REUSE = 2,     /* shared keys and indices: attend only                    */
    CSA2_SWA = 3,       /* sliding-window-only layer: attend to the window alone   */
    CSA2_REINDEX_TOKENS = 4 /* shared keys and pool, own q_idx: fresh token Top-K  */
} csa2_mode;

typedef enum { CSA2_F32 = 0, CSA2_BF16 = 1 } csa2_dtype;

/* How the block pass treats a query's own block when it is partial (t is not
 * its last position).  The pages say nothing about it; three readings:
 *   CSA2_TAIL_VISIBLE: eligible, keyed by the rounded mean of its rows at
 *                      positions <= t (the default);
 *   CSA2_TAIL_EXCLUDE: not eligible (its tokens are in the sliding window
 *                      whenever W >= B); a query at t < B-1 then has no
 *                      eligible block and selects nothing;
 *   CSA2_TAIL_WHOLE:   eligible, keyed by the rounded mean of all of its rows
 *                      that exist in k_idx (positions < T), i.e. including
 *                      positions after t (only prefill has any).
 * Complete blocks are the same under every reading, and the token Top-K
 * takes positions <= t only. */
typedef enum { CSA2_TAIL_VISIBLE = 0, CSA2_TAIL_EXCLUDE = 1, CSA2_TAIL_WHOLE = 2 } csa2_tail;

/* Selection and attention sizes (one struct shared by every call). */
typedef struct {
    int32_t block;     /* B: tokens per block; 1..16                              */
    int32_t pool;      /* P: blocks kept by the hierarchical pass; >= 1           */
    int32_t top_k;     /* K: selected main-KV entries; 0 (window only) .. P*B     */
    int32_t window;    /* W: sliding window length; 0 .. 1024; K + W >= 1         */
    int32_t d_idx;     /* indexer dimension: 32 or 64                             */
    int32_t n_heads;   /* H: query heads sharing one main-KV head; 1 .. 128       */
    int32_t head_dim;  /* D: 64 or 128                                            */
    int32_t dtype;     /* csa2_dtype of Q, K, V and the output                    */
    float scale;       /* logit scale; 0 means 1/sqrt(head_dim)                  */
    int32_t tail;      /* csa2_tail reading of a partial own block                */
    int32_t ratio;     /* tokens per main-KV entry, 0 or 1 .. 256; see below      */
} csa2_cfg;
/* Compressed main-KV (the architecture figure of the V4.1 Flash page names
 * CSA2(ratio, mode) and leaves the ratio undefined; this library reads it so):
 * with ratio r > 1 the main-KV and indexer caches (k_idx, k_blk, K and V
 * main) hold one entry per r tokens, entry j standing for tokens j*r ..
 * j*r + r - 1, made outside the library like every other K/V row.  q_pos
 * stays a token position; a query at token t sees the complete entries
 * 0 .. (t + 1) / r - 1 (it needs (t + 1) / r <= T, T counting entries), and
 * blocks, pool, Top-K ids and k_blk all count entries.  A query with no
 * complete entry (t < r - 1) selects nothing and attends to its window alone,
 * so r > 1 needs window >= 1.  The window caches keep one row per token.
 * Ratio 0 or 1: one entry per token.
 * Limits: P*B <= 16384 candidates per query (the pages' cap on candidates
 * scored by an indexer); T <= 2^24 positions.
 * Flat Top-K (no block hierarchy): block = 1 and pool = top_k select the K
 * best tokens of the whole prefix directly; the block keys of blocks of one
 * token are the k_idx rows themselves (csa2_build_block_keys copies them). */

int32_t csa2_abi_version(void);
const char *csa2_status_str(int32_t status);

/* Measurement aid; no call above needs it.  csa2_profile_begin arms a list of
 * max_launches (0 .. 65536) pairs of HIP events: while armed, each library
 * kernel launch whose kernel name contains kernel_filter (NULL or "" = every
 * kernel) takes the next pair, launched with hipExtLaunchKernel so that the
 * pair records that kernel's own execution interval.  Launches beyond the
 * list, and launches into a stream that is capturing a graph, are not timed.
 * csa2_profile_end disarms, waits for every timed launch and writes their
 * number; csa2_profile_record then reads back launch i (in launch order): its
 * kernel name (truncated to name_len - 1 bytes) and its duration in
 * milliseconds.  The records stay readable until the next csa2_profile_begin.
 * Process-wide state; calls are serialised by a mutex.  Errors: CSA2_E_SHAPE
 * for a bad count, filter or index (or reading while armed), CSA2_E_HIP when
 * an event cannot be created or read. */
int32_t csa2_profile_begin(const char *kernel_filter, int32_t max_launches);
int32_t csa2_profile_end(int32_t *n_timed);
int32_t csa2_profile_record(int32_t i, char *name, int32_t name_len, float *ms);

/* Bytes of workspace for calls of at most n_q query rows, caches of at most T
 * positions and at most n_layers layers per group call: an upper bound of
 * every such call's zero-between-calls head plus an upper bound of its
 * scratch, so one workspace of this size serves any sequence of them in
 * stream order.  Writes *bytes.  (Plumbing of the library, not a step of the
 * method.) */
int32_t csa2_workspace_bytes(const csa2_cfg *cfg, int32_t n_q, int32_t T, int32_t n_layers,
                             size_t *bytes);

/* Zero-fills `bytes` of device memory at `ws` with a kernel (safe to record
 * into a HIP graph).  `ws` 4-byte aligned, `bytes` a multiple of 4.  (Plumbing,
 * not a step of the method.) */
int32_t csa2_workspace_init(void *ws, size_t bytes, void *stream);

/* Block keys (the block-level indexer keys the hierarchical pass scores;
 * "Hierarchical indexer" key fact of the page "DeepSeek V4.1 Flash" and the
 * forum summary's blocks of candidates; the key of a block is fixed here as
 * the rounded mean of its k_idx rows).
 * For each sequence s < n_seq and each block j in [blk_begin, blk_end) that
 * is complete ((j+1)*B <= T):
 *     k_blk[s][j][c] = round_half_even(mean over p in [jB, jB+B) of k_idx[s][p][c])
 *   k_idx : device int8 [n_seq][T][d_idx]
 *   k_blk : device int8 [n_seq][T/B][d_idx]  (only blocks in range are written;
 *           NULL allowed when T < B, i.e. no block is complete)
 * A Full layer builds all blocks once (prefill) and, in decode, the block that
 * the newest token completes.  Incomplete blocks are never stored: the
 * selection calls compute the key of a query's own block from k_idx. */
int32_t csa2_build_block_keys(const csa2_cfg *cfg, const int8_t *k_idx, int32_t n_seq, int32_t T,
                              int32_t blk_begin, int32_t blk_end, int8_t *k_blk, void *stream);

/* Token append: the cache write before a Full layer's step ("CSA2 with
 * cross-layer reuse" mode table: a Full layer computes its own main KV and
 * indexer keys, which later layers of its group reuse).  For each new token
 * i < n_new, with s = seq[i] and t = pos[i] (0 <= s < n_seq, 0 <= t < T):
 *     k_idx[s][t]  = new_k_idx[i]    (d_idx int8)
 *     k_main[s][t] = new_k[i]        (head_dim elements of cfg->dtype)
 *     v_main[s][t] = new_v[i]
 * then, after every row of the call is written, for each token that completes
 * its block ((t + 1) % B == 0) the key of that block j = t / B, as in
 * csa2_build_block_keys (the "Hierarchical indexer" key fact's block level):
 *     k_blk[s][j][c] = round_half_even(mean over p in [jB, jB+B) of k_idx[s][p][c])
 *   seq, pos    : device int32 [n_new]; distinct (s, t) pairs (two new rows
 *                 for one position race); values trusted like q_seq/q_pos
 *   new_k_idx   : device int8 [n_new][d_idx], 16-byte aligned
 *   new_k/new_v : device [n_new][head_dim] of cfg->dtype, 16-byte aligned
 *   k_idx       : device int8 [n_seq][T][d_idx]         (in/out)
 *   k_main/v_main : device [n_seq][T][head_dim]         (in/out)
 *   k_blk       : device int8 [n_seq][T/B][d_idx], or NULL to leave block keys
 *                 to a later csa2_build_block_keys / Full layer group
 * With compressed main-KV (cfg->ratio > 1) the rows are entries and pos[i] an
 * entry index: the caller appends entry j once its r tokens have arrived.
 * n_new = 0 launches nothing and accepts empty (NULL) arrays.  No workspace. */
int32_t csa2_append_tokens(const csa2_cfg *cfg, int32_t n_new, const int32_t *seq, const int32_t *pos,
                           const int8_t *new_k_idx, const void *new_k, const void *new_v, int8_t *k_idx,
                           void *k_main, void *v_main, int8_t *k_blk, int32_t n_seq, int32_t T,
                           void *stream);

/* Hierarchical block pass ("Hierarchical indexer" key fact of the page
 * "DeepSeek V4.1 Flash": a block-level pass bounds the candidates an indexer
 * scores, at most P*B tokens whatever the context length; the forum summary's
 * hierarchical sparse indexer that narrows candidates down to blocks).
 * For query row i at position t = q_pos[i] in
 * sequence s = q_seq[i], the eligible blocks are j = 0 .. t/B (each holds at
 * least one visible token).  If there are at most P of them, all are pooled;
 * otherwise the P with the highest block score, ties to the lower block id.
 * Blocks j < t/B take their key from k_blk; block t/B (the query's own, maybe
 * incomplete) takes the rounded mean of its rows jB..t of k_idx.
 *   q_idx   : device int8  [n_q][d_idx]
 *   q_seq, q_pos : device int32 [n_q]
 *   k_idx   : device int8  [n_seq][T][d_idx]
 *   k_blk   : device int8  [n_seq][T/B][d_idx], blocks < t/B filled (NULL
 *             allowed when T < B: no block is complete)
 *   blk_ids : device int32 [n_q][P] out: pooled block ids ascending, then -1;
 *             may be NULL when every pool is the whole prefix ((T-1)/B + 1 <=
 *             P): the pool of row i is then blocks 0 .. blk_cnt[i]-1 and no id
 *             is stored (CSA2_E_NULL otherwise)
 *   blk_cnt : device int32 [n_q]    out: number of pooled blocks           */
int32_t csa2_index_blocks(const csa2_cfg *cfg, int32_t n_q, const int8_t *q_idx,
                          const int32_t *q_seq, const int32_t *q_pos, const int8_t *k_idx,
                          const int8_t *k_blk, int32_t n_seq, int32_t T, int32_t *blk_ids,
                          int32_t *blk_cnt, void *ws, size_t ws_bytes, void *stream);

/* Token Top-K ("Sparse attention" key fact of the page "DeepSeek V4.1
 * Flash": each query keeps its Top-K main-KV entries; "Hierarchical indexer":
 * only the tokens of the pooled blocks are scored).
 * The candidates of query row i are the visible positions
 * (p <= t) of its pooled blocks.  If there are at most K, all are selected;
 * otherwise the K with the highest token score, ties to the lower position.
 *   blk_ids, blk_cnt : as written by csa2_index_blocks for the same cfg, T and
 *                      queries; blk_ids may be NULL when every pool is the
 *                      whole prefix ((T-1)/B + 1 <= P), pool slot r then
 *                      holds block r (the many-query kernel reads neither)
 *   topk     : device int32 [n_q][K] out: selected positions ascending, then -1
 *   topk_cnt : device int32 [n_q]    out: number selected                   */
int32_t csa2_topk_tokens(const csa2_cfg *cfg, int32_t n_q, const int8_t *q_idx,
                         const int32_t *q_seq, const int32_t *q_pos, const int8_t *k_idx,
                         int32_t n_seq, int32_t T, const int32_t *blk_ids, const int32_t *blk_cnt,
                         int32_t *topk, int32_t *topk_cnt, void *ws, size_t ws_bytes,
                         void *stream);

/* Sparse attention for a group of n_layers layers that share one index set
 * and one main K/V cache (the layer-group call; n_layers = 1 is one layer).
 * "Sparse attention" key fact of the page "DeepSeek V4.1 Flash" (each query
 * attends to its Top-K main entries plus a sliding window) and the mode table
 * of "CSA2 with cross-layer reuse" (layers that share the main KV and the
 * indices; every layer has its own Q and its own window K/V).
 * For layer l, query row i, head h: one softmax over
 *   - main entries p in topk[i][0 .. topk_cnt[i]) with k_main/v_main rows of
 *     sequence q_seq[i] (skipped when topk is NULL: a window-only layer), and
 *   - window positions max(0, t-W+1) .. t with this layer's own k_swa/v_swa,
 *     whose row r holds position swa_first + r.
 *   q      : device [n_layers][n_q][H][D]             (dtype)
 *   k_main, v_main : device [n_seq][T][D]             (dtype)
 *   k_swa, v_swa   : device [n_layers][n_seq][swa_len][D] (dtype)
 *   topk, topk_cnt : device int32 [n_q][K], [n_q], or both NULL
 *   out    : device [n_layers][n_q][H][D]             (dtype) out
 *   lse    : device fp32 [n_layers][n_q][H] out (natural-log normaliser) or NULL
 * Window positions outside [swa_first, swa_first + swa_len) are not attended:
 * callers supply rows covering every query's window.  Window positions are
 * tokens; with compressed main-KV (ratio r) they may reach T*r + r - 2. */
int32_t csa2_attend_group(const csa2_cfg *cfg, int32_t n_layers, int32_t n_q, const void *q,
                          const int32_t *q_seq, const int32_t *q_pos, const void *k_main,
                          const void *v_main, int32_t n_seq, int32_t T, const void *k_swa,
                          const void *v_swa, int32_t swa_first, int32_t swa_len,
                          const int32_t *topk, const int32_t *topk_cnt, void *out, float *lse,
                          void *ws, size_t ws_bytes, void *stream);

/* One layer: csa2_attend_group with n_layers = 1 (same passages).  It takes
 * no layer mode: in the mode table of "CSA2 with cross-layer reuse" the
 * three modes attend identically and differ only in where the indices come
 * from (fresh for Full and Reindex, shared for Reuse), so the caller passes
 * the indices of whichever layer selected them; csa2_layer_group carries the
 * mode and does the selection the mode asks for. */
int32_t csa2_attend(const csa2_cfg *cfg, int32_t n_q, const void *q, const int32_t *q_seq,
                    const int32_t *q_pos, const void *k_main, const void *v_main, int32_t n_seq,
                    int32_t T, const void *k_swa, const void *v_swa, int32_t swa_first,
                    int32_t swa_len, const int32_t *topk, const int32_t *topk_cnt, void *out,
                    float *lse, void *ws, size_t ws_bytes, void *stream);

/* A CSA2 layer group in one call: the first layer's mode decides the
 * selection work, then all n_layers layers attend with the shared indices
 * (the mode table of "CSA2 with cross-layer reuse": a Full or Reindex layer
 * followed by the Reuse layers that take its indices).
 *   CSA2_FULL    : csa2_build_block_keys over [blk_update_begin, T/B) (pass
 *                  blk_update_begin >= T/B to skip it: the block pass reads
 *                  the keys of the blocks before each query's own, so skip
 *                  only when they are current, as in decode, or when every
 *                  pool is the whole prefix, where no key is read),
 *                  csa2_index_blocks,
 *                  csa2_topk_tokens, csa2_attend_group; the block pass also
 *                  stores into k_blk the key of every block that a query
 *                  completes ((t+1) % B == 0), so a decode step keeps k_blk
 *                  current without a separate launch
 *   CSA2_REINDEX : csa2_index_blocks + csa2_topk_tokens with this layer's q_idx
 *                  over the shared k_idx/k_blk (read only), csa2_attend_group
 *   CSA2_REUSE   : csa2_attend_group with the given topk/topk_cnt (read only)
 *   CSA2_SWA     : csa2_attend_group with no main entries (topk ignored)
 *   CSA2_REINDEX_TOKENS : csa2_topk_tokens with this layer's q_idx over the
 *                  given pool (blk_ids/blk_cnt of the group whose index set it
 *                  shares, read only), csa2_attend_group: the reading of the
 *                  Reindex layer that recomputes only the token Top-K
 * blk_ids/blk_cnt/topk/topk_cnt are outputs for FULL/REINDEX, inputs for
 * REUSE; for REINDEX_TOKENS blk_ids/blk_cnt are inputs and topk/topk_cnt
 * outputs.  Shapes as in the calls above; blk_ids may be NULL when every pool
 * is the whole prefix ((T-1)/B + 1 <= P), as in csa2_index_blocks. */
int32_t csa2_layer_group(const csa2_cfg *cfg, int32_t mode, int32_t n_layers, int32_t n_q,
                         const int8_t *q_idx, const int32_t *q_seq, const int32_t *q_pos,
                         const int8_t *k_idx, int8_t *k_blk, int32_t blk_update_begin,
                         int32_t n_seq, int32_t T, const void *q, const void *k_main,
                         const void *v_main, const void *k_swa, const void *v_swa,
                         int32_t swa_first, int32_t swa_len, int32_t *blk_ids, int32_t *blk_cnt,
                         int32_t *topk, int32_t *topk_cnt, void *out, float *lse, void *ws,
                         size_t ws_bytes, void *stream);

/* csa2_layer_group in one kernel launch (the same operation: the mode table
 * of "CSA2 with cross-layer reuse" and the "Sparse attention" and
 * "Hierarchical indexer" key facts of the page "DeepSeek V4.1 Flash"), for a
 * Full or Reindex group of few decode queries, where csa2_layer_group takes
 * its four-launch fused path (block scoring; pool selection with token
 * scoring; token Top-K with chunked attention; merge of the chunk records).
 * The four stages become phases of one kernel that hand over per query
 * through counters in the workspace head (zero between calls, left zero).
 * Arguments, outputs and workspace size are those of csa2_layer_group and
 * the results are identical to its; a call outside that regime (another mode,
 * many queries, or an attention plan without key-list chunks) returns
 * CSA2_E_UNSUPPORTED, a workspace too small for the fused path
 * CSA2_E_WORKSPACE.  The launch is cooperative (all workgroups resident)
 * unless the stream is capturing a graph; a capture records an ordinary
 * launch sized to what the device holds at once, and must not be replayed
 * while other work occupies the device.  Every wait inside the kernel is
 * bounded, so a replay that breaks this gives wrong output, not a hang.  On
 * MI355X the hand-offs cost more than the kernel boundaries they replace, so
 * csa2_layer_group stays the faster call. */
int32_t csa2_layer_group_single(const csa2_cfg *cfg, int32_t mode, int32_t n_layers, int32_t n_q,
                                const int8_t *q_idx, const int32_t *q_seq, const int32_t *q_pos,
                                const int8_t *k_idx, int8_t *k_blk, int32_t blk_update_begin,
                                int32_t n_seq, int32_t T, const void *q, const void *k_main,
                                const void *v_main, const void *k_swa, const void *v_swa,
                                int32_t swa_first, int32_t swa_len, int32_t *blk_ids, int32_t *blk_cnt,
                                int32_t *topk, int32_t *topk_cnt, void *out, float *lse, void *ws,
                                size_t ws_bytes, void *stream);

/* csa2_layer_group without a workspace argument, for callers that cannot
 * allocate device memory: code under graph capture, tight serving loops,
 * harnesses that forbid allocation.  It allocates nothing (no hipMalloc,
 * hipFree or allocating library routine): its scratch is a 16 MiB device
 * array inside the library (one per GPU, held until the process ends), whose
 * address is looked up once per device on the first call with that device
 * current.  Arguments, results and errors are those of csa2_layer_group; a
 * call whose stages need more than the 16 MiB returns CSA2_E_WORKSPACE
 * without launching anything (16 MiB holds the decode layer group at batch
 * 8 and 128K context with room to spare).  The histograms at the head of the
 * array are cleared by a kernel at the start of every call that selects.
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and give undefined
 * results; calls issued in order on one stream are safe. */
int32_t csa2_layer_group_static(const csa2_cfg *cfg, int32_t mode, int32_t n_layers, int32_t n_q,
                                const int8_t *q_idx, const int32_t *q_seq, const int32_t *q_pos,
                                const int8_t *k_idx, int8_t *k_blk, int32_t blk_update_begin,
                                int32_t n_seq, int32_t T, const void *q, const void *k_main,
                                const void *v_main, const void *k_swa, const void *v_swa,
                                int32_t swa_first, int32_t swa_len, int32_t *blk_ids, int32_t *blk_cnt,
                                int32_t *topk, int32_t *topk_cnt, void *out, float *lse, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
