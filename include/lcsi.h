/*
 * lcsi.h -- C ABI of liblcsi.so, the gfx950 (MI355X) hot path of sparse
 * attention with a lightning indexer and cross-layer index reuse.
 *
 * The method (described in prose on the pages this library follows):
 *  - An indexer in front of each layer's attention scores every causal key
 *    for every query and keeps the top-k positions; the main attention then
 *    reads only those rows.  IndexCache news article (app.myzaker.com),
 *    section "IndexCache"; IndexShare explainer (yun88.com), section on the
 *    hidden indexer cost of sparse attention.
 *  - The indexer is a dot product followed by a top-k.  IndexShare term
 *    page (earlyterms.com), opening definition.  This library fixes the score
 *    as  score[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:])  for s <= p_t,
 *    one key row per token shared by all indexer heads, and the selection as
 *    the k largest scores with ties going to the lower position.
 *  - Full (F) layers run the indexer and cache the index set; Shared (S)
 *    layers skip it and reuse the most recent F layer's set, while still
 *    running their own attention.  IndexCache article (linkstar.cloud),
 *    section on adjacent layers repeating work; IndexShare explainer
 *    (yun88.com), section on the sharing mechanism (groups of four layers,
 *    the first one selects, the other three reuse).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE memory owned by the caller; the library
 *    never allocates, frees or synchronises.  Work is enqueued on `stream`
 *    (a hipStream_t passed as void*; NULL = the default stream) and runs
 *    asynchronously.
 *  - Strides are in ELEMENTS of the pointed-to type; the innermost dimension
 *    of every tensor is contiguous.
 *  - Status codes: 0 on success, a negative LCSI_E* code otherwise.  All
 *    argument checks run on the host before the first launch, so a failing
 *    call enqueues nothing.  Nothing prints, throws or aborts.
 *  - Calls are thread-safe as long as concurrent calls use distinct
 *    workspaces and outputs.
 *  - Results are deterministic: the same call on the same inputs gives the
 *    same bits, and no result depends on how many other rows share the call:
 *      - scores and index sets (idx_score_topk) are bit-identical across runs,
 *        batch sizes and query chunkings of the same rows;
 *      - sparse_attn computes each row with arithmetic fixed by top_k and by
 *        the kind of call alone: a multi-row call (T_q > 1) takes a row's
 *        index list in one pass, a decode call (T_q == 1) in a fixed number
 *        of parts, ceil(top_k / 256), merged by log-sum-exp.  A row's output bits therefore do
 *        not depend on B, and multi-row calls agree bit for bit whatever the
 *        chunking; a decode call may differ from the same row computed inside
 *        a multi-row call in the last bits (within the parity tolerance).
 *  - Workspaces (ws, ws_bytes) follow one rule in every call:
 *      ws == NULL, ws_bytes != NULL : query mode -- *ws_bytes receives the
 *                                     required size; nothing is launched.
 *                                     Only the descriptors are checked
 *                                     (output pointers may be NULL).
 *      ws == NULL, ws_bytes == NULL : run without a workspace; fails with
 *                                     LCSI_EWORKSPACE if one is required.
 *      ws != NULL                   : ws_bytes must point to the capacity of
 *                                     ws; a capacity below the requirement
 *                                     fails with LCSI_EWORKSPACE.
 *    Workspaces are device memory, 256-byte aligned, owned by the caller.
 */
#ifndef LCSI_H
#define LCSI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes */
#define LCSI_OK 0
#define LCSI_EINVAL -1       /* null pointer, bad dimension, top_k < 1, bad dtype, q_pos0 + T_q > T_kv */
#define LCSI_EUNSUPPORTED -2 /* valid but outside the kernels' envelope (see each call) */
#define LCSI_EWORKSPACE -3   /* workspace missing or smaller than required */
#define LCSI_EPATTERN -4     /* layer pattern starts with S, or #F != number of indexer descriptors */
#define LCSI_EALIGN -5       /* a base pointer or stride breaks the alignment rules */
#define LCSI_EHIP -6         /* a kernel launch or event record returned a HIP error */
#define LCSI_ESCRATCH -7     /* sparse_attn_noalloc: the call needs more than the static scratch */

/* ------------------------------------------------------------ key dtypes */
#define LCSI_KEY_BF16 0
#define LCSI_KEY_FP8_E4M3 1  /* OCP E4M3 ("fn": no infinities, max 448) + fp32 per-key scale > 0 */

/* ---------------------------------------------------------- query dtypes */
#define LCSI_Q_BF16 0
#define LCSI_Q_FP8_E4M3 1    /* OCP E4M3 + fp32 per-(token, head) scale > 0; needs fp8 keys */

/* ------------------------------------------------------ idx_score_topk flags */
#define LCSI_SCORES_PRESET 1u /* skip scoring: select from the scores already in score_ws */
#define LCSI_SCORES_ONLY 2u   /* score only: leave the scores in score_ws, write no indices */
#define LCSI_UNFUSED 4u       /* write every score row, then select (no fused candidate pass) */

#define LCSI_MAX_TOPK 2048

/* Indexer inputs of one F layer for query rows p = q_pos0 .. q_pos0+T_q-1
 * (the same positions for every batch entry).  Row p sees keys 0..p.
 *   q      bf16  [B][T_q][H_I][D_I]   strides q_sb, q_st, q_sh
 *   k      bf16  [B][T_kv][D_I]       strides k_sb, k_st    (LCSI_KEY_BF16)
 *          fp8   [B][T_kv][D_I]       strides k_sb, k_st    (LCSI_KEY_FP8_E4M3)
 *   k_scale fp32 [B][T_kv]            stride ks_sb          (fp8 only; else NULL)
 *   w      fp32  [B][T_q][H_I]        strides w_sb, w_st
 * Alignment: q, k, w base 16 bytes; q and k strides multiples of 16 bytes;
 * w strides multiples of 4 floats; k_scale 4 bytes.
 * fp8 queries (q_dtype = LCSI_Q_FP8_E4M3, keys fp8 too): q holds e4m3 bytes
 * [B][T_q][H_I][D_I] (strides in bytes), q_scale fp32 [B][T_q][H_I] with
 * strides qs_sb, qs_st (heads contiguous); a query element stands for its
 * value times the scale of its (token, head), as a key element does with its
 * key's scale.  The products then run on fp8 x fp8 MFMA.  With q_dtype =
 * LCSI_Q_BF16, q_scale is ignored (NULL).
 * Envelope: H_I in {4, 8, 16, 32, 64}; D_I in {64, 128}; 1 <= top_k <= 2048;
 * (512 / H_I) * lcsi_score_ld(T_kv) * 4 < 2^31 (the score rows one
 * workgroup writes stay below 2 GiB: T_kv < 2^22 for H_I = 4, < 2^26 for
 * H_I = 64), and a key row stride below 16 MiB, else LCSI_EUNSUPPORTED.
 * The fp8 scale of every key must be positive (it is applied
 * after the ReLU); NaN inputs are outside the contract. */
typedef struct lcsi_indexer {
    int32_t B, T_q, T_kv, H_I, D_I, top_k, key_dtype, q_dtype;
    int64_t q_pos0;
    const void *q;
    int64_t q_sb, q_st, q_sh;
    const void *k;
    int64_t k_sb, k_st;
    const float *k_scale;
    int64_t ks_sb;
    const float *w;
    int64_t w_sb, w_st;
    const float *q_scale;
    int64_t qs_sb, qs_st;
} lcsi_indexer;

/* Main-attention inputs of one layer (every layer, F or S, has its own).
 *   q    bf16 [B][T_q][H_q][D_qk]   strides q_sb, q_st, q_sh
 *   k    bf16 [B][T_kv][D_qk]       strides k_sb, k_st
 *   v    bf16 [B][T_kv][D_v]        strides v_sb, v_st   (may alias k: V = first D_v columns of the K row)
 *   out  bf16 [B][T_q][H_q][D_v]    strides o_sb, o_st, o_sh
 * All query heads attend through the one shared KV head.  Query row t sits
 * at position p_t = q_pos0 + t; an index that is negative, larger than p_t
 * or >= T_kv is skipped (it contributes nothing).  A row with no usable
 * index yields zeros.  Logits are sm_scale * q.k (sm_scale finite and > 0).
 * Alignment: all base pointers and strides multiples of 16 bytes.
 * Envelope: (D_qk, D_v) in {(128,128), (576,512)}; 1 <= H_q <= 64;
 * 1 <= top_k <= 2048; k and v row strides below 4 GiB. */
typedef struct lcsi_attn {
    int32_t B, T_q, T_kv, H_q, D_qk, D_v, top_k;
    float sm_scale;
    int64_t q_pos0;
    const void *q;
    int64_t q_sb, q_st, q_sh;
    const void *k;
    int64_t k_sb, k_st;
    const void *v;
    int64_t v_sb, v_st;
    void *out;
    int64_t o_sb, o_st, o_sh;
} lcsi_attn;

/* Row stride (in floats) of the score workspace for T_kv keys:
 * T_kv rounded up to a multiple of 64. */
int64_t lcsi_score_ld(int32_t T_kv);

/* Indexer score + top-k for one F layer (both steps of the indexer).
 *
 * Writes idx[b*idx_sb + t*idx_st + j], j < top_k, int32: the min(top_k, p_t+1)
 * positions with the largest score (ties to the lower position) in ascending
 * order, then -1 padding.  idx may be a slot of an index cache.
 *
 * score_ws: fp32 workspace holding the head-reduced score rows,
 * [B][T_q][lcsi_score_ld(T_kv)], row (b,t) at (b*T_q + t)*ld; only entries
 * s <= p_t are defined.  Per-head scores are never written.  Its size is
 * B*T_q*ld*4 bytes rounded up to 256, plus, when few long rows are selected
 * (B*T_q <= 128 rows of >= 32768 keys: decode), the selection's candidate
 * lists after the rows, plus, when the call takes the fused pass below,
 * B*T_q*4 bytes (rounded up to 256) of counts, 512 bytes for the list of
 * unsettled rows (a count and 64 row ids, rounded up to 256) and
 * B*T_q*16384*8 bytes of candidate slots; query mode returns the total for
 * the given flags
 * (workspace rule above; it is always required).
 *
 * Fused pass (the default for H_I >= 16 when the prefill kernel runs, i.e.
 * the rows fill the chip, and the longest row has more than 16384 keys):
 * score rows are not written.  The scoring kernel
 * keeps, per row, only the scores at or above a threshold drawn from a
 * sample of the row's scores (at most 16384 (score, position) pairs per
 * row) and the selection runs on those; a row whose sample misjudged it
 * (fewer than top_k or more than 16384 pairs) is rescored in full into
 * score_ws and selected from there.  The indices are bit-identical to the
 * unfused path (the same scores, the same selection rule); after a fused
 * call score_ws holds no defined scores.
 *
 * flags: LCSI_SCORES_PRESET selects from the scores the caller left in
 * score_ws (same layout) without scoring -- the hook for checking the
 * selection alone; LCSI_SCORES_ONLY stops after scoring (idx may be NULL);
 * LCSI_UNFUSED writes every score row and selects from them.  PRESET and
 * ONLY both set is LCSI_EINVAL.  With LCSI_SCORES_PRESET only B, T_q, T_kv,
 * q_pos0, top_k of `a` are read. */
int idx_score_topk(const lcsi_indexer *a, int32_t *idx, int64_t idx_sb,
                   int64_t idx_st, float *score_ws, size_t *ws_bytes,
                   unsigned flags, void *stream);

/* Sparse attention of every query head over the rows listed in
 * idx[b*idx_sb + t*idx_st + j], j < a->top_k (the index set of this row,
 * as written by idx_score_topk).  Output to a->out in bf16.
 * ws / ws_bytes: workspace for the partial results of a decode call
 * (T_q == 1 with top_k > 256: each row's list runs in ceil(top_k / 256)
 * parts of equal length, a multiple of 32 indices, on separate workgroups,
 * then a log-sum-exp merge): each part's output divided by its softmax sum
 * in fp16, then its (max logit, sum) in fp32.  The requirement is
 * B * parts * H_q * D_v * 2 bytes rounded up to 256, plus
 * B * parts * H_q * 8 bytes.  For any other
 * call it is 0 and ws may be NULL with ws_bytes NULL (workspace rule
 * above). */
int sparse_attn(const lcsi_attn *a, const int32_t *idx, int64_t idx_sb,
                int64_t idx_st, float *ws, size_t *ws_bytes, void *stream);

/* sparse_attn without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, kernels and results as sparse_attn;
 * the partial results of a decode call go to a static device scratch of
 * LCSI_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends (looked up on the first call per device).  A call
 * whose sparse_attn workspace requirement exceeds it returns LCSI_ESCRATCH
 * (at H_q = 64, D_v = 512, top_k = 2048: more than 95 sequences) and launches
 * nothing; LCSI_EINVAL also when `stream` belongs to another device than the
 * current one.  The call allocates nothing.  Every call on one GPU uses that
 * GPU's one scratch: calls that overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller; calls in order
 * on one stream are safe. */
#define LCSI_NOALLOC_SCRATCH_BYTES (48u << 20)
int sparse_attn_noalloc(const lcsi_attn *a, const int32_t *idx, int64_t idx_sb,
                        int64_t idx_st, void *stream);

/* The F/S layer loop over L layers (one conditional per layer):
 *   for l in 0..L-1:
 *     if pattern[l] (F): idx_score_topk(&idx_args[f], slot f % n_slots, flags 0); f++
 *     sparse_attn(&attn_args[l], current slot)
 * An S layer reads the slot written by the most recent F layer (the nearest
 * preceding F) and recomputes nothing.
 *   pattern    HOST array of L bytes, 1 = F, 0 = S; pattern[0] must be F.
 *   idx_args   HOST array of n_idx_args descriptors, one per F layer in
 *              layer order (n_idx_args must equal the number of F layers).
 *   attn_args  HOST array of L descriptors.  B, T_q, q_pos0 and top_k must
 *              be the same in every descriptor of the group (LCSI_EINVAL).
 *   idx_cache  device int32, n_slots slots of [B][T_q] rows laid out with
 *              idx_sb, idx_st; slot s starts at idx_cache + s*slot_stride.
 *              n_slots = 1 reuses one buffer for every F layer (no extra
 *              memory); n_slots = #F keeps every F layer's set.
 *   ws / ws_bytes  one workspace for all steps (they run in order on one
 *              stream); query mode returns what the group needs: the largest
 *              single requirement, or for a decode group (T_q == 1, whose
 *              attention splits every index list) the indexer's largest
 *              requirement plus two attention partial regions (below).
 *   events     optional HOST array of 4*L hipEvent_t (as void*), or NULL.
 *              For layer l: [4l] before the layer, [4l+1] after scoring
 *              (with the fused pass: after it and the two rescoring
 *              launches),
 *              [4l+2] after selection, [4l+3] after attention (for an S
 *              layer the first three are recorded at the same point).
 * Decode groups: the log-sum-exp merge of layer l's attention parts is done
 * by the workgroups of layer l+1's attention launch, before their own work
 * (the last layer's by a merge launch of its own), so no merge launch sits
 * between two layers; the results are the same bytes as sparse_attn's.  The
 * parts of consecutive layers alternate between the two partial regions.
 * Layer l's output is therefore complete only once layer l+1's attention
 * has run (event [4(l+1)+3]; every output at the end of the group), and no
 * layer's output may overlap another layer's inputs.
 * Pattern errors return LCSI_EPATTERN before anything is launched. */
int run_layer_group(int L, const uint8_t *pattern, const lcsi_indexer *idx_args,
                    int n_idx_args, const lcsi_attn *attn_args,
                    int32_t *idx_cache, int n_slots,
                    int64_t slot_stride, int64_t idx_sb, int64_t idx_st,
                    float *ws, size_t *ws_bytes, void *const *events,
                    void *stream);

/* Overlap of two layers' index sets, row by row: the statistic a search
 * for which layers keep an indexer is driven by (adjacent layers select
 * largely the same positions: IndexCache news article (app.myzaker.com),
 * section "IndexCache"; the F/S split of an existing model is chosen
 * greedily, layer by layer: IndexCache article after VentureBeat
 * (linkstar.cloud), section on the two deployment routes).
 *   a, b    device int32 index lists [B][T_q][top_k] (strides a_sb, a_st and
 *           b_sb, b_st in elements), each row ascending with -1 padding at
 *           the end, as idx_score_topk writes them.
 *   counts  device int32 [B*T_q]: counts[b*T_q + t] = number of positions
 *           (entries >= 0) present in both rows.
 * Status as for the other calls (LCSI_EINVAL for null pointers, negative
 * strides or sizes < 1; LCSI_EUNSUPPORTED for top_k > 2048; LCSI_EALIGN for
 * pointers not 4-byte aligned).  Asynchronous on `stream`; no workspace. */
int idx_overlap(const int32_t *a, int64_t a_sb, int64_t a_st,
                const int32_t *b, int64_t b_sb, int64_t b_st,
                int32_t B, int32_t T_q, int32_t top_k, int32_t *counts,
                void *stream);

/* Static description of a status code (never NULL). */
const char *lcsi_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* LCSI_H */
