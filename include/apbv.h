/*
 * apbv.h - C ABI of the APB-V / Spava approximate-attention prefill for MI355X (gfx950).
 *
 * The method ("APB-V: Accelerating Long-Video Understanding via Sequence-Parallelism-aware
 * Approximate Attention", also published as "Spava"; technical summary on gist.science,
 * section Metodologia) splits the prefill input into an anchor block B_a, context blocks
 * B^(h) and a query block B_qr. For every context block the hot path
 *   1. scores the block's keys against the query block and keeps, per KV head, the l_p
 *      highest-scoring key/value pairs as the block's passing block  (apbv_score_select),
 *   2. collects the anchor and the passing blocks of all blocks into one prefix per KV head
 *      (apbv_gather_passing),
 *   3. runs attention of the block's rows over [anchor | passing blocks of the preceding
 *      blocks | the block's own keys, causal]                        (apbv_approx_attn_prefill).
 * apbv_prefill_layer runs the three steps in one call, optionally with the selection of later
 * blocks on a second stream beside the attention. The rows of the query block itself, which
 * see the whole sequence, come from apbv_query_forward; apbv_layer_forward yields every row
 * of a layer (anchor, context and query rows) in one call.
 * All virtual blocks of the method's sequence-parallel layout live on one GPU; ZigZag
 * pairing of block p with block n-1-p (same page, "Suddivisione del Contesto e
 * Disposizione ZigZag" and "Bilanciamento del Carico dell'Attenzione Approssimata") is the
 * work schedule of step 3.
 *
 * Conventions shared by every call
 *  - Tensors are bf16 (raw bit patterns, apbv_bf16) or fp32 / int32, in device memory,
 *    owned by the caller. The library never allocates, frees or synchronises; every call
 *    enqueues its kernels on `stream` (a hipStream_t, NULL = the default stream) and
 *    returns. Kernel faults surface at the caller's next synchronisation.
 *  - Token-major layouts: q [tokens, hq, d], k/v [tokens, hkv, d]. The row stride (elements
 *    between consecutive tokens) of q_ctx and of k_ctx/v_ctx may be larger than hq*d /
 *    hkv*d (for a fused QKV buffer); all other tensors are contiguous.
 *  - Device pointers and row strides must give 16-byte aligned rows.
 *  - Query head h uses KV head h / (hq / hkv).
 *  - `block_starts` is HOST memory: n_blocks + 1 strictly increasing offsets, block_starts[0]
 *    = 0, block_starts[n_blocks] = N (context tokens; anchor and query block excluded).
 *  - Every argument is validated before anything is enqueued; on error nothing is launched
 *    and the call returns a non-zero apbv_status (apbv_last_error() gives details for the
 *    calling thread). A failed launch returns APBV_EHIP (apbv_prefill_layer may have
 *    enqueued its earlier launches by then).
 *  - Calls on one stream may be issued from several threads; the library keeps no mutable
 *    global state apart from the per-thread error message, and the per-device scratch of
 *    apbv_score_select_noalloc (with its address, looked up once per device).
 */
#ifndef APBV_H
#define APBV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t apbv_bf16;   /* raw bf16 bits */
typedef int32_t apbv_status;

#define APBV_OK 0
#define APBV_EINVAL 1          /* malformed argument (null pointer, bad sizes, misalignment) */
#define APBV_EUNSUPPORTED 2    /* well-formed but outside what the kernels implement */
#define APBV_EWORKSPACE 3      /* workspace missing or too small */
#define APBV_EHIP 4            /* a HIP launch or query failed */

#define APBV_MAX_BLOCKS 64     /* block_starts travels in kernel arguments */

typedef struct apbv_layout {
  int32_t n_blocks;            /* virtual context blocks, 1..APBV_MAX_BLOCKS */
  const int32_t* block_starts; /* HOST [n_blocks + 1] */
  int32_t l_anchor;            /* anchor rows (>= 0) */
  int32_t l_query;             /* query-block rows used for scoring (>= 0) */
  int32_t l_pass;              /* passing rows per block and KV head, 0..min block length */
  int32_t hq, hkv;             /* query heads and KV heads, hq % hkv == 0 */
  int32_t head_dim;            /* 64 or 128 */
  float scale;                 /* softmax scale; 0 means 1/sqrt(head_dim) */
  int32_t zigzag;              /* 1: ZigZag bucket schedule, 0: block order (same results) */
  int64_t q_row_stride;        /* elements between tokens of q_ctx; 0 means hq*head_dim */
  int64_t kv_row_stride;       /* elements between tokens of k_ctx, v_ctx; 0 means hkv*head_dim;
                                  below 2^22 */
} apbv_layout;

/* Workspace bytes needed by apbv_score_select for this layout (written to *bytes). */
apbv_status apbv_score_select_workspace(const apbv_layout* layout, size_t* bytes);

/*
 * Step 1: passing-block selection (gist.science summary, Metodologia part 1, "Meccanismo di
 * Attenzione Approssimata", passing blocks chosen by query-to-context attention scores).
 *
 * For block v, KV head g and every context row j of block v:
 *   scores[g, j] = sum over the G = hq/hkv heads h of group g and the l_query query rows i of
 *                  softmax over the keys j' of block v of (scale * q_query[i,h] . k_ctx[j',g])
 * (each block's scores sum to G * l_query), computed in fp32 from bf16 inputs with a fixed
 * reduction order (bitwise reproducible). sel[v, g, :] receives the l_pass rows of block v
 * with the largest scores, ties to the lower row, as absolute context rows in ascending order.
 * G * l_query is limited by LDS (about 32000 score rows at head_dim 128; larger gives
 * APBV_EUNSUPPORTED).
 *
 *   q_query   [l_query, hq, d] bf16, contiguous
 *   k_ctx     [N, hkv, d] bf16 (kv_row_stride)
 *   scores    [hkv, N] fp32 out, or NULL (then kept in the workspace)
 *   sel       [n_blocks, hkv, l_pass] int32 out
 *   workspace device buffer of at least apbv_score_select_workspace() bytes, 256-byte
 *             aligned: split row statistics, the score rows packed per KV head, and the
 *             scores when `scores` is NULL (no initialisation needed; calls that overlap in
 *             time must not share it)
 */
apbv_status apbv_score_select(const apbv_layout* layout, const apbv_bf16* q_query,
                              const apbv_bf16* k_ctx, float* scores, int32_t* sel,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Step 1 without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same kernels and
 * results as apbv_score_select; the workspace is a 16 MiB scratch array inside the library,
 * one per device, held until the process ends. Nothing is allocated or freed by the call.
 *
 *   q_query, k_ctx, scores, sel, stream: as apbv_score_select (stream must belong to the
 *   calling thread's current device, whose scratch is used)
 * A layout needing more than 16 MiB (apbv_score_select_workspace() with scores given, or
 * with scores NULL when they are kept in the scratch) returns APBV_EUNSUPPORTED before
 * anything is enqueued. The scratch keeps the last call's contents (every call writes what
 * it reads); calls that overlap in time on one device (several streams or threads) race on
 * it and must be ordered by the caller.
 */
apbv_status apbv_score_select_noalloc(const apbv_layout* layout, const apbv_bf16* q_query,
                                      const apbv_bf16* k_ctx, float* scores, int32_t* sel,
                                      void* stream);

/*
 * Step 2: collect anchor and passing blocks (same page and part: every host gathers the
 * passing blocks of the hosts before it; on one GPU all of them sit in one prefix buffer).
 *   k_pre[g] = k_anchor[:, g] ++ k_ctx[sel[0, g], g] ++ ... ++ k_ctx[sel[n-1, g], g]
 * and the same for v. Block v later reads rows [0, l_anchor + v*l_pass) of its KV head.
 *
 *   k_anchor, v_anchor [l_anchor, hkv, d] bf16, contiguous (may be NULL if l_anchor == 0)
 *   k_ctx, v_ctx       [N, hkv, d] bf16 (kv_row_stride)
 *   sel                [n_blocks, hkv, l_pass] int32; every entry of sel[v] must be a row
 *                      of block v, i.e. in [block_starts[v], block_starts[v+1])
 *   k_pre, v_pre       [hkv, l_anchor + n_blocks*l_pass, d] bf16 out
 *   sel_errors         device int32 counter, or NULL: the number of sel entries outside
 *                      their own block is ADDED to it (the caller zeroes it beforehand and
 *                      reads it after the stream has reached this call)
 * An entry outside its block is an error of the caller; it is counted into sel_errors when
 * one is given, and is clamped into its block (the first or last row) so that no read leaves
 * the context: the prefix row it produces is then meaningless but memory stays safe.
 */
apbv_status apbv_gather_passing(const apbv_layout* layout, const apbv_bf16* k_anchor,
                                const apbv_bf16* v_anchor, const apbv_bf16* k_ctx,
                                const apbv_bf16* v_ctx, const int32_t* sel, apbv_bf16* k_pre,
                                apbv_bf16* v_pre, int32_t* sel_errors, void* stream);

/*
 * Step 3: approximate attention of the context rows (same page and part: attention over
 * anchor, passing blocks and local context; "Limitazioni": with one block it is plain
 * flash attention). Row i of block v, head h, KV head g sees
 *   k_pre[g, 0 : l_anchor + v*l_pass]  (all visible)  then  k_ctx[block_starts[v] .. i, g]
 * (causal, diagonal included), softmax in fp32 with scale, bf16 MFMA products:
 *   out[i, h, :] = softmax(scale * q_ctx[i,h] . keys) @ values        (bf16, round-to-nearest)
 *   lse[h, i]    = natural-log log-sum-exp of the scaled logits         (fp32, optional)
 *
 *   q_ctx        [N, hq, d] bf16 (q_row_stride)
 *   k_pre, v_pre [hkv, l_anchor + n_blocks*l_pass, d] bf16 (from apbv_gather_passing)
 *   k_ctx, v_ctx [N, hkv, d] bf16 (kv_row_stride)
 *   out          [N, hq, d] bf16 out, contiguous
 *   lse          [hq, N] fp32 out, or NULL
 *   range_begin, range_end: the part of the work to run. With zigzag = 1 these are ZigZag
 *     buckets (bucket p = blocks p and n-1-p, apbv_num_buckets() of them), with zigzag = 0
 *     blocks. (0, 0) runs everything. Rows outside the range are left untouched.
 * With n_blocks = 1, l_anchor = 0 and l_pass = 0 this is dense causal attention.
 */
apbv_status apbv_approx_attn_prefill(const apbv_layout* layout, const apbv_bf16* q_ctx,
                                     const apbv_bf16* k_pre, const apbv_bf16* v_pre,
                                     const apbv_bf16* k_ctx, const apbv_bf16* v_ctx,
                                     apbv_bf16* out, float* lse, int32_t range_begin,
                                     int32_t range_end, void* stream);

/*
 * One layer of steps 1-3 with the selection and gather of later blocks overlapped with
 * attention (same page, Metodologia, "Comunicazione Sovrapposta": moving the passing blocks
 * runs beside the attention computation; on one GPU the producer of the passing blocks is
 * the scoring, selection and gather of the later blocks). Results are bit-identical to
 * apbv_score_select + apbv_gather_passing + apbv_approx_attn_prefill over the same buffers.
 *
 *   q_query, k_ctx, scores, sel, workspace, workspace_bytes: as apbv_score_select
 *   k_anchor, v_anchor, v_ctx, k_pre, v_pre:                 as apbv_gather_passing
 *   q_ctx, out, lse:                                         as apbv_approx_attn_prefill
 *   stream      hipStream_t all work is ordered on: on return the whole layer is enqueued
 *               there (work on the aux stream is joined back into it)
 *   aux_stream  a second hipStream_t of the same device, or NULL (then the three steps run
 *               in order on stream)
 *   ready_event, done_event  two hipEvent_t of the device, owned by the caller, recorded by
 *               this call (needed with aux_stream; calls that overlap in time must not share
 *               them)
 *   compute_units  CUs the split is planned for; 0 = the current device's count (other
 *               values only move the split, never the results)
 * With aux_stream, stream runs: selection and gather of blocks [0, early), attention of
 * buckets [late, n_buckets), then (after the aux stream) attention of buckets [0, late);
 * aux_stream runs the selection and gather of blocks [early, n) beside the first attention
 * launch. (late, early) come from apbv_prefill_layer_plan with compute_units.
 */
apbv_status apbv_prefill_layer(const apbv_layout* layout, const apbv_bf16* q_query,
                               const apbv_bf16* q_ctx, const apbv_bf16* k_ctx,
                               const apbv_bf16* v_ctx, const apbv_bf16* k_anchor,
                               const apbv_bf16* v_anchor, float* scores, int32_t* sel,
                               apbv_bf16* k_pre, apbv_bf16* v_pre, apbv_bf16* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream,
                               void* aux_stream, void* ready_event, void* done_event,
                               int32_t compute_units);

/*
 * Host only: the split apbv_prefill_layer uses on a device with compute_units CUs.
 * Attention of ZigZag buckets [late, n_buckets) needs the selections of blocks [0, early)
 * only (bucket b holds blocks b and n-1-b, so early = n-1-late); late is the largest bucket
 * index whose late set of workgroups fills whole rounds of the compute units (one attention
 * workgroup per CU at a time), else 0 with early = n-1. With l_pass = 0, or zigzag = 0 (a
 * late block set always contains the last block), late = 0; early = 0 when l_pass = 0.
 */
apbv_status apbv_prefill_layer_plan(const apbv_layout* layout, int32_t compute_units,
                                    int32_t* late_bucket_begin, int32_t* early_blocks);

/* Workspace bytes needed by apbv_query_forward for this layout (written to *bytes; 0 when
 * l_query is 0). */
apbv_status apbv_query_forward_workspace(const apbv_layout* layout, size_t* bytes);

/*
 * Rows of the query block (same page, part 2, "Forward Fuso di Contesto e Query": the
 * query runs in the same forward as the context and its partial results over different key
 * sets are merged through their log-sum-exp). The query block closes the sequence
 * [anchor | context | query block], so its rows are exact: row i of head h (KV head g) sees
 *   k_anchor[:, g]  ++  k_ctx[0 .. N-1, g]  ++  k_query[0 .. i, g]
 *   out[i, h, :] = softmax(scale * q_query[i,h] . keys) @ values       (bf16, round-to-nearest)
 *   lse[h, i]    = natural-log log-sum-exp of the scaled logits         (fp32, optional)
 * computed as partial results over chunks of 1024-8192 keys (bf16 MFMA, fp32 softmax; the
 * chunk length depends only on the layout), merged in a second kernel.
 *
 *   q_query          [l_query, hq, d] bf16, contiguous
 *   k_query, v_query [l_query, hkv, d] bf16, contiguous
 *   k_anchor, v_anchor [l_anchor, hkv, d] bf16, contiguous (may be NULL if l_anchor == 0)
 *   k_ctx, v_ctx     [N, hkv, d] bf16 (kv_row_stride)
 *   out              [l_query, hq, d] bf16 out, contiguous
 *   lse              [hq, l_query] fp32 out, or NULL
 *   workspace        device buffer of at least apbv_query_forward_workspace() bytes,
 *                    256-byte aligned (partial outputs; contents need no initialisation)
 * With l_query == 0 nothing is launched.
 */
apbv_status apbv_query_forward(const apbv_layout* layout, const apbv_bf16* q_query,
                               const apbv_bf16* k_query, const apbv_bf16* v_query,
                               const apbv_bf16* k_anchor, const apbv_bf16* v_anchor,
                               const apbv_bf16* k_ctx, const apbv_bf16* v_ctx, apbv_bf16* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Every row of one layer in one call: the anchor rows, the context rows (steps 1-3) and the
 * query rows, all on one stream, in that order. The page's sequence is [anchor | context
 * blocks | query block] (Metodologia, "Suddivisione del Contesto e Disposizione ZigZag");
 * the anchor opens it, so its rows are dense causal attention over the anchor alone (the
 * case "Limitazioni" names: one block is plain attention), computed by the same kernel as
 * the context rows with one block, no prefix. Context rows are bit-identical to
 * apbv_score_select + apbv_gather_passing + apbv_approx_attn_prefill and query rows to
 * apbv_query_forward over the same buffers.
 *
 * Fields of apbv_layer_io (shapes as in the calls named):
 *   q_anchor     [l_anchor, hq, d] bf16, contiguous (needed when anchor_out is set)
 *   k_anchor, v_anchor, k_ctx, v_ctx, k_pre, v_pre, sel:   as apbv_gather_passing
 *   q_ctx, out, lse:                                       as apbv_approx_attn_prefill
 *   q_query, scores:                                       as apbv_score_select
 *   k_query, v_query, query_out, query_lse:   as apbv_query_forward's k/v_query, out, lse
 *   anchor_out   [l_anchor, hq, d] bf16 out, contiguous; NULL skips the anchor rows
 *   anchor_lse   [hq, l_anchor] fp32 out, or NULL
 *   query_out    NULL skips the query rows (then k_query, v_query may be NULL)
 *   workspace    device buffer of at least apbv_layer_workspace() bytes, 256-byte aligned
 *                (scoring statistics, scores when `scores` is NULL, query partials; no
 *                initialisation needed; calls that overlap in time must not share it)
 * Everything is validated before the first launch; an error launches nothing.
 */
typedef struct apbv_layer_io {
  const apbv_bf16* q_anchor;
  const apbv_bf16* k_anchor;
  const apbv_bf16* v_anchor;
  const apbv_bf16* q_ctx;
  const apbv_bf16* k_ctx;
  const apbv_bf16* v_ctx;
  const apbv_bf16* q_query;
  const apbv_bf16* k_query;
  const apbv_bf16* v_query;
  float* scores;
  int32_t* sel;
  apbv_bf16* k_pre;
  apbv_bf16* v_pre;
  apbv_bf16* anchor_out;
  float* anchor_lse;
  apbv_bf16* out;
  float* lse;
  apbv_bf16* query_out;
  float* query_lse;
  void* workspace;
  size_t workspace_bytes;
} apbv_layer_io;

/* Workspace bytes needed by apbv_layer_forward for this layout (written to *bytes). */
apbv_status apbv_layer_workspace(const apbv_layout* layout, size_t* bytes);

apbv_status apbv_layer_forward(const apbv_layout* layout, const apbv_layer_io* io,
                               void* stream);

/* Number of schedulable ranges: ZigZag buckets (ceil(n/2)) if zigzag, else n_blocks.
 * Returns -1 for an invalid layout. Host only. */
int32_t apbv_num_buckets(const apbv_layout* layout);

/* Host-only view of the attention work list for [range_begin, range_end): *count receives
 * the number of work units; if `units` is non-NULL and capacity >= *count, unit u is
 * written as 4 ints {block_a, tile_a, block_b, tile_b} (-1 when a unit has one part).
 * Tile t of block v is context rows [bs[v] + t*rows, min(bs[v] + (t+1)*rows, bs[v+1])) with
 * rows = apbv_attn_tile_rows(head_dim). Every unit is launched for all hq heads. */
apbv_status apbv_schedule(const apbv_layout* layout, int32_t range_begin, int32_t range_end,
                          int32_t* units, int32_t capacity, int32_t* count);

/* Query rows per attention work tile for a head dimension (0 if unsupported). */
int32_t apbv_attn_tile_rows(int32_t head_dim);

const char* apbv_status_str(apbv_status status);
/* Detail of the calling thread's most recent failed call ("" if none). */
const char* apbv_last_error(void);
/* Library version string. */
const char* apbv_version(void);

#ifdef __cplusplus
}
#endif
#endif /* APBV_H */
