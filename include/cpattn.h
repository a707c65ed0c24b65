/*
 * cpattn.h -- one GPU's share of context-parallel attention on MI355X (gfx950).
 *
 * C ABI of libcpattn.so.  The operation: causal, grouped-query, optionally
 * document-masked softmax attention of a chunk of queries against a chunk of
 * keys/values, computed blockwise and combined exactly through the per-row
 * log-sum-exp, forward and backward; plus drivers that run one rank's share of
 * the ring (P2P) and Ulysses (all-to-all) context-parallel schemes on a single
 * GPU, with the KV chunks that would travel between GPUs resident in HBM.
 *
 * Sources (the pages the method is described on):
 *   [MaxText] nougat.kr, "MaxText long-context training: KV parallelism":
 *     section "입력을 나눠도 KV가 다시 모이는 이유" (why the KV meets again) -- a
 *     causal query needs the KV of all earlier tokens; diagram text -- the
 *     sequence split and the All-gather / A2A / P2P data movement; section
 *     "헤드를 나누거나, KV를 돌리거나" (split the heads, or rotate the KV) -- heads
 *     are independent (A2A/Ulysses), the ring computes a partial result per
 *     visiting KV chunk and merges it, causal work must be balanced, USP =
 *     A2A group x ring.
 *   [Ulysses] aionda.blog, "Ulysses sequence parallelism for long-context
 *     training", section "현황" (current state) -- all-to-all from the token
 *     split to a head split, each GPU computing some of the heads.
 *   [Llama3] siliconandsystems.com, "Llama 3 parallelism", section "네
 *     병렬화는 서로 다른 자원을 확보하는 방식" -- context parallelism over packed
 *     documents must keep the document mask; section "긴 문맥은 어텐션 비용
 *     이상을 바꾸는 방식" -- balance work by actual attention compute.
 *
 * Definition (the pages state none; this is the plain reading).  Query head h
 * reads KV head h*hkv/hq (contiguous GQA groups).  Query i may attend key j iff
 * (not causal or pos_j <= pos_i) and (no docs or doc_j == doc_i), positions
 * being global token positions.  With s_ij = scale * <q_i, k_j>:
 *   lse_i = ln sum_{allowed j} exp(s_ij),  o_i = sum_{allowed j} exp(s_ij - lse_i) v_j,
 * and o_i = 0, lse_i = -inf when no key is allowed.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing except where a workspace is documented (it never
 *     calls hipMalloc; workspaces are caller-provided).
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and returns after enqueueing its kernels.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued, outputs are untouched, the call returns a
 *     negative cp_status and cp_last_error() describes it.  No C++ exception
 *     crosses the ABI.  CP_ERR_HIP reports a launch failure.
 *   - Layouts are token-major: q [L, *, d] with `q_stride` elements between
 *     consecutive tokens (so a head slice of a wider tensor is passed without
 *     a copy); k, v likewise with `kv_stride`; o, dout, dq [Lq, hq, d] and dk,
 *     dv [Lk, hkv, d] are contiguous.  lse and delta are [hq, Lq] fp32
 *     (natural log), row-major.
 *   - Supported: d in {64, 128}; hq % hkv == 0 with hq/hkv a power of two
 *     <= 64; 16-byte aligned pointers and strides (CP_ERR_ALIGN otherwise);
 *     token strides of at most 16 MiB and spans of at most 2^29 tokens
 *     (CP_ERR_UNSUPPORTED otherwise: the kernels address a tile of up to 128
 *     tokens, and a per-token fp32 row, through 32-bit byte offsets).
 *   - Document ids are int32 per local token, >= 0 and non-decreasing along
 *     global order (positions increase along a span's local order, so a
 *     span's ids are non-decreasing too).  The kernels rely on this: with ids
 *     that break it, tiles are classified from wrong id ranges and results
 *     are wrong (possibly not finite); memory accesses stay in bounds.  Set
 *     CP_CHECK_DOCS in cp_shape.flags to have every call that takes ids check
 *     them first (a host copy, so the call waits for its stream) and return
 *     CP_ERR_DOCS, with nothing enqueued, when an id is negative or
 *     decreases; cp_check_docs checks an array on its own.
 *   - Not thread-safe per stream: calls on one stream are ordered by the
 *     stream; calls that write the same outputs from different streams race.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CP_ABI_VERSION 2

typedef enum {
  CP_OK = 0,
  CP_ERR_ARG = -1,          /* invalid argument (null pointer, bad size or count) */
  CP_ERR_UNSUPPORTED = -2,  /* valid but not implemented (d, head ratio)          */
  CP_ERR_ALIGN = -3,        /* pointer or stride not 16-byte aligned             */
  CP_ERR_DOCS = -4,         /* doc ids for only one side, or (checked) ids < 0 or decreasing */
  CP_ERR_WORKSPACE = -5,    /* workspace missing or too small                     */
  CP_ERR_HIP = -6           /* a HIP launch failed                                */
} cp_status;

typedef enum { CP_BF16 = 0, CP_F32 = 1 } cp_dtype;

/* A chunk of tokens: up to two runs of global positions.  Local token
 * t < len[0] has position pos[0] + t; local token t >= len[0] has position
 * pos[1] + (t - len[0]).  Requires len[] >= 0 and, when len[1] > 0,
 * pos[1] >= pos[0] + len[0].  `doc` is NULL or a device array of len[0]+len[1]
 * int32 document ids.  A zigzag ring shard is exactly two runs.
 * [MaxText] diagram text: the sequence is split by tokens across chips. */
typedef struct {
  int64_t pos[2];
  int32_t len[2];
  const int32_t *doc;
} cp_span;

/* Shape and numerics shared by the calls of one layer's share. */
typedef struct {
  int32_t hq, hkv, d;   /* query heads, KV heads, head dim of this call            */
  int64_t q_stride;     /* elements between consecutive tokens of q (>= hq*d)      */
  int64_t kv_stride;    /* elements between consecutive tokens of k, v (>= hkv*d)  */
  float scale;          /* softmax scale on q.k (1/sqrt(d) in the usual reading)   */
  int32_t causal;       /* 1: mask keys after the query (diagonal included)       */
  cp_dtype dtype;       /* element type of q, k, v and dout                        */
  int32_t flags;        /* 0 or CP_CHECK_DOCS; other bits are CP_ERR_ARG           */
} cp_shape;

/* cp_shape.flags: check document ids before anything is enqueued
 * ([Llama3] "네 병렬화는 서로 다른 자원을 확보하는 방식": the document mask must
 * survive context parallelism, so ids that cannot describe packed documents
 * are refused rather than silently misread).  Costs a device-to-host copy of
 * the ids and a wait for the stream. */
#define CP_CHECK_DOCS 1

/* Forward attention of a Q chunk against one KV chunk: the partial result a
 * ring step produces before merging ([MaxText] "헤드를 나누거나, KV를 돌리거나").
 *   q: [Lq] tokens (q_stride), k, v: [Lk] tokens (kv_stride), Lq/Lk = span lengths.
 *   o: [Lq, hq, d] written in o_dtype (CP_F32 for a partial to be merged,
 *      CP_BF16 for a final output); lse: [hq, Lq] fp32 written.
 *   Rows with no allowed key get o = 0, lse = -inf.  qs.doc and ks.doc must be
 *   both NULL or both set (CP_ERR_DOCS).  bf16 inputs use bf16 MFMA with fp32
 *   accumulation; fp32 inputs use the fp64-accumulating precision path. */
cp_status cp_attn_chunk_fwd(const cp_shape *sh, const void *q, cp_span qs,
                            const void *k, const void *v, cp_span ks,
                            void *o, cp_dtype o_dtype, float *lse, void *stream);

/* In-place exact merge of a partial result into an accumulator
 * ([MaxText] "헤드를 나누거나, KV를 돌리거나": merge of partial results):
 *   L = ln(e^La + e^Lb);  O = e^(La-L) Oa + e^(Lb-L) Ob;  -inf is the identity.
 *   o_acc, o_part: [rows, h, d] fp32; lse_acc, lse_part: [h, rows] fp32.
 *   Weights are computed in fp64.  The two sets may not overlap. */
cp_status cp_lse_merge(int64_t rows, int32_t h, int32_t d, float *o_acc, float *lse_acc,
                       const float *o_part, const float *lse_part, void *stream);

/* Backward's row term: delta[h, r] = sum_e dout[r, h, e] * o[r, h, e], from the
 * FINAL (merged) output.  o, dout: [rows, h, d] in o_dtype / dout_dtype;
 * delta: [h, rows] fp32 written. */
cp_status cp_attn_delta(int64_t rows, int32_t h, int32_t d, const void *o, cp_dtype o_dtype,
                        const void *dout, cp_dtype dout_dtype, float *delta, void *stream);

/* Backward of one chunk pair from the saved FINAL lse and delta (P is
 * recomputed).  Accumulates (+=) into dq [Lq, hq, d], dk and dv [Lk, hkv, d],
 * all fp32: callers zero them first.  dout: [Lq, hq, d] in sh->dtype.
 * dk/dv are summed over the query heads of each KV group.  No atomics are
 * used: repeated calls on the same inputs give bitwise-identical results. */
cp_status cp_attn_chunk_bwd(const cp_shape *sh, const void *q, cp_span qs,
                            const void *k, const void *v, cp_span ks, const void *dout,
                            const float *lse, const float *delta,
                            float *dq, float *dk, float *dv, void *stream);

/* The two halves of cp_attn_chunk_bwd, same arguments and layouts: the
 * key-side gradients (dk, dv +=) and the query-side gradient (dq +=).  In a
 * ring the visiting chunk's dk/dv travel back to its owner, so computing them
 * first lets that transfer overlap the dq work. */
cp_status cp_attn_chunk_bwd_dkdv(const cp_shape *sh, const void *q, cp_span qs,
                                 const void *k, const void *v, cp_span ks, const void *dout,
                                 const float *lse, const float *delta,
                                 float *dk, float *dv, void *stream);
cp_status cp_attn_chunk_bwd_dq(const cp_shape *sh, const void *q, cp_span qs,
                               const void *k, const void *v, cp_span ks, const void *dout,
                               const float *lse, const float *delta, float *dq, void *stream);

/* Zigzag sharding for causal load balance ([MaxText] "헤드를 나누거나, KV를
 * 돌리거나" and [Llama3] "긴 문맥은...": later tokens see more context, so work
 * is balanced across ranks).  S tokens are cut into 2P chunks of c = S/(2P);
 * rank r holds chunks r and 2P-1-r.  Writes pos0 = {r*c, (2P-1-r)*c} and
 * len = {c, c}.  Host-only.  CP_ERR_ARG unless P >= 1, S % (2P) == 0,
 * 0 <= rank < P. */
cp_status cp_zigzag_layout(int64_t S, int32_t P, int32_t rank, int64_t pos0[2], int32_t len[2]);

/* Ring schedule ([MaxText] diagram text, P2P: pass the KV chunk to the
 * neighbour): at step s rank r holds the KV shard of rank (r - s) mod P.
 * kind[a*2 + b] classifies r's Q chunk a against the source's KV chunk b:
 * 0 skip (KV after Q), 1 diagonal (same chunk), 2 full (KV before Q).
 * Host-only. */
cp_status cp_ring_schedule(int64_t S, int32_t P, int32_t rank, int32_t step,
                           int32_t *src_rank, int8_t kind[4]);

/* Workspace bytes cp_ring_emulate needs for these arguments (0 on bad args). */
size_t cp_ring_workspace_bytes(const cp_shape *sh, int64_t S, int32_t P, int32_t rank,
                               cp_dtype o_dtype, int32_t backward);

/* One rank's share of ring (P2P) context parallelism, or every rank's
 * (rank = -1), with all shards resident on this GPU
 * ([MaxText] "헤드를 나누거나, KV를 돌리거나"; USP when q/k/v are head slices).
 * Inputs are in SHARDED order: the S rows hold rank 0's local shard (global
 * chunks 0 and 2P-1), then rank 1's (chunks 1 and 2P-2), and so on; q uses
 * sh->q_stride, k and v sh->kv_stride; doc is NULL or [S] int32 in the same
 * order.  For each step s the rank's Q shard attends the KV shard of rank
 * (r - s) mod P (one chunk-attention call with both shards as two-run spans;
 * skip blocks are skipped tile by tile) and the fp32 partial is merged into
 * the running (O, LSE).  Outputs:
 *   rank >= 0: o [2c, hq, d] (o_dtype), lse [hq, 2c];
 *   rank = -1: o [S, hq, d] in sharded order, lse [P, hq, 2c] (rank blocks).
 * step_o [P, 2c, hq, d] fp32 and step_lse [P, hq, 2c] (rank >= 0 only; both
 * NULL to skip) receive each step's partial before it is merged.
 * If dout (like o, in sh->dtype) is non-NULL the backward runs too: delta from
 * the final o, then each step's chunk backward with the final lse.  dq (like
 * o, fp32) is written; dk, dv ([S, hkv, d] fp32, sharded order) are written
 * with this rank's query rows' contributions, each in the visiting rank's rows
 * (what a real ring carries back to the KV owners), or the full gradients for
 * rank = -1.  The workspace (>= cp_ring_workspace_bytes, 256-byte aligned) is
 * scratch owned by the caller. */
cp_status cp_ring_emulate(const cp_shape *sh, int64_t S, int32_t P, int32_t rank,
                          const void *q, const void *k, const void *v, const int32_t *doc,
                          void *o, cp_dtype o_dtype, float *lse,
                          const void *dout, float *dq, float *dk, float *dv,
                          float *step_o, float *step_lse,
                          void *workspace, size_t ws_bytes, void *stream);

/* cp_ring_emulate under an explicit two-chunks-per-rank layout instead of
 * zigzag ([Llama3] "긴 문맥은 어텐션 비용 이상을 바꾸는 방식": with packed
 * documents the ranks are balanced by attention work, e.g. by the pairing
 * cp_balanced_pairs returns).  chunks: HOST array of 2P int32, rank r holds
 * the S/(2P)-token chunks chunks[2r] < chunks[2r+1], each chunk exactly once
 * (CP_ERR_ARG otherwise); the zigzag table is chunks = {r, 2P-1-r}.  Inputs
 * are in the sharded order of this layout (rank 0's two chunks, then rank
 * 1's, ...); step s still brings rank (r - s) mod P's shard.  Outputs,
 * workspace (cp_ring_workspace_bytes) and everything else as for
 * cp_ring_emulate, without per-step capture. */
cp_status cp_ring_emulate_layout(const cp_shape *sh, int64_t S, int32_t P, int32_t rank, const int32_t *chunks,
                                 const void *q, const void *k, const void *v, const int32_t *doc,
                                 void *o, cp_dtype o_dtype, float *lse,
                                 const void *dout, float *dq, float *dk, float *dv,
                                 void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes cp_ring_emulate_overlap needs (0 on bad args). */
size_t cp_ring_overlap_workspace_bytes(const cp_shape *sh, int64_t S, int32_t P,
                                       cp_dtype o_dtype, int32_t backward);

/* cp_ring_emulate for one rank (rank >= 0, no per-step capture) with the
 * ring's traffic emulated on a second stream, so that its cost beside the
 * compute can be measured ([MaxText] diagram text, P2P: each GPU computes with
 * the chunk it holds while the next one arrives; section "헤드를 나누거나,
 * KV를 돌리거나": the ring can overlap communication with computation).  Step
 * s >= 1 of the forward and of the backward reads its KV shard from a
 * double-buffered receive area in the workspace, filled on copy_stream one
 * step ahead (a strided copy of the shard's rows, i.e. what the neighbour
 * sends); after each backward step the shard's dK, dV rows are copied into a
 * send area on copy_stream (what goes back to the owner).  Events order the
 * copies against the compute; when the work queued on `stream` completes, so
 * has the copy work.  Outputs are bitwise those of cp_ring_emulate for the
 * same rank.  copy_stream must differ from stream (both at the default
 * priority).  Workspace: >= cp_ring_overlap_workspace_bytes, 256-byte
 * aligned, caller-owned; calls that share a workspace must not overlap. */
cp_status cp_ring_emulate_overlap(const cp_shape *sh, int64_t S, int32_t P, int32_t rank,
                                  const void *q, const void *k, const void *v, const int32_t *doc,
                                  void *o, cp_dtype o_dtype, float *lse,
                                  const void *dout, float *dq, float *dk, float *dv,
                                  void *workspace, size_t ws_bytes, void *stream, void *copy_stream);

/* Workspace bytes cp_ulysses_share needs (0 on bad args). */
size_t cp_ulysses_workspace_bytes(const cp_shape *sh_full, int64_t S, int32_t sp, int32_t backward);

/* One rank's share of Ulysses (all-to-all) sequence parallelism
 * ([Ulysses] "현황"; [MaxText] diagram text, A2A): after the all-to-all each
 * of sp ranks holds the whole sequence for hq/sp query heads and hkv/sp KV
 * heads (sp must divide both: the KV heads bound the degree), so its share is
 * full-sequence attention for that head slice.  sh_full describes the full
 * layer: q [S, hq, d] with q_stride, k/v [S, hkv, d] with kv_stride, global
 * order; doc NULL or [S].  The share's heads are read in place (no copy).
 * Outputs for the share: o [S, hq/sp, d] (o_dtype), lse [hq/sp, S]; with
 * dout [S, hq/sp, d] non-NULL: dq [S, hq/sp, d], dk and dv [S, hkv/sp, d]
 * (fp32, written). */
cp_status cp_ulysses_share(const cp_shape *sh_full, int64_t S, int32_t sp, int32_t sp_rank,
                           const void *q, const void *k, const void *v, const int32_t *doc,
                           void *o, cp_dtype o_dtype, float *lse,
                           const void *dout, float *dq, float *dk, float *dv,
                           void *workspace, size_t ws_bytes, void *stream);

/* Size of the device scratch built into the library for
 * cp_ulysses_share_noalloc (per GPU, held until the process ends). */
#define CP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* cp_ulysses_share for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments and results, bitwise, without the workspace.  The
 * backward's Delta rows ((hq/sp) * S fp32) go to a scratch array built into
 * the library, CP_NOALLOC_SCRATCH_BYTES per GPU; larger shares get
 * CP_ERR_WORKSPACE.  The call allocates nothing (no hipMalloc, no library
 * allocation); the scratch's device address is looked up once per GPU on the
 * first call there.  Every call on one GPU shares that GPU's scratch: calls
 * that overlap on one GPU (different streams, or threads) race and must be
 * ordered by the caller.  Delta is written in full before it is read, so
 * nothing depends on what an earlier call left there.  CP_CHECK_DOCS is
 * refused (CP_ERR_ARG): it copies ids to the host and waits; run
 * cp_check_docs beforehand instead. */
cp_status cp_ulysses_share_noalloc(const cp_shape *sh_full, int64_t S, int32_t sp, int32_t sp_rank,
                                   const void *q, const void *k, const void *v, const int32_t *doc,
                                   void *o, cp_dtype o_dtype, float *lse,
                                   const void *dout, float *dq, float *dk, float *dv, void *stream);

/* Workspace bytes cp_allgather_share needs (0 on bad args). */
size_t cp_allgather_workspace_bytes(const cp_shape *sh, int64_t S, int32_t P, int32_t has_doc, int32_t backward);

/* One rank's share of all-gather context parallelism ([MaxText] diagram text,
 * All-gather; section "입력을 나눠도 KV가 다시 모이는 이유": causal queries
 * need every earlier token's KV): the rank keeps its zigzag query shard and
 * gathers the KV of the whole sequence, so its share is one chunk attention
 * of its two query runs against all S keys.
 *   q: the rank's 2c = S/P query rows in local order (chunks rank and
 *      2P-1-rank; q_stride); k, v: [S, hkv, d] in GLOBAL order (kv_stride);
 *   doc: NULL or [S] int32 in global order (device).
 *   Outputs: o [2c, hq, d] (o_dtype), lse [hq, 2c]; with dout [2c, hq, d]
 *   non-NULL: dq [2c, hq, d] and dk, dv [S, hkv, d] (fp32, written) -- dk, dv
 *   hold this rank's query rows' contributions (a real job reduce-scatters
 *   them).  workspace >= cp_allgather_workspace_bytes, 256-byte aligned. */
cp_status cp_allgather_share(const cp_shape *sh, int64_t S, int32_t P, int32_t rank,
                             const void *q, const void *k, const void *v, const int32_t *doc,
                             void *o, cp_dtype o_dtype, float *lse,
                             const void *dout, float *dq, float *dk, float *dv,
                             void *workspace, size_t ws_bytes, void *stream);

/* Checks n document ids: each >= 0 and none smaller than the one before
 * ([Llama3] "네 병렬화는 서로 다른 자원을 확보하는 방식": packed documents keep
 * their mask).  doc: a HOST array if on_host != 0, else a device array that
 * is copied to the host on `stream` (the call then waits for the stream).
 * CP_OK, or CP_ERR_DOCS naming the first offending index; CP_ERR_ARG for
 * n < 0 or a NULL doc with n > 0. */
cp_status cp_check_docs(const int32_t *doc, int64_t n, int32_t on_host, void *stream);

/* Causal work of the 2P chunks of a sequence ([Llama3] "긴 문맥은 어텐션
 * 비용 이상을 바꾸는 방식": balance ranks by attention compute, not tokens):
 * work[i] = the number of allowed (query, key) pairs whose query lies in
 * chunk i (tokens [i*S/(2P), (i+1)*S/(2P))), under the causal mask and, if
 * doc (HOST array of S int32, non-decreasing, >= 0) is given, the document
 * mask.  work: HOST array of 2P.  CP_ERR_ARG unless P >= 1 and S > 0 is a
 * multiple of 2P; CP_ERR_DOCS for ids that are negative or decrease.
 * Host-only. */
cp_status cp_chunk_work(int64_t S, int32_t P, const int32_t *doc, int64_t *work);

/* Document-aware alternative to the zigzag layout: assigns the 2P chunks two
 * per rank so that the largest rank's work (cp_chunk_work) is as small as
 * possible -- the k-th lightest chunk goes with the k-th heaviest, optimal
 * for two chunks per rank.  Writes chunks[2r] < chunks[2r+1] (HOST, 2P
 * entries) and rank_work[r] (HOST, P entries).  With no documents the result
 * is the zigzag pairing.  Host-only; errors as cp_chunk_work. */
cp_status cp_balanced_pairs(int64_t S, int32_t P, const int32_t *doc, int32_t *chunks, int64_t *rank_work);

/* Emulated Ulysses all-to-all, forward direction ([Ulysses] "현황";
 * [MaxText] diagram text, A2A): from the token split to the head split.
 * The sp ranks' token shards are resident together in x [S, h, d] (rank j's
 * shard is rows [j*S/sp, (j+1)*S/sp); consecutive tokens x_stride elements
 * apart); rank `rank` receives every token of its heads into y [S, h_out, d]
 * (contiguous):
 *   h % sp == 0:  h_out = h/sp,  y[s, i] = x[s, rank*h/sp + i];
 *   sp % h == 0:  h_out = 1,     y[s, 0] = x[s, rank*h/sp]  (more ranks than
 *                 heads -- KV heads under GQA: each of the sp/h ranks that
 *                 share a KV head receives its own copy).
 * elt_bytes: 2 (bf16) or 4 (fp32).  S must be a multiple of sp; d*elt_bytes
 * and x_stride*elt_bytes multiples of 16; pointers 16-byte aligned.  A copy
 * bound by HBM bandwidth.  Errors as for every call (nothing enqueued). */
cp_status cp_a2a_tokens_to_heads(int64_t S, int32_t h, int32_t d, int32_t elt_bytes, int32_t sp, int32_t rank,
                                 const void *x, int64_t x_stride, void *y, void *stream);

/* The reverse exchange (the attention output going back to the token split):
 * rank `rank`'s head-split result o [S, h/sp, d] (contiguous) is written into
 * the token-split tensor z [S, h, d] (token stride z_stride):
 *   z[s, rank*h/sp + i] = o[s, i].
 * Called for every rank it assembles z, whose rows [j*S/sp, ...) are what rank
 * j holds after the exchange.  h must be a multiple of sp. */
cp_status cp_a2a_heads_to_tokens(int64_t S, int32_t h, int32_t d, int32_t elt_bytes, int32_t sp, int32_t rank,
                                 const void *o, void *z, int64_t z_stride, void *stream);

/* Debug dump of the tile classification that drives tile skipping: out
 * [ceil(Lq/bq), ceil(Lk/bk)] int8 (device), 0 = no allowed entry (skipped),
 * 1 = every entry allowed (no element mask), 2 = otherwise.  Entries outside
 * [0,Lq) x [0,Lk) are ignored.  Exact for spans of up to two runs. */
cp_status cp_tile_map(const cp_shape *sh, cp_span qs, cp_span ks, int32_t bq, int32_t bk,
                      int8_t *out, void *stream);

/* Message of the last failed call on this thread ("" if none). */
const char *cp_last_error(void);

/* CP_ABI_VERSION of the loaded library. */
int32_t cp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
