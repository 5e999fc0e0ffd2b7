/*
 * cpattn.h - C ABI of libcpattn: one context-parallel rank's share of ring
 * attention on MI355X (gfx950).
 *
 * The operation (compassingai.com context-parallelism page, section "數學基礎"
 * and section "線上 Softmax"): rank i of a ring of N holds the query shard
 * Q_i of L = S/N contiguous tokens; it visits the key/value blocks K_j, V_j of
 * every rank in ring order and keeps, per query row, a running max m, a
 * running sum l and an unnormalised output O, merged block by block with the
 * online-softmax recurrence; at the end O/l is the attention output and
 * (m, l), lse = m + ln l are exported.  Masks: none (bidirectional), causal
 * (key c visible to query p iff c <= p; blocks j > i are skipped and the
 * diagonal block j = i is triangular - section "因果掩碼的特殊處理" of the same
 * page) and packed documents with causal order (visible iff
 * doc_start(p) <= c <= p, document boundaries kept across shards - the
 * process-cxr.github.io page, sections "配置关注点" and "常见失败模式").
 *
 * Conventions for every entry point
 *  - Tensors are caller-owned DEVICE memory, contiguous, row-major:
 *      Q, K_j, V_j, out, O-state, partial O:   [B, L, H, d]
 *      m, l, lse (state, outputs, partials):   [B, H, L]   (float32)
 *    Q/K/V/out element type is desc->dtype (CP_F32: float32, CP_BF16:
 *    bfloat16); running state, partial outputs, m, l and lse are float32.
 *    Tensor base pointers must be 16-byte aligned; float32 vectors of
 *    [B, H, L] must be 4-byte aligned.
 *  - Host arrays (cu_seqlens, block pointer tables, merge order) are read
 *    during the call only; the library keeps no pointer to them.
 *  - Streams are hipStream_t passed as void* (NULL = the default stream).
 *  - Calls are asynchronous: CP_OK means every argument was validated and the
 *    work was enqueued.  All validation happens before anything is enqueued;
 *    on a validation error nothing is enqueued.  A HIP launch failure returns
 *    CP_ERR_HIP (work enqueued before it may remain in the stream).  Device
 *    faults surface at the caller's next synchronisation.
 *  - No exception or abort crosses the ABI.  On an error, cp_attn_last_error()
 *    returns a message for the calling thread.
 *  - The library allocates no device memory: scratch comes from the caller's
 *    workspace (see cp_attn_workspace_bytes).
 *
 * Readings of points the pages leave open:
 *  - the diagonal is visible under the causal mask (c <= p);
 *  - a row that sees no key of a block has m = -inf, l = 0, lse = -inf and a
 *    zero partial output; merging ignores it; finalising l = 0 gives O = 0;
 *  - m is in natural-log units (the max of score * scale), l = sum exp(s - m);
 *  - softmax scale defaults to 1/sqrt(d);
 *  - cu_seqlens are global token positions over the whole sequence S = N L.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CP_OK = 0,
  CP_ERR_INVALID_ARG = 1,   /* a null/misaligned pointer, bad shape, bad index, malformed cu_seqlens */
  CP_ERR_UNSUPPORTED = 2,   /* a valid request this library does not implement (e.g. d not in {64,128}) */
  CP_ERR_WORKSPACE = 3,     /* workspace missing or smaller than cp_attn_workspace_bytes() */
  CP_ERR_HIP = 4            /* a HIP runtime call failed; the message names it */
} cp_status;

typedef enum { CP_MASK_NONE = 0, CP_MASK_CAUSAL = 1, CP_MASK_DOC_CAUSAL = 2 } cp_mask;
typedef enum { CP_F32 = 0, CP_BF16 = 1 } cp_dtype;

/* Modes of cp_attn_block_partial. */
typedef enum {
  CP_MODE_INIT = 0,         /* state := (O, m, l) of this block alone */
  CP_MODE_ACCUMULATE = 1,   /* state := online merge of state and this block */
  CP_MODE_PARTIAL_LSE = 2   /* o_part := normalised O of this block alone, lse_part := its lse */
} cp_block_mode;

/* Flags of cp_attn_rank_forward. */
#define CP_RING_PREFETCH 1  /* receive block t+1 on copy_stream while block t is computed */
#define CP_RING_REVERSE 2   /* visit (i + t) mod N instead of (i - t) mod N */

#define CP_MAX_RING 64      /* largest ring size N (and merge count n) accepted */

/* Bytes of the static device scratch of cp_attn_rank_forward_static (96 MiB
 * per GPU the library runs on, held until the process ends). */
#define CP_STATIC_SCRATCH_BYTES ((size_t)96 << 20)

/* Problem description (the shard statement of the pages: Q_i, K_j, V_j of
 * shape (S/N) x H x d, rank i, ring size N, mask).  */
typedef struct {
  int32_t B;                     /* batch, >= 1 */
  int32_t H;                     /* heads, >= 1 (same for Q and K/V) */
  int32_t d;                     /* head dimension: 64 or 128 */
  int32_t N;                     /* ring size, 1 <= N <= CP_MAX_RING */
  int64_t L;                     /* shard length S/N, >= 1 */
  int32_t rank;                  /* 0 <= rank < N: this shard's queries are tokens [rank L, (rank+1) L) */
  int32_t dtype;                 /* cp_dtype of Q, K, V and out */
  int32_t mask;                  /* cp_mask */
  int32_t ndocs;                 /* DOC_CAUSAL only: number of documents */
  const int32_t* cu_seqlens;     /* DOC_CAUSAL only: HOST array of ndocs+1 global boundaries,
                                    cu[0] = 0 < cu[1] < ... < cu[ndocs] = N L */
  const int32_t* cu_seqlens_dev; /* DOC_CAUSAL only: DEVICE copy of the same ndocs+1 values */
  float scale;                   /* softmax scale; 0 means 1/sqrt(d) */
} cp_attn_desc;

/* Running state of one rank (device, float32): o unnormalised [B, L, H, d];
 * m (natural-log units) and l [B, H, L]. */
typedef struct {
  float* o;
  float* m;
  float* l;
} cp_state;

/* Opaque per-launch timer: HIP events recorded around each attention kernel
 * of cp_attn_rank_forward (and _fp8, _static) on the compute stream, and
 * around each ring receive on the stream that carries it (the copy stream
 * with CP_RING_PREFETCH, else the compute stream). */
typedef struct cp_attn_profiler cp_attn_profiler;

/* One block of the online-softmax recurrence (compassingai.com page, section
 * "線上 Softmax": S_ij = Q_i K_j^T / sqrt(d), mask, m_ij, P_ij, l_ij, merge into
 * (O, m, l)), run for block j (0 <= j < N) of the desc's ring.
 *   q, k_j, v_j : device [B, L, H, d] of desc->dtype.
 *   mode INIT/ACCUMULATE: `state` (device, caller-owned) is written (and read
 *     for ACCUMULATE); o_part/lse_part must be NULL.
 *   mode PARTIAL_LSE: o_part [B, L, H, d] and lse_part [B, H, L] (device
 *     float32) receive the block's normalised output and lse; state must be
 *     NULL.
 * Rows with no visible key in the block: INIT sets m = -inf, l = 0, O = 0;
 * ACCUMULATE leaves them unchanged; PARTIAL_LSE writes O = 0, lse = -inf.
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_HIP. */
cp_status cp_attn_block_partial(const cp_attn_desc* desc, int32_t j, int32_t mode,
                                const void* q, const void* k_j, const void* v_j,
                                const cp_state* state, float* o_part, float* lse_part,
                                void* stream);

/* Merge of n per-block partials (O_j, lse_j) in the given order, the
 * log-sum-exp form of the same recurrence: lse = ln sum_j exp(lse_j),
 * O = sum_j exp(lse_j - lse) O_j (process-cxr.github.io page, section
 * "Long Context Attention 中的通信": attention output aggregation with the
 * softmax max/sum reductions).
 *   o_parts, lse_parts : HOST arrays of n device pointers ([B, L, H, d] and
 *                        [B, H, L] float32); 1 <= n <= CP_MAX_RING.
 *   order              : HOST array of n distinct indices into the parts, or
 *                        NULL for 0..n-1; terms are summed in this order.
 *   out                : device [B, L, H, d] of desc->dtype;
 *   lse_out            : device [B, H, L] float32, or NULL.
 * Rows where every part is empty get O = 0 and lse = -inf.
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_HIP. */
cp_status cp_attn_merge_lse(const cp_attn_desc* desc, int32_t n, const float* const* o_parts,
                            const float* const* lse_parts, const int32_t* order, void* out,
                            float* lse_out, void* stream);

/* Final step of the recurrence: out = O / l (0 where l = 0) in desc->dtype
 * (bf16 rounded to nearest even), and optionally m_out, l_out and
 * lse_out = m + ln l (device [B, H, L] float32, each may be NULL).
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_HIP. */
cp_status cp_attn_finalize(const cp_attn_desc* desc, const cp_state* state, void* out,
                           float* m_out, float* l_out, float* lse_out, void* stream);

/* Bytes of workspace cp_attn_rank_forward needs for this desc: two K/V
 * receive slots, the running state and alignment padding.  Returns 0 if the
 * desc is invalid (cp_attn_last_error() says why). */
size_t cp_attn_workspace_bytes(const cp_attn_desc* desc);

/* The whole forward of rank desc->rank (compassingai.com page, section
 * "線上 Softmax", and the wangyu.me page, sections "Ring Attention" and
 * "通信模式"), with the ring simulated on one GPU: K/V block j lives at
 * k_blocks[j], v_blocks[j] (HOST arrays of N device pointers; the rank's own
 * block is k_blocks[rank]).  At ring step t the rank holds block
 * j_t = (rank - t) mod N (or (rank + t) mod N with CP_RING_REVERSE); blocks no
 * row can see are skipped (causal: j > rank; documents: blocks that end before
 * the document of the shard's first token begins).  Every step after the
 * first receives its block into one of two workspace slots with a
 * device-to-device copy (V is written in head-dim-major key tiles, the
 * layout the attention kernels read best; the caller's blocks are only
 * read); with CP_RING_PREFETCH the copy runs on copy_stream
 * while the previous block is computed (events order slot reuse), otherwise
 * it runs on compute_stream.  The last step writes the final output.
 *   out          : device [B, L, H, d] of desc->dtype;
 *   m_out, l_out, lse_out : device [B, H, L] float32, each may be NULL;
 *   workspace    : device, >= cp_attn_workspace_bytes(desc) bytes, 256-byte
 *                  aligned, not shared with a concurrent call;
 *   copy_stream  : used only with CP_RING_PREFETCH; must differ from
 *                  compute_stream; the function returns with all its work
 *                  ordered before later work on compute_stream;
 *   prof         : NULL, or a profiler that records each attention kernel.
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_WORKSPACE, CP_ERR_HIP. */
cp_status cp_attn_rank_forward(const cp_attn_desc* desc, const void* q,
                               const void* const* k_blocks, const void* const* v_blocks,
                               void* out, float* m_out, float* l_out, float* lse_out,
                               void* workspace, size_t workspace_bytes, void* compute_stream,
                               void* copy_stream, int32_t flags, cp_attn_profiler* prof);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): cp_attn_rank_forward
 * with the same arguments except the workspace, which is a static device array
 * of CP_STATIC_SCRATCH_BYTES inside the library (one per GPU, on the current
 * device).  It runs the same kernels in the same order, so its results are
 * bit-identical to cp_attn_rank_forward's.  It calls no allocation routine
 * (only the per-call HIP events of the ring hand-offs are created and
 * destroyed).  Every call on one GPU shares that GPU's array and leaves its
 * contents behind (no part of it needs clearing: the receive writes whole
 * slots and the first step writes the running state), so calls that overlap
 * on one GPU race: the caller runs them one after another.
 * Errors: CP_ERR_WORKSPACE when cp_attn_workspace_bytes(desc) exceeds
 * CP_STATIC_SCRATCH_BYTES (then nothing is enqueued); otherwise as
 * cp_attn_rank_forward. */
cp_status cp_attn_rank_forward_static(const cp_attn_desc* desc, const void* q,
                                      const void* const* k_blocks, const void* const* v_blocks, void* out,
                                      float* m_out, float* l_out, float* lse_out, void* compute_stream,
                                      void* copy_stream, int32_t flags, cp_attn_profiler* prof);

/* ---- All-to-all (Ulysses) context parallelism, one rank's share ----------
 * The second scheme of the compassingai.com page (section
 * "方案二：All-to-All（全交換）"): the ranks hold the same sequence shards as
 * in the ring; an all-to-all regroups Q, K, V from split-by-sequence to
 * split-by-head, each rank computes attention over the whole sequence for its
 * heads, and a second all-to-all regroups the outputs back to
 * split-by-sequence.  Under a causal or document mask the invalid region is
 * masked, not skipped (same page, section "技術路線對比"); the two
 * exchanges move about 2 x S H d elements (section "通訊量分析").  Rank r
 * takes the contiguous head group [r H/N, (r+1) H/N); desc->H must be a
 * multiple of desc->N.  The masks use the same global positions as the ring
 * (shard i covers [i L, (i+1) L)). */

/* Bytes of workspace cp_attn_ulysses_forward needs: the whole sequence of
 * the rank's heads for Q, K, V and the output, 4 x B S (H/N) d elements of
 * desc->dtype, 256-byte aligned pieces.  Returns 0 if the desc is invalid or
 * H is not a multiple of N (cp_attn_last_error() says why). */
size_t cp_attn_ulysses_workspace_bytes(const cp_attn_desc* desc);

/* The share of rank r = desc->rank, with the two all-to-alls simulated on one
 * GPU: q_shards[i], k_shards[i], v_shards[i] (HOST arrays of N device
 * pointers, [B, L, H, d] of desc->dtype each) are what rank i holds; this
 * call reads only heads [r H/N, (r+1) H/N) of them (the first exchange, as
 * received by rank r), runs the attention of the whole sequence S = N L on
 * those heads (one launch of the block kernel), and writes the result into
 * the same heads of o_shards[i] (HOST array of N device pointers, [B, L, H,
 * d] of desc->dtype; the second exchange, as sent by rank r), leaving the
 * other heads of o_shards untouched.  Calling it for every rank fills all of
 * o_shards.
 *   m_out, l_out, lse_out : device [B, H/N, S] float32 for rank r's heads over
 *                  the whole sequence (natural-log units), each may be NULL;
 *   workspace    : device, >= cp_attn_ulysses_workspace_bytes(desc) bytes,
 *                  256-byte aligned, not shared with a concurrent call;
 *   stream       : all work is enqueued on it, in order.
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_WORKSPACE, CP_ERR_HIP. */
cp_status cp_attn_ulysses_forward(const cp_attn_desc* desc, const void* const* q_shards,
                                  const void* const* k_shards, const void* const* v_shards,
                                  void* const* o_shards, float* m_out, float* l_out, float* lse_out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ---- FP8 (e4m3) ---------------------------------------------------------
 * The compassingai.com page notes that the bytes CP moves depend on whether
 * blocks travel compressed or in FP8 (section "通訊量分析") and that
 * FlashAttention-3 computes attention in FP8 (section "技術演進史").  This
 * library's FP8 format is OCP E4M3 (largest value 448) with one float32
 * scale per (batch, head) and block, a power of two: with y = float32(x * c)
 * (c = 1 for keys and values; for the query, c = the desc's softmax scale
 * times log2(e), rounded to float32), amax = max |y| over the block's tokens
 * and head dim and scale = 2^e, e the smallest integer >= -126 with
 * amax <= 448 * 2^e (0 when amax = 0).  A value x is stored as the e4m3 code
 * nearest to y * 2^-e, ties to even, and stands for decode(code) * scale / c.
 * Power-of-two scales are applied exactly by the FP8 matrix core's block-scale
 * operands, and the query's c makes its products with the key codes base-2
 * logits. */
#define CP_FP8_KV 0     /* role of a key or value block: c = 1 */
#define CP_FP8_QUERY 1  /* role of the query: c = softmax scale * log2(e) */

/* Quantise one bf16 block x (device [B, L, H, d] with desc's B, L, H, d) to
 * codes (device [B, L, H, d] bytes, 8-byte aligned) and scales (device [B, H]
 * float32) in the given role (CP_FP8_KV or CP_FP8_QUERY; the query's c uses
 * desc->scale, 1/sqrt(d) when 0).  x must be finite.  Four launches on stream
 * (fill, per-head maxima, codes, scales); scales is overwritten.
 * Errors: CP_ERR_INVALID_ARG (also an unknown role), CP_ERR_UNSUPPORTED
 * (desc->dtype not bf16), CP_ERR_HIP. */
cp_status cp_attn_quantize_fp8(const cp_attn_desc* desc, const void* x, int32_t role, void* codes, float* scales,
                               void* stream);

/* The whole forward of rank desc->rank over the simulated ring, as
 * cp_attn_rank_forward, with FP8 inputs: q (device [B, L, H, d] e4m3 codes)
 * with q_scale (device [B, H] float32), and per block j the codes k_blocks[j],
 * v_blocks[j] with k_scales[j], v_scales[j] (HOST arrays of N device
 * pointers; entries of blocks the rank never visits may be NULL), all as
 * written by cp_attn_quantize_fp8: q in the CP_FP8_QUERY role under a desc
 * with this desc's scale, the blocks in the CP_FP8_KV role.  Scales must be
 * powers of two from 2^-126 to 2^127 (only their exponents are read; they
 * live in device memory and are not checked).  The ring moves the one-byte
 * codes (half the bytes of bf16).  Both products run on the FP8 matrix cores with float32
 * accumulation; P is rounded to e4m3 for the P V product and l sums the same
 * rounded values.  out is bf16 (desc->dtype must be CP_BF16); m, l, lse as in
 * cp_attn_rank_forward; workspace of cp_attn_workspace_bytes(desc).
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_WORKSPACE, CP_ERR_HIP. */
cp_status cp_attn_rank_forward_fp8(const cp_attn_desc* desc, const void* q, const float* q_scale,
                                   const void* const* k_blocks, const float* const* k_scales,
                                   const void* const* v_blocks, const float* const* v_scales, void* out,
                                   float* m_out, float* l_out, float* lse_out, void* workspace,
                                   size_t workspace_bytes, void* compute_stream, void* copy_stream, int32_t flags,
                                   cp_attn_profiler* prof);

/* ---- Backward of one rank shard ------------------------------------------
 * The backward walks the ring's K/V blocks again and recomputes what the
 * forward did not keep (compassingai.com page, section "反向傳播"; the Q, K, V
 * gradients go back around the ring, process-cxr.github.io page, section
 * "Long Context Attention 中的通信").  Per visible block j, with P_j
 * recomputed from the forward's log-sum-exp and the chain rule of the forward
 * definition (compassingai.com page, section "數學基礎"):
 *   P_j = exp(Q K_j^T * scale - lse) (masked),  dP_j = dO V_j^T,
 *   dS_j = P_j * (dP_j - delta),  delta = rowsum(dO * O),
 *   dQ += scale dS_j K_j,  dK_j = scale dS_j^T Q,  dV_j = P_j^T dO.
 * dK_j, dV_j are this rank's contributions to block j's gradients; summed over
 * all ranks they give the full-sequence gradient.  bf16 inputs only (an f32
 * desc gives CP_ERR_UNSUPPORTED); gradients are float32.  The scale is the
 * desc's (1/sqrt(d) when 0), the same as the forward's. */

/* delta [B, H, L] (device float32) = sum over the head dim of dO * O, with
 * o the forward output and d_o its gradient (device bf16 [B, L, H, d]).
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_HIP. */
cp_status cp_attn_bwd_delta(const cp_attn_desc* desc, const void* o, const void* d_o, float* delta,
                            void* stream);

/* One block's backward for block j (0 <= j < N) of the desc's ring.
 *   q, k_j, v_j, d_o : device bf16 [B, L, H, d];
 *   lse              : device [B, H, L] float32, the forward's lse over ALL
 *                      blocks (natural log, e.g. lse_out of
 *                      cp_attn_rank_forward);
 *   delta            : device [B, H, L] float32 from cp_attn_bwd_delta;
 *   dq               : device [B, L, H, d] float32: mode CP_MODE_INIT writes
 *                      this block's dQ part, CP_MODE_ACCUMULATE adds it;
 *   dk_j, dv_j       : device [B, L, H, d] float32, written (zero when no row
 *                      of the rank sees the block).
 * Rows whose lse is -inf contribute nothing.
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_HIP. */
cp_status cp_attn_block_backward(const cp_attn_desc* desc, int32_t j, int32_t mode, const void* q,
                                 const void* k_j, const void* v_j, const void* d_o, const float* lse,
                                 const float* delta, float* dq, float* dk_j, float* dv_j, void* stream);

/* The whole backward of rank desc->rank: delta, then every block in the
 * forward's ring order (CP_RING_REVERSE honoured), all on `stream`.
 *   k_blocks, v_blocks : HOST arrays of N device bf16 pointers (as for the
 *                        forward; only visible blocks are read);
 *   o, d_o             : device bf16 [B, L, H, d]: forward output, its gradient;
 *   lse                : device [B, H, L] float32 of the forward;
 *   delta              : device [B, H, L] float32, written (caller-owned scratch);
 *   dq                 : device [B, L, H, d] float32, written;
 *   dk_blocks, dv_blocks : HOST arrays of N device float32 [B, L, H, d]
 *                        pointers, each written (zeros for blocks the rank
 *                        does not see).
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_UNSUPPORTED, CP_ERR_HIP. */
cp_status cp_attn_rank_backward(const cp_attn_desc* desc, const void* q, const void* const* k_blocks,
                                const void* const* v_blocks, const void* o, const void* d_o,
                                const float* lse, float* delta, float* dq, float* const* dk_blocks,
                                float* const* dv_blocks, int32_t flags, void* stream);

/* Host-only: the blocks cp_attn_rank_forward computes on, in visiting order.
 * Writes at most `capacity` block ids to blocks_out and the count to
 * *count_out.  Errors: CP_ERR_INVALID_ARG (also when capacity is too small). */
cp_status cp_attn_ring_schedule(const cp_attn_desc* desc, int32_t flags, int32_t* blocks_out,
                                int32_t capacity, int32_t* count_out);

/* Host-only: number of visible (query, key) pairs of ONE head of one batch
 * element of this rank (causal-adjusted work is 4 d B H times this in
 * flops).  Errors: CP_ERR_INVALID_ARG. */
cp_status cp_attn_visible_pairs(const cp_attn_desc* desc, int64_t* pairs_out);

/* Profiler: capacity = number of kernel launches (and, separately, of ring
 * receives) it can time; records beyond capacity are dropped.  read() waits
 * for the recorded events and writes each attention launch's duration in
 * milliseconds; read_copies() does the same for each ring receive (the
 * device-to-device copy of K_j and the re-layout of V_j into a workspace
 * slot: the simulated communication of one ring step, compassingai.com page,
 * section "關鍵指標", communication/computation ratio); reset() forgets both.
 * Errors: CP_ERR_INVALID_ARG (capacity too small, NULL arguments),
 * CP_ERR_HIP. */
cp_status cp_attn_profiler_create(int32_t capacity, cp_attn_profiler** out);
cp_status cp_attn_profiler_reset(cp_attn_profiler* prof);
cp_status cp_attn_profiler_read(cp_attn_profiler* prof, float* ms_out, int32_t capacity,
                                int32_t* count_out);
cp_status cp_attn_profiler_read_copies(cp_attn_profiler* prof, float* ms_out, int32_t capacity,
                                       int32_t* count_out);
void cp_attn_profiler_destroy(cp_attn_profiler* prof);

/* Measurement helper (not part of the method): read `bytes` of device memory
 * at src once through the global -> LDS fetch the attention kernels use for
 * their K/V tiles (16 bytes per lane), discarding the data.  A profiler's
 * count of HBM bytes fetched for this kernel against `bytes` calibrates the
 * same counter read for the attention kernels.  src: device, 16-byte
 * aligned; bytes: a positive multiple of 4096.  Asynchronous on `stream`.
 * Errors: CP_ERR_INVALID_ARG, CP_ERR_HIP. */
cp_status cp_attn_measure_lds_stream(const void* src, size_t bytes, void* stream);

/* Static name of a status code. */
const char* cp_attn_status_string(int32_t status);
/* Message of the last error on the calling thread ("" if none). */
const char* cp_attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CPATTN_H */
