/*
 * gdn_cpr.h -- C ABI of the chunkwise-parallel recurrent (CPR) Gated DeltaNet
 * layer for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For each head the layer carries a state S (d_k x d_v,
 * fp32; S = M^T for the d_v x d_k matrix M of the update rule) and, token by
 * token,
 *     M_t = alpha_t M_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = M_t q_t,        alpha_t = exp(g_t).
 * CPR (IsoExec pages, "Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet";
 * Chinese page, the section on a third way for Gated DeltaNet) evaluates this
 * recurrence so that training, prefill and decode round identically:
 *   - prefill / training first compute the state at every chunk boundary
 *     (every C tokens from each sequence's start) with the chunk (WY/UT) form,
 *     then run the per-token recurrence inside every chunk, all chunks in
 *     parallel, each starting from its boundary state;
 *   - decode runs the same per-token step and, every C tokens, replaces its
 *     running state by the chunk-boundary computation over the last C tokens.
 * Between boundaries the per-token step keeps the running state as
 * exp(lg) N: the decay accumulates in one scalar lg per head instead of
 * being applied to every state element at every token (gdn_cpr_cache,
 * run_log_scale).  The per-token step is the same routine in prefill and
 * decode.
 * Every output of this library is therefore bit-identical between prefill
 * and decode, and between a sequence run alone and the same sequence packed
 * with others.  The results match the exact recurrence within fp32 rounding
 * (fp32 inputs) or within the rounding of bf16 chunk operands (bf16 inputs).
 *
 * Conventions (all calls):
 *   - Pointers are DEVICE pointers owned by the caller unless marked host.
 *     The library allocates no device memory and keeps none between calls;
 *     scratch lives in the caller's workspace (size from
 *     gdn_cpr_workspace_size).  The one exception is
 *     gdn_cpr_decode_step_noalloc, whose scratch is a fixed array inside the
 *     library.  Calls only enqueue work on `stream` (a
 *     hipStream_t; NULL = the legacy default stream) and return; results are
 *     ready when the stream reaches them.  No call synchronises the host.
 *     This is what lets a serving engine keep its scheduler, its KV-cache
 *     management and graph capture unchanged under the method (Chinese page,
 *     opening summary, and the section on the method's two parts, the
 *     execution contract and the unified model): every call can be recorded
 *     into a hipGraph and replayed.
 *   - The initial state h0 and the final state hT are plain fp32 states in
 *     the S layout below, indexed by batch entry; the final state is
 *     written from the kernels that produce it (the chain for a sequence
 *     that ends on a chunk boundary, the scan of its last chunk otherwise),
 *     with no extra pass.
 *   - Token-major packed layouts: q, k [T, H_k, d_k]; v, o [T, H, d_v];
 *     g, beta [T, H]; all rows contiguous.  H_k = H unless the shape asks
 *     for fewer key heads.  The pages name hybrid Gated DeltaNet models
 *     (Chinese page, the paragraph on the released code and the model
 *     classes it supports) without their layer dimensions; layers of that
 *     kind may give q and k fewer heads than v, so the library takes H_k
 *     key heads, each serving H / H_k consecutive value heads.  cu_seqlens int32 [N + 1] with
 *     cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N] = T.
 *   - States [N, H, d_k, d_v] fp32, key dimension first (S layout).
 *   - dtype GDN_DTYPE_F32: q, k, v, g, beta, o (and d_o, dq, dk, dv) are fp32.
 *     dtype GDN_DTYPE_BF16: they are bf16 (raw 16-bit patterns); outputs are
 *     rounded to nearest even.  States, dg, dbeta are always fp32.
 *   - g must be <= 0 (alpha in (0, 1]); beta is used as given.  Values are
 *     not checked on the device.
 *   - Supported shapes: d_k, d_v in {64, 128}; C in {16, 32, 64}; H >= 1;
 *     H_k divides H.  The pages' layers use C = 64 (the chunk size of the
 *     chunked kernels they name); other hybrid Gated DeltaNet layers may
 *     resynchronise more often, so 16 and 32 are accepted: a chunk of C < 64
 *     tokens is evaluated as a 64-row chunk whose rows past C are identity
 *     steps (k = v = 0, g = beta = 0), which changes no real row's value.
 *     The comparators (gdn_cmp_*) take C = 64 only.
 *   - d_k = d_v = 256 is accepted for bf16 inputs by gdn_cpr_prefill,
 *     gdn_cpr_decode_step(_noalloc), gdn_cpr_prefill_continue,
 *     gdn_cpr_cache_state and gdn_cpr_fwd_bwd (the pages give no layer
 *     dimensions, so heads wider than their shapes are served too).  A state
 *     column's 256 keys are then split over two lanes whose partial dot
 *     products meet in one add (order in gdn_cpr_numerics_id); prefill and
 *     decode still agree bit for bit.  fwd_bwd's forward at 256 is the
 *     prefill; its backward takes fp32 products and a larger workspace
 *     (gdn_cpr_workspace_size).  The comparators take 64 and 128 only.
 *   - Every pointer must be 16-byte aligned.
 *   - Errors detectable on the host (null or misaligned pointer, unsupported
 *     shape, workspace too small, negative sizes) return a status before any
 *     work is enqueued; gdn_cpr_last_error() then describes it.  Launch
 *     failures return GDN_ERR_HIP.  A malformed cu_seqlens (not
 *     non-decreasing, or not ending at T) is the caller's error and is not
 *     detected.
 *   - A bf16 prefill of up to 128 sequences runs its chunk products, chain
 *     and scan as one launch in which work-groups wait for results of other
 *     work-groups of the same launch.  Every such wait is on work that
 *     started earlier and is bounded (about a second of polling); none is
 *     expected to give up.  If one does, that call's outputs are not valid,
 *     and gdn_cpr_wait_status (below) reports it without a host
 *     synchronisation.
 */
#ifndef GDN_CPR_H
#define GDN_CPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1,
  GDN_ERR_UNSUPPORTED = 2,
  GDN_ERR_WORKSPACE = 3,
  GDN_ERR_HIP = 4
} gdn_status;

typedef enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 } gdn_dtype;

typedef enum {
  GDN_OP_PREFILL = 0,
  GDN_OP_DECODE = 1,
  GDN_OP_FWD_BWD = 2,
  GDN_OP_PREFILL_CONTINUE = 3
} gdn_op;

/* Layer shape (host struct). */
typedef struct {
  int32_t num_heads;     /* H: value heads (v, g, beta, o, states, caches) */
  int32_t head_dim_k;    /* d_k */
  int32_t head_dim_v;    /* d_v */
  int32_t chunk;         /* C, the boundary / resynchronisation period: 16, 32 or 64 */
  int32_t dtype;         /* gdn_dtype of q, k, v, g, beta, o and the tail buffers */
  int32_t num_key_heads; /* H_k: heads of q and k; 0 means H.  H_k divides H and
                            value head h reads key head h / (H / H_k) */
} gdn_cpr_shape;

/*
 * Per-sequence CPR cache (host struct of device pointers), N sequences.
 * This is everything decode needs to continue a sequence bit-exactly, and it
 * is position independent: copying it elsewhere (or to the host and back)
 * and continuing gives the same bits.
 *   s_bnd     [N, H, d_k, d_v] fp32  state at the last chunk boundary
 *   s_run     [N, H, d_k, d_v] fp32  state after the last token in scaled
 *                                    form: the state is exp(run_log_scale) *
 *                                    s_run (gdn_cpr_cache_state writes it
 *                                    out); when tail_len = 0, s_run = s_bnd
 *                                    and run_log_scale = 0
 *   tail_k    [N, H, C, d_k] dtype   tokens since that boundary
 *   tail_v    [N, H, C, d_v] dtype
 *   tail_g    [N, H, C]      dtype
 *   tail_beta [N, H, C]      dtype
 *   tail_len  [N, H] int32 in [0, C-1]; equal across the heads of a sequence
 *                                    (one counter per head so that each head's
 *                                    work item owns its own counter)
 *   slot_index [N] int32, or NULL    slot-indexed caches: batch entry i uses
 *                                    row slot_index[i] of every array above
 *                                    (which then have at least
 *                                    max(slot_index) + 1 rows in place of N);
 *                                    rows must be distinct within a call.
 *                                    NULL: row i.  Rows not named are not
 *                                    touched, so a serving engine can keep a
 *                                    pool of cache rows and pass each step's
 *                                    batch by row number.
 *   run_log_scale [N, H] fp32        log of s_run's scale: the cumulative
 *                                    log-decay since the last boundary (or
 *                                    since the last renormalisation, which
 *                                    sets it to 0 when it would fall below
 *                                    -32).  Keeping the decay in this scalar
 *                                    rather than in every state element is
 *                                    part of the pinned per-token step that
 *                                    prefill and decode share.
 */
typedef struct {
  float* s_bnd;
  float* s_run;
  void* tail_k;
  void* tail_v;
  void* tail_g;
  void* tail_beta;
  int32_t* tail_len;
  const int32_t* slot_index;
  float* run_log_scale;
} gdn_cpr_cache;

/*
 * Bytes of workspace a call needs (host only; never fails, returns 0 for an
 * invalid or unsupported shape).  op is a gdn_op.  For GDN_OP_DECODE,
 * total_tokens is ignored (one token per sequence).
 */
size_t gdn_cpr_workspace_size(const gdn_cpr_shape* shape, int32_t num_seqs,
                              int64_t total_tokens, int32_t op);

/*
 * Wait status of the most recent gdn_cpr_prefill, gdn_cpr_prefill_continue
 * or gdn_cpr_fwd_bwd call that used `workspace`, called with that call's
 * shape, num_seqs and total_tokens: enqueues on `stream` a copy of one
 * int32 into `status` (device memory, 16-byte aligned), 0 if every bounded
 * wait of that call ended with its data published and 1 if one gave up (see
 * the conventions above).  Stream-ordered like the calls; the host reads
 * the value once the stream has reached it.  For callers that check a
 * result without synchronising the device, e.g. a service's health check.
 * After a call with num_seqs = 0 (which enqueues nothing) the word is that
 * of the call before.  Errors: see the conventions.
 */
gdn_status gdn_cpr_wait_status(const gdn_cpr_shape* shape, int32_t num_seqs, int64_t total_tokens,
                               const void* workspace, size_t workspace_bytes, int32_t* status,
                               void* stream);

/*
 * Test hook for the failure path above: a positive `polls` bounds every
 * such wait at that many polls instead of about a second's worth, so that
 * a test can make waits give up (the call's outputs are then not valid, but
 * every work-group still finishes); 0 restores the default.  Applies to the
 * current device, synchronously, to calls enqueued afterwards; not for use
 * beside other work on the device.  Errors: GDN_ERR_INVALID_ARG for a
 * negative count, GDN_ERR_HIP if the copy fails.
 */
gdn_status gdn_cpr_debug_set_wait_polls(int32_t polls);

/*
 * Prefill: the engine_prefill case of the pages' execution contract, whose
 * cases name the stage a kernel region runs in (English page, "The IsoExec
 * Unified Execution Contract", cases and regions; Chinese page, section on
 * the method's two parts).  CPR evaluates it as the pages' third way for
 * Gated DeltaNet prescribes for prefill and training (Chinese page, that
 * section; English page, CPR section): the recurrent state at every chunk
 * boundary first, then the recurrence inside all chunks in parallel, each
 * from its boundary state.  Runs N packed sequences from their initial
 * states and fills the cache so that decode can continue them.  Chunks
 * start at each sequence's first token.  The chain of boundary states covers
 * a sequence's full chunks; the tokens after its last full chunk (L mod C of
 * them) become the cache's tail.
 *   q, k, v, g, beta  inputs, layouts above (T = total_tokens rows)
 *   cu_seqlens        [N + 1] int32
 *   h0                [N, H, d_k, d_v] fp32 initial states indexed by batch
 *                     entry (not by cache row), or NULL for zero states.
 *                     May alias cache_out->s_bnd or ->s_run when the cache
 *                     has no slot_index, and may alias hT.
 *   hT                [N, H, d_k, d_v] fp32 final states (the state after
 *                     each sequence's last token, h0 for an empty one)
 *                     indexed by batch entry, or NULL.  Must not alias the
 *                     cache.  Equal bit for bit to what gdn_cpr_cache_state
 *                     reads out of cache_out afterwards.
 *   cache_out         host struct; every field required; written in full
 *   o                 [T, H, d_v] outputs
 * Zero-length sequences are allowed: their cache becomes h0 and no output
 * rows exist for them.  Errors: see the conventions; nothing is enqueued on
 * a host-detected error.
 */
gdn_status gdn_cpr_prefill(const gdn_cpr_shape* shape, int32_t num_seqs, int64_t total_tokens,
                           const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const int32_t* cu_seqlens, const float* h0, float* hT,
                           const gdn_cpr_cache* cache_out, void* o, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Decode: the engine_decode case of the execution contract (English page,
 * contract section, cases; Chinese page, section on the method's two parts).
 * CPR decodes in recurrent form and resynchronises the running state to the
 * chunk-boundary computation every C tokens (English page, CPR section;
 * Chinese page, third-way section), so its outputs equal prefill's bit for
 * bit.  One token for each of N sequences.
 *   q, k, v, g, beta  one token per sequence: q, k [N, H_k, d_k]; v [N, H, d_v];
 *                     g, beta [N, H]
 *   cache             read-modify-write in place
 *   hT                [N, H, d_k, d_v] fp32 state after the token, indexed by
 *                     batch entry, or NULL (the usual case: the cache holds
 *                     it in scaled form and gdn_cpr_cache_state reads it
 *                     out; asking for it here writes 64 KB more per
 *                     (sequence, head) at d = 128).  Must not alias the cache.
 *   o                 [N, H, d_v]
 * The token's output comes from the per-token step on s_run, the routine
 * prefill's in-chunk scan runs.  When the step completes a chunk (tail_len
 * reaches C), s_bnd and s_run are both replaced by the chunk-boundary
 * computation from s_bnd over the C tail tokens (prefill's chunk products
 * and chain step), and tail_len returns to 0.  A cache row whose tail_len is
 * outside [0, C) is left untouched.
 */
gdn_status gdn_cpr_decode_step(const gdn_cpr_shape* shape, int32_t num_seqs, const void* q,
                               const void* k, const void* v, const void* g, const void* beta,
                               const gdn_cpr_cache* cache, float* hT, void* o, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * gdn_cpr_decode_step for callers that cannot allocate device memory: code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors are those of gdn_cpr_decode_step (the same
 * kernels; bit-identical outputs and cache), without the workspace.
 * Scratch: one fixed array of GDN_NOALLOC_SCRATCH_BYTES (64.5 MiB) per
 * device, in the library's code object, which each device that runs it
 * holds until the process ends.  It holds the per-(sequence, head) resync
 * flags and the chunk products of the tails that fill; everything in it is
 * written before it is read, so no call needs it cleared.
 * Limits (GDN_ERR_UNSUPPORTED, nothing enqueued): num_seqs * H <=
 * GDN_NOALLOC_MAX_PAIRS (65,536), and H no larger than the chunk-product
 * slots of 64 MiB (1,024 at d_k = d_v = 128 bf16, 682 for fp32).  Tails that
 * fill are resynchronised in groups of as many sequences as those slots
 * hold, one launch per group (bf16; two for fp32), so at large batches a
 * step takes a few more launches than gdn_cpr_decode_step.
 * Concurrency: every call on a device uses that device's one array, which
 * keeps the last call's contents.  Calls that overlap on one device (on
 * different streams, or from several threads) race; the caller orders them.
 * The device is the stream's.  The first call on a device looks up the
 * array's address there (hipGetSymbolAddress), with that device current:
 * make it outside graph capture.
 */
#define GDN_NOALLOC_MAX_PAIRS 65536
#define GDN_NOALLOC_SCRATCH_BYTES (2 * GDN_NOALLOC_MAX_PAIRS * 4 + (64 << 20))
gdn_status gdn_cpr_decode_step_noalloc(const gdn_cpr_shape* shape, int32_t num_seqs, const void* q,
                                       const void* k, const void* v, const void* g, const void* beta,
                                       const gdn_cpr_cache* cache, float* hT, void* o, void* stream);

/*
 * Prefill continued from a cache (serving: a further prompt segment, or
 * several decode tokens at once, for sequences whose state is in `cache`).
 * The pages state that the serving engine's scheduler, KV-cache management
 * and graph capture keep working under the method (Chinese page, opening
 * summary and the section on its two parts, the execution contract and the
 * unified model); this call extends a cached sequence by any number of tokens
 * with the bits that one prefill of the whole sequence (or decode token by
 * token) would give, with no host synchronisation.
 *   q, k, v, g, beta  the new tokens of the N sequences, packed, layouts
 *                     above (T = total_tokens rows)
 *   cu_seqlens        [N + 1] int32 over the new tokens
 *   cache             read-modify-write in place; cache i continues with
 *                     sequence i's new tokens
 *   hT                [N, H, d_k, d_v] fp32 final states (after each
 *                     sequence's last token; the cached state when it has
 *                     no new tokens) indexed by batch entry, or NULL.  Must
 *                     not alias the cache.
 *   o                 [T, H, d_v] outputs of the new tokens
 * Per sequence with tail_len = r and L new tokens: the first min(C - r, L)
 * tokens (none when r = 0) take the decode step from s_run and join the
 * tail; if they complete the chunk, s_bnd = s_run = the chunk-boundary
 * computation over the C tail tokens.  The remaining tokens, which start on a
 * chunk boundary, are prefilled from s_bnd.  L = 0 leaves the cache as it is.
 * So gdn_cpr_prefill(A + B) equals gdn_cpr_prefill(A) followed by this call
 * on B, bit for bit, and one token per sequence equals gdn_cpr_decode_step.
 * Workspace: gdn_cpr_workspace_size(..., GDN_OP_PREFILL_CONTINUE).
 */
gdn_status gdn_cpr_prefill_continue(const gdn_cpr_shape* shape, int32_t num_seqs, int64_t total_tokens,
                                    const void* q, const void* k, const void* v, const void* g,
                                    const void* beta, const int32_t* cu_seqlens, const gdn_cpr_cache* cache,
                                    float* hT, void* o, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * The state after each cached sequence's last token (the final state of
 * prefill, decode or continuation), written out from the cache's scaled form:
 *   state_out[i, h] = exp(run_log_scale[row, h]) * s_run[row, h]
 * with row = slot_index[i] (or i).  state_out is [N, H, d_k, d_v] fp32 and
 * must not alias the cache.  When tail_len = 0 the result equals s_bnd bit
 * for bit.  gdn_cpr_fwd_bwd's hT is this same product.
 */
gdn_status gdn_cpr_cache_state(const gdn_cpr_shape* shape, int32_t num_seqs, const gdn_cpr_cache* cache,
                               float* state_out, void* stream);

/*
 * Training forward + backward: the trainer_fwd case of the execution
 * contract (English page, contract section; Chinese page, section on the
 * method's two parts) plus its gradient; the pages time the pair as one
 * stage (English page, CPR table, trainer forward + backward row).  The
 * forward is the prefill computation (o and hT are bit-identical to
 * gdn_cpr_prefill's on the same inputs).  The backward is the exact gradient
 * of the recurrence for the loss sum(o * d_o) + sum(hT * d_hT), evaluated
 * per chunk from the boundary states.
 *   d_o               [T, H, d_v] dtype, upstream gradient of o
 *   d_hT              [N, H, d_k, d_v] fp32 upstream gradient of the final
 *                     states, or NULL (zero)
 *   o                 [T, H, d_v] forward output
 *   hT                [N, H, d_k, d_v] fp32 final states, or NULL
 *   dq, dk, dv        dtype, shaped like q, k, v
 *   dg, dbeta         [T, H] fp32
 *   dh0               [N, H, d_k, d_v] fp32, or NULL
 * For bf16 inputs the call runs independent stages side by side on two
 * streams: `stream` and a second stream on the same device that the call
 * takes from a small pool the library keeps per device (at most eight
 * streams, created at the default priority when first needed and kept until
 * the process ends; a call holds its stream only while it enqueues, so
 * concurrent callers never share one).  After the forward's chunk products,
 * the backward's local terms and reverse chain run on the second stream
 * beside the forward chain and in-chunk scan on `stream`; the state and
 * gradient stages follow the reverse chain on the second stream once the
 * forward chain is done (they do not read the scan's outputs), beside the
 * rest of the scan.  Events fork the work from `stream` and join it back, so
 * everything the call does is ordered on `stream` as with one stream (also
 * under graph capture, where the fork and join become graph edges; make a
 * first call outside a capture, since a call may create a pooled stream).
 * The bits do not depend on this: each kernel computes the same values in
 * either order.  If no second stream can be had the call runs on `stream`
 * alone.
 */
gdn_status gdn_cpr_fwd_bwd(const gdn_cpr_shape* shape, int32_t num_seqs, int64_t total_tokens,
                           const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const int32_t* cu_seqlens, const float* h0,
                           const void* d_o, const float* d_hT, void* o, float* hT, void* dq,
                           void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Comparators (not CPR).  The pages measure CPR against the evaluation orders
 * it replaces: chunkwise-parallel prefill and training with a recurrent
 * decode, whose outputs disagree (English page, CPR section and its table;
 * Chinese page, third-way section).  These calls build those orders from
 * this library's routines so that the disagreement and the cost of each
 * order can be measured on the same inputs; bf16 inputs only.
 *   GDN_CMP_RECURRENT  prefill = the per-token step over each whole sequence
 *                      (no chunk boundaries); decode = the same step.  Prefill
 *                      and decode agree bitwise, but prefill is sequential
 *                      along the sequence.
 *   GDN_CMP_CHUNKWISE  prefill = boundary states over every chunk (the last,
 *                      partial chunk zero-padded) and outputs from the chunk
 *                      form O = diag(Gamma) Q B + (Q K^T .* D) Delta with bf16
 *                      B, Delta and (Q K^T .* D) operands, no per-token scan.
 *                      Followed by gdn_cmp_decode_step it is the "native
 *                      mixed" serving path: prefill and decode round
 *                      differently.
 * gdn_cmp_prefill: h0 [N, H, d_k, d_v] or NULL (zeros); state_out
 * [N, H, d_k, d_v] receives each sequence's final state; o [T, H, d_v].
 * gdn_cmp_decode_step: the per-token step on state [N, H, d_k, d_v] (read-
 * modify-write), one token per sequence, no tail and no resynchronisation.
 * Workspace: gdn_cmp_workspace_size (the recurrent mode needs none beyond
 * 256 bytes; the decode step needs none).
 */
typedef enum { GDN_CMP_RECURRENT = 0, GDN_CMP_CHUNKWISE = 1 } gdn_cmp_mode;

size_t gdn_cmp_workspace_size(const gdn_cpr_shape* shape, int32_t mode, int32_t num_seqs, int64_t total_tokens);

gdn_status gdn_cmp_prefill(const gdn_cpr_shape* shape, int32_t mode, int32_t num_seqs, int64_t total_tokens,
                           const void* q, const void* k, const void* v, const void* g, const void* beta,
                           const int32_t* cu_seqlens, const float* h0, float* state_out, void* o,
                           void* workspace, size_t workspace_bytes, void* stream);

gdn_status gdn_cmp_decode_step(const gdn_cpr_shape* shape, int32_t num_seqs, const void* q, const void* k,
                               const void* v, const void* g, const void* beta, float* state, void* o,
                               void* stream);

/*
 * gdn_cmp_chunk_decode_step: the chunkwise-everywhere decode (the pages'
 * chunkwise decode column, English page, CPR table).  Each token recomputes
 * the chunk products of its partial chunk -- the cached tail, the token, zero
 * padding -- and takes its output from the chunk form on cache->s_bnd, so it
 * equals, bit for bit, the output gdn_cmp_prefill(GDN_CMP_CHUNKWISE) gives
 * the same token; the token is appended to the tail.  A token that completes
 * its chunk moves s_bnd (and s_run) to the next boundary by the same chain
 * step as the prefill, and empties the tail.  The cache is the CPR cache of
 * gdn_cpr_prefill, whose s_bnd and tail are what the chunkwise prefill
 * computes for the same tokens (the chunk products and the chain are shared);
 * between boundaries this call leaves s_run as it is, so the cache must not
 * then go on through gdn_cpr_decode_step.  Arguments, layouts, slot_index
 * and workspace (gdn_cpr_workspace_size with GDN_OP_DECODE) as
 * gdn_cpr_decode_step; a row with tail_len outside 0..C-1 is left untouched.
 */
gdn_status gdn_cmp_chunk_decode_step(const gdn_cpr_shape* shape, int32_t num_seqs, const void* q,
                                     const void* k, const void* v, const void* g, const void* beta,
                                     const gdn_cpr_cache* cache, void* o, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Measurement hook (the pages report per-stage timings of the layer, English
 * page, CPR table).  events points to an array of hipEvent_t handles owned by
 * the caller, or NULL to switch the hook off (the default).  While set, on
 * the calling thread, each call records events[0] before its first kernel
 * and events[i] after its stage i, on the call's stream:
 *   prefill / fwd_bwd forward: 1 plan, 2 chunk products, 3 boundary chain,
 *                              4 in-chunk scan
 *   decode:                    1 per-token step, 2 resynchronisation
 *   fwd_bwd backward:          5 reverse boundary chain, 6 per-chunk gradients
 * For bf16 fwd_bwd, whose backward local terms and reverse chain run on a
 * second stream beside stages 2-4, event 5 is recorded once the reverse chain
 * has joined `stream`; events 0 -> 6 span the whole call.
 * n_events is the array length; stages beyond it are not recorded.  Nothing
 * is allocated and nothing else changes.
 */
void gdn_cpr_set_stage_events(void* const* events, int32_t n_events);

/* Description of the last error on the calling thread ("" if none); valid
 * until the thread's next call into the library. */
const char* gdn_cpr_last_error(void);

/*
 * Text naming every choice that fixes the library's rounding (routine
 * versions, accumulation orders, operand precisions).  Two builds with the
 * same text produce the same bits.  It plays the part of the pages'
 * numerical-policy identity, a digest over every choice that affects the
 * numbers, which the trainer and the rollout engine compare before they run
 * together (English page, contract section, identities; Chinese page,
 * section on the method's two parts).  The returned string is static.
 */
const char* gdn_cpr_numerics_id(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CPR_H */
