/*
 * gla.h - C ABI of libgla.so: chunkwise Gated Linear Attention (GLA) forward
 * pass and single-token recurrent decode step for AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Gated Linear Attention (GLA): Mathematical Foundations,
 * Data-Dependent Gating, Chunkwise Parallel Forms ...", section "The Gated
 * Recurrent Update"): for each independent unit (sequence n, head h) and each
 * token t of that sequence, with the per-key-channel gate alpha_t = exp(g_t),
 *
 *     S_t = diag(alpha_t) S_{t-1} + k_t^T v_t          (S is d_k x d_v, fp32)
 *     o_t = q_t S_t                                    (the updated state)
 *
 * starting from S_0 = initial_state (zeros when NULL).  gla_chunk_fwd evaluates
 * it with the chunkwise-parallel form of the same page (section "Mathematical
 * Formulation of Chunk Computations": per chunk of 64 tokens an in-chunk
 * cumulative log-gate, gated causal intra-chunk attention, an inter-chunk term
 * from the carried state, and the state update), which equals the recurrence
 * up to rounding.  gla_recurrent_step is one token of the recurrence per
 * sequence: the decode step of the FlashLinearAttention page, section "The
 * O(1) Inference Memory Revolution".  There is no 1/sqrt(d_k) scale: callers
 * pre-scale q or k if they want one.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or equivalent) owned
 *     by the caller; the library keeps no pointer after the call returns and
 *     allocates no device memory.  Only gla_chunk_fwd_ws and gla_chunk_bwd
 *     take a workspace, which the caller allocates; gla_chunk_fwd_noalloc uses
 *     a scratch array the library holds (see there).
 *   - Layouts are row-major, last index fastest, densely packed, and every
 *     tensor pointer must be 16-byte aligned.
 *   - dtype selects the element type of q, k, v, g and o: GLA_BF16 (bfloat16)
 *     or GLA_F32 (float).  States are always fp32.
 *   - stream is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work; they never synchronize.  Results are deterministic run to run.
 *   - g = log(alpha) must be <= 0 (alpha in (0, 1]) and not +inf; this is not
 *     checked.  g = -inf (alpha = 0) is allowed.  NaN and Inf inputs propagate;
 *     in gla_chunk_fwd a NaN/Inf in v or k of token t can also reach outputs of
 *     earlier tokens of the same 64-token chunk (a masked score 0 times NaN).
 *   - Return value: GLA_OK, or an error code with nothing enqueued.  Argument
 *     checks happen on the host before any HIP call; the contents of device
 *     arrays (cu_seqlens) are trusted.  gla_last_error() gives the reason for
 *     the calling thread's last non-OK return.  No C++ exception crosses this
 *     boundary.
 */
#ifndef GLA_H_
#define GLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GLA_OK = 0,
  GLA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer      */
  GLA_ERR_UNSUPPORTED = 2, /* valid but not implemented (d_k, d_v, dtype, C)   */
  GLA_ERR_LAUNCH = 3       /* the HIP runtime refused the kernel launch        */
} gla_status;

typedef enum { GLA_BF16 = 0, GLA_F32 = 1 } gla_dtype;

/*
 * Chunkwise-parallel GLA forward.
 *
 *   q, k, g       [B, H, T, dk]  dtype          (g = log alpha per key channel)
 *   v             [B, H, T, dv]  dtype
 *   o             [B, H, T, dv]  dtype, written
 *   initial_state [Nseq, H, dk, dv] fp32, or NULL for zeros
 *   final_state   [Nseq, H, dk, dv] fp32, written, or NULL to skip.  It may be
 *                 the same pointer as initial_state (updated in place).
 *
 * Fixed length: cu_seqlens == NULL, Nseq = B, every sequence has T tokens.
 * Packed variable length: cu_seqlens = device int32[num_seqs + 1], B == 1,
 * Nseq = num_seqs, cu_seqlens[0] == 0, non-decreasing, cu_seqlens[num_seqs] == T;
 * sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]) of the T axis, chunks
 * restart at each sequence start, and a sequence may be empty (its final state
 * is its initial state).
 *
 * Supported: chunk_size == 64; dk in {64, 128}; dv a positive multiple of 64 up
 * to 512 (both dtypes).  T >= 0 (T == 0 only writes
 * final_state).  B * H * T and all index products must fit in int32 per tensor.
 */
int gla_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                  const float* initial_state, void* o, float* final_state,
                  const int32_t* cu_seqlens, int num_seqs, int B, int H, int T,
                  int dk, int dv, int chunk_size, int dtype, void* stream);

/*
 * gla_chunk_fwd with the width of its d_v slices chosen by the caller.  The
 * columns of the state evolve independently under the recurrence (page "Gated
 * Linear Attention (GLA) ...", section "The Gated Recurrent Update"), so each
 * work item is one (sequence, head, slice of dv_slice value columns); the page's
 * section "Architectural Trade-Offs and Limitations" (item 2) asks for such
 * tile sizes to be tuned to the hardware.
 *
 *   dv_slice   64, 128 (bf16 with dv a multiple of 128, else
 *              GLA_ERR_UNSUPPORTED), or 0 for gla_slice_plan's choice, which is
 *              what gla_chunk_fwd takes.  Other values: GLA_ERR_INVALID_ARG.
 *
 * Never splits sequences.  Other arguments, layouts and errors as for
 * gla_chunk_fwd; the results equal gla_chunk_fwd's up to rounding at either
 * width.
 */
int gla_chunk_fwd_sliced(const void* q, const void* k, const void* v, const void* g,
                         const float* initial_state, void* o, float* final_state,
                         const int32_t* cu_seqlens, int num_seqs, int B, int H, int T,
                         int dk, int dv, int chunk_size, int dtype, int dv_slice, void* stream);

/*
 * Device workspace, in bytes, that gla_chunk_fwd_ws needs for this shape; 0 when
 * the call would not split its sequences (then the workspace may be NULL).
 * Arguments as for gla_chunk_fwd (num_seqs > 0 means packed sequences, which
 * are never split).  Invalid shapes give 0; gla_chunk_fwd_ws reports them.
 */
size_t gla_chunk_fwd_workspace_size(int num_seqs, int B, int H, int T, int dk, int dv,
                                    int chunk_size, int dtype);

/*
 * gla_chunk_fwd with a sequence split for inputs whose (sequence, head, 64-column
 * slice) work items do not fill the device: each sequence is cut into segments
 * of whole 64-token chunks, the segment count chosen by gla_split_plan (bf16
 * work items of a split cover 128 columns of d_v when d_v is a multiple of 128,
 * else 64).  The recurrence is linear in the state
 * with a diagonal transition, so over one segment S_end = diag(a) S_start +
 * S_zero, with a = exp(sum of the segment's g) and S_zero the state reached
 * from zero (page "Gated Linear Attention (GLA) ...", section "The Gated
 * Recurrent Update", unrolled over the segment).  The call runs three kernels
 * on the stream: S_zero and a for every segment in parallel; a scan over the
 * segments giving every incoming state and the final states; the forward pass
 * of every segment from its incoming state.  Results equal gla_chunk_fwd's up
 * to rounding.
 *
 *   workspace       device buffer of at least gla_chunk_fwd_workspace_size(...)
 *                   bytes, 256-byte aligned, owned by the caller; its contents
 *                   are scratch, used until the call's kernels complete (the
 *                   caller must not reuse it before that on another stream).
 *                   May be NULL when that size is 0.
 *   workspace_bytes its size.
 *
 * Other arguments, layouts and errors as for gla_chunk_fwd; a missing, small or
 * misaligned workspace gives GLA_ERR_INVALID_ARG.  Packed sequences, fp32 and
 * shapes that already fill the device run unsplit, exactly as gla_chunk_fwd.
 */
int gla_chunk_fwd_ws(const void* q, const void* k, const void* v, const void* g,
                     const float* initial_state, void* o, float* final_state,
                     const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk,
                     int dv, int chunk_size, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Size, in bytes, of the scratch array behind gla_chunk_fwd_noalloc. */
#define GLA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * gla_chunk_fwd_ws for callers that cannot allocate device memory and cannot
 * bring a workspace: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  The same plan, kernels and results as
 * gla_chunk_fwd_ws, bitwise; the split's scratch (segment states and decays)
 * lives in a file-scope device array of GLA_NOALLOC_SCRATCH_BYTES owned by the
 * library, one copy per device, held from the library's load until the process
 * ends.  The call itself allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); its first call on a device looks the array's device address
 * up once (hipGetSymbolAddress).
 *
 * Every call on one device shares that device's array, and the kernels of one
 * call use it until they complete: calls that overlap on one device (on
 * different streams, or from different threads without ordering) race and give
 * wrong results.  Calls on one stream are ordered and safe.  The array keeps the
 * last call's contents; no call depends on them (every element a call reads, an
 * earlier kernel of the same call wrote).
 *
 * Arguments, layouts and errors as for gla_chunk_fwd.  Shapes whose split would
 * need more scratch than GLA_NOALLOC_SCRATCH_BYTES (the sizes of
 * gla_chunk_fwd_workspace_size) give GLA_ERR_INVALID_ARG with nothing enqueued;
 * shapes that run unsplit need none.  A failed address lookup gives
 * GLA_ERR_LAUNCH.
 */
int gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g,
                          const float* initial_state, void* o, float* final_state,
                          const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk,
                          int dv, int chunk_size, int dtype, void* stream);

/*
 * The segment count that gla_chunk_fwd_ws, gla_chunk_fwd_noalloc and the size
 * query gla_chunk_fwd_workspace_size use for fixed-length bf16 inputs of units
 * = B x H (sequence, head) pairs of T tokens and d_v = dv columns on a device
 * with num_cus compute units; 1 means the call runs unsplit.  *seg_len (if not
 * NULL) receives the segment length in tokens, a multiple of 64 (T when
 * unsplit); the last segment may be shorter.  Host-only: no GPU is touched.
 *
 * The choice minimises a cost model (page "Qwen Team Releases FlashQLA for
 * High-Performance Linear Attention", section "Core Technical Principles"): in
 * the "one wave" case a split's per-segment passes cost lambda_1 per chunk of
 * segment length L and its scan across segments lambda_2 per segment, so
 * T = lambda_1 L + lambda_2 N / L for N chunks; plus lambda_0 per split call,
 * against mu_1 N + mu_0 unsplit.  The constants are fitted on MI355X.  Splits
 * are considered only when units x dv / 64 < num_cus, and only for segment
 * counts whose work items fit one wave.  dtype other than GLA_BF16, T <= 0,
 * units <= 0 or dv not a positive multiple of 64 give 1.
 */
int gla_split_plan(long long units, int T, int dv, int dtype, int num_cus, int* seg_len);

/*
 * The d_v slice width, 64 or 128 value columns per work item, that the unsplit
 * forward (gla_chunk_fwd, and gla_chunk_fwd_ws / gla_chunk_fwd_noalloc when they
 * do not split) takes for units = Nseq x H (sequence, head) pairs, dv value
 * columns and dtype on a device with num_cus compute units.  Host-only.
 *
 * A work item holds a compute unit for its whole sequence, so a call runs in
 * rounds of num_cus items; a last partial round with a fraction f of the units
 * busy counts 0.5 + 0.5 f of a full round, and a round of 128-column items 1.8
 * rounds of 64-column items (both ratios measured on MI355X).  The result is
 * 128 when 1.8 x rounds(units x dv / 128) < rounds(units x dv / 64), else 64;
 * always 64 unless dtype is GLA_BF16 and dv a positive multiple of 128, and
 * for units <= 0 or num_cus <= 0.
 */
int gla_slice_plan(long long units, int dv, int dtype, int num_cus);

/*
 * Device workspace, in bytes, that gla_chunk_fwd_segments needs: 0 when
 * num_segments gives one segment, else (segment states B x H x segments x dk x dv
 * fp32 and decays B x H x segments x dk fp32, each rounded up to 256 bytes).
 * Invalid shapes or num_segments outside [1, ceil(T / 64)] give 0.
 */
size_t gla_chunk_fwd_segments_workspace_size(int B, int H, int T, int dk, int dv, int num_segments);

/*
 * The sequence split of gla_chunk_fwd_ws with a segment count the caller
 * chooses (as a fixed context-parallel degree is chosen by hand across GPUs),
 * for fixed-length inputs (no cu_seqlens).  Each sequence is cut into segments
 * of L = ceil(ceil(T / 64) / num_segments) whole chunks; the segment count used
 * is ceil(ceil(T / 64) / L), at most num_segments.  One segment runs unsplit as
 * gla_chunk_fwd (any dtype); more need bf16 (else GLA_ERR_UNSUPPORTED).
 *
 *   num_segments    1 .. ceil(T / 64), else GLA_ERR_INVALID_ARG.
 *   workspace       device buffer of at least
 *                   gla_chunk_fwd_segments_workspace_size(...) bytes, 256-byte
 *                   aligned, as for gla_chunk_fwd_ws.
 *
 * Other arguments, layouts and errors as for gla_chunk_fwd_ws.  Results equal
 * gla_chunk_fwd's up to rounding for every segment count.
 */
int gla_chunk_fwd_segments(const void* q, const void* k, const void* v, const void* g,
                           const float* initial_state, void* o, float* final_state, int B, int H,
                           int T, int dk, int dv, int chunk_size, int dtype, int num_segments,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device workspace, in bytes, that gla_chunk_bwd needs for this shape: the bf16
 * state entering every 64-token chunk (H x (sequences + tokens/64 + 1) slots of
 * dk x dv, rounded up to 256), the sequence split's state gradients when the
 * call splits, and for dv above 128 fp32 partial sums of dq, dk and dg
 * (3 x H x tokens x dk floats).  num_seqs > 0 for packed sequences (then T is
 * the packed total), 0 otherwise.  Unsupported shapes give 0.
 */
size_t gla_chunk_bwd_workspace_size(int num_seqs, int B, int H, int T, int dk, int dv,
                                    int chunk_size, int dtype);

/*
 * Chunkwise backward pass: the gradients of
 *
 *     L = sum_t <d_o_t, o_t> + <d_final_state, S_T>
 *
 * for the forward computed by gla_chunk_fwd on the same arguments, i.e. the
 * training half that the GLA page's section "I/O-Aware Kernel Design in
 * FlashLinearAttention" pairs with the chunkwise forward (chunk states are
 * recomputed here, not kept from the forward call).
 *
 *   q, k, g, v       as for gla_chunk_fwd (GLA_BF16 only)
 *   initial_state    [Nseq, H, dk, dv] fp32 or NULL (zeros), as in the forward
 *   d_o              [B, H, T, dv] bf16: gradient of the outputs
 *   d_final_state    [Nseq, H, dk, dv] fp32 or NULL (zeros): gradient of S_T
 *   d_q, d_k, d_g    [B, H, T, dk] bf16, written (d_g is the gradient of g = log alpha)
 *   d_v              [B, H, T, dv] bf16, written
 *   d_initial_state  [Nseq, H, dk, dv] fp32 or NULL (not written): gradient of S_0
 *   cu_seqlens, num_seqs, B, H, T, chunk_size   as for gla_chunk_fwd
 *   workspace        device buffer of at least gla_chunk_bwd_workspace_size(...)
 *                    bytes, 256-byte aligned, owned by the caller; scratch until
 *                    the call's kernels complete.
 *
 * Supported: dtype GLA_BF16, dk in {64, 128}, dv a multiple of 64, chunk_size 64;
 * others give GLA_ERR_UNSUPPORTED.  dv above 128 runs as column slices of 128 (the
 * last one 64 for an odd multiple of 64), one kernel launch each, in order on the
 * stream: dq, dk and dg are sums over the slices, kept in the workspace in fp32
 * until the last slice rounds them to bf16.  A missing, small or misaligned
 * workspace gives
 * GLA_ERR_INVALID_ARG.  Gates must keep every channel's decay over any 16
 * consecutive tokens of a sequence at or above 2^-240 (so alpha = 0 is not
 * supported here); a sequence that breaks this gets NaN gradients.
 */
int gla_chunk_bwd(const void* q, const void* k, const void* v, const void* g,
                  const float* initial_state, const void* d_o, const float* d_final_state,
                  void* d_q, void* d_k, void* d_v, void* d_g, float* d_initial_state,
                  const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk, int dv,
                  int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * The forward of gla_chunk_fwd (unsplit, 64-column d_v slices) that also writes
 * the bf16 state entering every 64-token chunk, in the layout and place the
 * backward's chunk-state pass uses: chunk_states is the workspace a later
 * gla_chunk_bwd_saved call on the same inputs is given (at least
 * gla_chunk_bwd_workspace_size(...) bytes, 256-byte aligned, owned by the
 * caller; this call writes its chunk-state part).  The states are the ones
 * gla_chunk_bwd computes for itself, bitwise; o and final_state are gla_chunk_fwd's,
 * up to the slice width (bitwise where gla_chunk_fwd also takes 64 columns).
 * Same recurrence as gla_chunk_fwd (page "Gated Linear Attention (GLA) ...",
 * section "The Gated Recurrent Update"), one state per chunk boundary.
 *
 * Arguments, layouts and errors as for gla_chunk_fwd, with the backward's limits:
 * dtype GLA_BF16, dk in {64, 128} and dv a multiple of 64, else
 * GLA_ERR_UNSUPPORTED; a missing,
 * small or misaligned chunk_states buffer gives GLA_ERR_INVALID_ARG.
 */
int gla_chunk_fwd_states(const void* q, const void* k, const void* v, const void* g,
                         const float* initial_state, void* o, float* final_state,
                         const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk,
                         int dv, int chunk_size, int dtype, void* chunk_states,
                         size_t chunk_states_bytes, void* stream);

/*
 * gla_chunk_bwd for a workspace whose chunk states a gla_chunk_fwd_states call on
 * the same k, v, g, initial_state and cu_seqlens has already written: the chunk-
 * state pass is skipped, everything else (the sequence split's passes, the
 * gradients) runs as in gla_chunk_bwd, with the same results.  Arguments and
 * errors as for gla_chunk_bwd.  Different inputs, or a workspace written for
 * another shape, give wrong gradients without an error.
 */
int gla_chunk_bwd_saved(const void* q, const void* k, const void* v, const void* g,
                        const float* initial_state, const void* d_o, const float* d_final_state,
                        void* d_q, void* d_k, void* d_v, void* d_g, float* d_initial_state,
                        const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk, int dv,
                        int chunk_size, int dtype, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * One recurrent decode step for N sequences x H heads, in place on the state.
 *
 *   q, k, g  [N, H, dk]  dtype;   v  [N, H, dv]  dtype
 *   state    [N, H, dk, dv] fp32, read and overwritten with S_t
 *   o        [N, H, dv]  dtype, written (o = q S_t with the updated state)
 *
 * Supported: dk in {64, 128, 256}, dv in {64, 128, 256}, both dtypes.
 */
int gla_recurrent_step(const void* q, const void* k, const void* v, const void* g,
                       float* state, void* o, int N, int H, int dk, int dv, int dtype,
                       void* stream);

/*
 * Chunkwise Gated DeltaNet forward (page "Qwen Team Releases FlashQLA for
 * High-Performance Linear Attention": the GDN update with a forget gate alpha
 * and an update gate beta per token, the transition I - beta k k^T, and its
 * chunkwise WY form).  For every unit (sequence, head) and token t in order:
 *
 *     S_t = alpha_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t,
 *     o_t = q_t S_t,            alpha_t = exp(g_t),
 *
 * S a dk x dv fp32 matrix, k_t a row vector.  The keys are meant to have unit
 * L2 norm (not checked); beta in [0, 1], g <= 0 (not checked; g = -inf is
 * allowed and acts as alpha = 0).  Accuracy: the chunk form runs its products
 * on bf16 operands with fp32 accumulation (scores, the triangular solve's
 * right-hand sides and solution, the state), which gives about 1e-2 relative
 * error or less for independent keys.  Keys that all share one direction with
 * beta near 1 make the solve ill-conditioned for bf16 operands: about 2e-2
 * relative error at beta = 1.  The fp32 inverses of the 16-token diagonal
 * blocks are good to about 2e-3 relative while beta |k|^2 <= 1 (where
 * I - beta k^T k is a contraction), about 3% at beta |k|^2 = 2.
 *
 *   q, k          [B, H, T, dk]  bf16        v, o  [B, H, T, dv]  bf16
 *   g, beta       [B, H, T]      fp32 (one value per token and head)
 *   initial_state [Nseq, H, dk, dv] fp32 or NULL (zeros)
 *   final_state   [Nseq, H, dk, dv] fp32 or NULL (not written); may alias
 *                 initial_state
 *   cu_seqlens    packed sequences exactly as for gla_chunk_fwd (B == 1,
 *                 device int32 [num_seqs + 1]); NULL for fixed length
 *
 * q, k, v, o, the states and cu_seqlens must be 16-byte aligned, g and beta
 * 4-byte aligned, all contiguous device memory owned by the caller.  The call
 * only enqueues work on `stream` (a hipStream_t; NULL is the null stream), keeps
 * no pointer and allocates nothing.  Supported: dtype GLA_BF16, dk in {64, 128},
 * dv a multiple of 64 up to 512, chunk_size 64; others give GLA_ERR_UNSUPPORTED.
 */
int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                  const float* initial_state, void* o, float* final_state,
                  const int32_t* cu_seqlens, int num_seqs, int B, int H, int T, int dk, int dv,
                  int chunk_size, int dtype, void* stream);

/* Static, human-readable name of a gla_status value. */
const char* gla_status_string(int status);

/* Detail of the calling thread's last non-OK return ("" if none). */
const char* gla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H_ */
