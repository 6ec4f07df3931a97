/*
 * muir.h -- C ABI of the Muir gated delta-rule operator on AMD Instinct
 * MI355X (gfx950).
 *
 * The operator (arXiv 2611.08376, "Muir: Linear Attention with
 * Sensitivity-Allocated Gating and Matched-Filter Readout"; abstract and the
 * Methodology section of the wolonglab summary page) keeps, per batch row b
 * and head h, a state S in R^{dk x dv} (rows = key channels) and for every
 * token t:
 *
 *   S'_t = diag(exp(log_a_t)) S_{t-1}                      row-wise decay
 *   d_t  = write_t * v_t - S'_t^T (erase_t * k_t)          erase the key's prediction
 *   S_t  = S'_t + k_t d_t^T                                gated write
 *   o_t  = S_t^T (gamma_t * q_t)                           readout gate on the query
 *
 * q and k are expected unit-normalised by the caller (the pages normalise
 * them before the operator); the library does not normalise.
 *
 * Training runs the recurrence chunkwise: each chunk of `chunk` tokens is a
 * triangular system whose cumulative log-decay is split at interval
 * boundaries so every exponential factor lies in (0, 1] (Methodology;
 * fig:kernel caption).  Decode is the single-token recurrence.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer to dense, contiguous memory,
 *    aligned to 16 bytes.  Inputs and o/dO use the element type `dtype`
 *    (MUIR_F32 or MUIR_BF16); the gradients of the inputs use `grad_dtype`
 *    (fp32 by default, bf16 on request for bf16 inputs); states and state
 *    gradients are fp32; the workspace's content is opaque.
 *  - Sequence tensors are [B, T, H, D] with D contiguous; states are
 *    [B, H, dk, dv] row-major (dv contiguous).
 *  - The caller owns every buffer, including the workspace; the library
 *    never allocates, frees or synchronises, and keeps no state between
 *    calls, with two exceptions stated where they apply: the no-allocation
 *    forward's fixed scratch array, and the hipBLASLt handle and plans of
 *    the bf16 gate projection.  Calls are asynchronous on `stream` (a
 *    hipStream_t; NULL is the default stream).  Calls on different streams with disjoint buffers may
 *    run concurrently.
 *  - Outputs must not alias inputs (muir_step's S is updated in place by
 *    design).
 *  - Argument errors are detected before any launch and returned as a
 *    status; nothing is launched then.  A launch failure returns
 *    MUIR_ERR_HIP.  On error, outputs are undefined.  No C++ exception
 *    crosses this interface.
 *  - log_a must be finite and <= 0.  "No decay" is log_a = 0; "full decay"
 *    is a large negative value (e.g. -1e4), for which exp() is 0.
 *  - Supported sizes: dk == dv, dk in {64, 128}; chunk in {64, 128, 256};
 *    any T >= 0.  A T that is not a multiple of chunk ends in a partial
 *    chunk: the call then runs on zero-padded copies of the sequences in its
 *    workspace (a zero token leaves the state unchanged) and needs a larger
 *    workspace.  Sizes B, T, H may be 0 (no sequence work is launched).
 *  - nc = ceil(T / chunk) is the number of chunks of a sequence.
 */
#ifndef MUIR_H_
#define MUIR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MUIR_OK = 0,
  MUIR_ERR_NULL = 1,      /* a required pointer is NULL */
  MUIR_ERR_SHAPE = 2,     /* unsupported or inconsistent sizes */
  MUIR_ERR_DTYPE = 3,     /* unknown dtype code */
  MUIR_ERR_WORKSPACE = 4, /* workspace pointer NULL or smaller than required */
  MUIR_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned */
  MUIR_ERR_HIP = 6,       /* a kernel launch failed */
  MUIR_ERR_MODE = 7,      /* unknown readout-gate mode */
  MUIR_ERR_SCRATCH = 8,   /* more work than the fixed scratch of a no-allocation call holds */
  MUIR_ERR_NONFINITE = 9  /* an input breaks its precondition: NaN or infinite values, or log_a > 0
                             (reported by the checks built on muir_check_values, never by the
                             compute calls, which do not read their inputs on the host) */
} muir_status_t;

typedef enum { MUIR_F32 = 0, MUIR_BF16 = 1 } muir_dtype_t;

/*
 * Form of the readout gate gamma (wolonglab summary, §Methodology and
 * tab:abl: dynamic, static or no readout gate).
 *   MUIR_GAMMA_TOKEN : per token, [B, T, H, dk] (decode: [N, H, dk]) dtype;
 *                      its gradient has the same shape, in grad_dtype
 *   MUIR_GAMMA_STATIC: one per (head, key channel), [H, dk] dtype; its
 *                      gradient is [H, dk] fp32, summed over batch and tokens
 *   MUIR_GAMMA_NONE  : gamma = 1; the gamma and dgamma pointers are not used
 *                      and may be NULL
 */
typedef enum { MUIR_GAMMA_TOKEN = 0, MUIR_GAMMA_STATIC = 1, MUIR_GAMMA_NONE = 2 } muir_gamma_mode_t;

/*
 * Sizes of a chunkwise call.  `grad_dtype` is the element type of the
 * per-token gradients that the backward writes (dq, dk, dv, dlog_a, derase,
 * dwrite and a per-token dgamma): MUIR_F32 (0, so a zero-initialised struct
 * asks for fp32 gradients) or, with dtype MUIR_BF16 only, MUIR_BF16 (each
 * gradient accumulated in fp32 and rounded once on the store).  The forward
 * calls ignore it.
 */
typedef struct {
  int32_t B, T, H;     /* batch, tokens, heads */
  int32_t dk, dv;      /* key / value head size */
  int32_t chunk;       /* tokens per triangular system */
  int32_t dtype;       /* muir_dtype_t of q, k, v, gates, o, dO */
  int32_t gamma_mode;  /* muir_gamma_mode_t */
  int32_t grad_dtype;  /* muir_dtype_t of the per-token gradients (backward) */
} muir_dims_t;

/* Version of this interface (bumped on any signature change). */
int32_t muir_abi_version(void);

/*
 * Per-kernel timing for profilers and benchmarks.  `events` points to
 * `count` hipEvent_t handles created by the caller (hipEventCreate).  After
 * registration, each entry point records the next unused event on its
 * stream before its first kernel and after each kernel it launches, until
 * all `count` events are used.  Registering (NULL, 0) turns this off.  The
 * registration is per host thread; the events stay owned by the caller.
 * Returns MUIR_OK, or MUIR_ERR_NULL for (NULL, count > 0).
 */
int32_t muir_set_profile_events(void** events, int32_t count);

/* Events recorded since the last muir_set_profile_events on this thread. */
int32_t muir_profile_events_recorded(void);

/* Human-readable text for a status code (static storage; never NULL). */
const char* muir_status_string(muir_status_t status);

/*
 * Debug check of one input tensor against the operator's preconditions
 * (every value finite; a log-decay at most 0, since a decay exp(log_a) above
 * 1 would make the recurrence grow without bound).  Adds to counts[0] the
 * number of NaN or infinite values among the n elements of x (dtype), and,
 * when log_decay is nonzero, to counts[1] the number of finite values above 0.
 * counts is an int32 [2] DEVICE array that the call only adds to, so one
 * zeroed array can gather several tensors; read it back after the stream has
 * run the call.  Asynchronous; x needs no particular alignment beyond its
 * element size.  n == 0 launches nothing.  Meant for debugging: a caller
 * that reads the counts back synchronises with the stream.
 */
muir_status_t muir_check_values(int64_t n, int32_t dtype, const void* x, int32_t log_decay,
                                int32_t* counts, void* stream);

/* Bytes of workspace muir_chunk_fwd needs for `dims` (0 if dims are invalid). */
size_t muir_chunk_fwd_workspace(const muir_dims_t* dims);

/*
 * Chunkwise forward over T tokens (Methodology: each chunk is a triangular
 * system with boundary-split cumulative log-decay).
 *
 *   q, k, log_a, erase : [B, T, H, dk]  dtype
 *   gamma              : by dims->gamma_mode: [B, T, H, dk] or [H, dk] dtype,
 *                        or unused (NULL allowed) for MUIR_GAMMA_NONE
 *   v, write           : [B, T, H, dv]  dtype
 *   S0       : [B, H, dk, dv] fp32 initial state, or NULL for zeros
 *   o        : [B, T, H, dv]  dtype, output
 *   S_T      : [B, H, dk, dv] fp32 final state, or NULL to skip
 *   S_chunks : [B, H, nc, dk, dv] dtype: the state at the START of every
 *              chunk, rounded once to the input type (kept for
 *              muir_chunk_bwd, which takes the state in that type), or NULL
 *              to skip.  Each [dk, dv] state is stored as 16 x 16 tiles:
 *              element (r, j) is at ((r/16) * (dv/16) + j/16) * 256 +
 *              (r%16) * 16 + j%16 of its state (each tile row-major).
 *   workspace: device scratch of at least muir_chunk_fwd_workspace(dims)
 *              bytes.  On return it holds the chunk summaries (the
 *              per-chunk solve results; with S_chunks also each chunk's
 *              deltas when dtype is MUIR_BF16) and, when few heads make the
 *              state scan split the sequence into segments, each segment's
 *              state transition; a caller that keeps it unchanged may pass
 *              it to muir_chunk_bwd as `summaries`, together with S_chunks.
 */
muir_status_t muir_chunk_fwd(const muir_dims_t* dims,
                             const void* q, const void* k, const void* v,
                             const void* log_a, const void* erase,
                             const void* write, const void* gamma,
                             const float* S0, void* o, float* S_T, void* S_chunks,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * No-allocation forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  It is muir_chunk_fwd (same arguments, results and errors)
 * with its workspace taken from a fixed scratch array of
 * MUIR_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on,
 * from the first such call on that GPU until the process ends; the call
 * itself allocates and frees nothing.  The caller still passes every input
 * and output.
 *   - A call for which muir_chunk_fwd_workspace(dims) exceeds
 *     MUIR_NOALLOC_SCRATCH_BYTES returns MUIR_ERR_SCRATCH and launches
 *     nothing.  At dk = dv = 128, bf16, chunk 64 a call needs about 2.4 to
 *     3.2 KB per token and head (more when few heads split the state scan
 *     into segments): one 2,048-token sequence of 16 heads takes 98 MiB.
 *   - Every call on one GPU uses that GPU's one array.  Calls that overlap in
 *     time on the same GPU (other streams or host threads) race on it; the
 *     caller serialises them.  Successive calls on one stream are ordered.
 *   - What the array holds after a call is not part of the interface: it
 *     cannot be passed to muir_chunk_bwd as `summaries`.
 */
#define MUIR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
muir_status_t muir_chunk_fwd_noalloc(const muir_dims_t* dims,
                                     const void* q, const void* k, const void* v,
                                     const void* log_a, const void* erase,
                                     const void* write, const void* gamma,
                                     const float* S0, void* o, float* S_T, void* S_chunks,
                                     void* stream);

/* Bytes of workspace muir_chunk_bwd needs for `dims` (0 if dims are invalid). */
size_t muir_chunk_bwd_workspace(const muir_dims_t* dims);

/*
 * Chunkwise backward: gradients of sum(dO * o) + sum(dS_T * S_T) with
 * respect to every input of muir_chunk_fwd (the pages state only that a
 * custom backward pass is used; this is the adjoint of the recurrence above).
 *
 *   inputs as in muir_chunk_fwd, plus
 *   S_chunks : [B, H, nc, dk, dv] dtype from muir_chunk_fwd, or NULL
 *              (then recomputed inside, in the workspace)
 *   summaries: the workspace of a muir_chunk_fwd call on the same inputs,
 *              dims and S0, unchanged since (the chunk summaries and segment
 *              transitions it left there), or NULL (then recomputed inside,
 *              in the workspace); read only.  With dtype MUIR_BF16 the backward also reads the
 *              chunk deltas that the forward keeps when it saves S_chunks:
 *              there summaries and S_chunks are used only together, from the
 *              same muir_chunk_fwd call, and both are recomputed when either
 *              is NULL.
 *   dO       : [B, T, H, dv] dtype upstream gradient of o
 *   dS_T     : [B, H, dk, dv] fp32 upstream gradient of S_T, or NULL for 0
 *   dq, dk, dlog_a, derase : [B, T, H, dk] grad_dtype outputs
 *   dv, dwrite             : [B, T, H, dv] grad_dtype outputs
 *              (accumulated in fp32; in bf16 rounded once on the store)
 *   dgamma   : by dims->gamma_mode: [B, T, H, dk] grad_dtype; [H, dk] fp32
 *              (the sum over batch and tokens, in a fixed order); unused
 *              (NULL allowed) for MUIR_GAMMA_NONE
 *   A grad_dtype other than MUIR_F32 or, for bf16 inputs, MUIR_BF16 returns
 *   MUIR_ERR_DTYPE.
 *   dS0      : [B, H, dk, dv] fp32 output, or NULL to skip
 *   workspace: device scratch of at least muir_chunk_bwd_workspace(dims)
 *              bytes; contents are clobbered.
 */
muir_status_t muir_chunk_bwd(const muir_dims_t* dims,
                             const void* q, const void* k, const void* v,
                             const void* log_a, const void* erase,
                             const void* write, const void* gamma,
                             const float* S0, const void* S_chunks, const void* summaries,
                             const void* dO, const float* dS_T,
                             void* dq, void* dk, void* dv, void* dlog_a,
                             void* derase, void* dwrite, void* dgamma, float* dS0,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Packed variable-length sequences (the pages train on documents of mixed
 * length; packing them end to end without padding is the usual layout).
 * Sequence n is rows cu_seqlens[n] .. cu_seqlens[n+1]-1 of every sequence
 * tensor, which is [T_total, H, D] with T_total = cu_seqlens[B]; each
 * sequence starts from its own state and none sees another's tokens.
 *
 *   dims       : B = number of sequences, T = an upper bound on every
 *                sequence's length (the longest one); the other fields as
 *                for muir_chunk_fwd.  The workspace size depends on B * T.
 *   cu_seqlens : [B + 1] int32 DEVICE array, cu_seqlens[0] = 0 and
 *                non-decreasing.  Precondition (not checked, as the array is
 *                on the device): every length is <= dims->T.  If one is
 *                longer, the call still reads and writes only the given
 *                tensors and its workspace, but its results are unspecified.
 *   q, k, log_a, erase, (per-token) gamma : [T_total, H, dk] dtype
 *   v, write, o                           : [T_total, H, dv] dtype
 *   S0, S_T    : [B, H, dk, dv] fp32 per sequence, as in muir_chunk_fwd
 * The call copies the sequences into one sequence in its workspace, each
 * starting at a chunk boundary and zero-padded to its last chunk's end; the
 * scans start each sequence from its own S0 and end it at its own S_T, and
 * the chunk kernels see only the sequences' own chunks.  It then copies the
 * real tokens' results back.  (Shapes whose B * T_pad reaches 2^31 rows, with
 * T_pad = T rounded up to the chunk, run on zero-padded [B, T_pad, H, D]
 * copies instead.)
 *   keep       : nonzero: the chunk-start states are saved and, with the
 *                chunk summaries, the packed inputs and the packing plan,
 *                left in the workspace, which the backward of the same
 *                sequences may then take as fwd_workspace instead of
 *                recomputing them; 0: not saved.  (The padded form ignores
 *                it.)  The workspace size does not depend on it.
 */
size_t muir_chunk_varlen_fwd_workspace(const muir_dims_t* dims);

muir_status_t muir_chunk_varlen_fwd(const muir_dims_t* dims, const int32_t* cu_seqlens,
                                    const void* q, const void* k, const void* v,
                                    const void* log_a, const void* erase,
                                    const void* write, const void* gamma,
                                    const float* S0, void* o, float* S_T, int32_t keep,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of muir_chunk_varlen_fwd: as muir_chunk_bwd, with the packed
 * layout and cu_seqlens of muir_chunk_varlen_fwd for every sequence tensor
 * (dO is [T_total, H, D] dtype, the per-token gradients [T_total, H, D]
 * grad_dtype).  dS_T and dS0 are
 * [B, H, dk, dv] per sequence; a static gate's gradient is [H, dk] fp32,
 * summed over every sequence's tokens.
 *   fwd_workspace : NULL, or the workspace of a muir_chunk_varlen_fwd call
 *                   with keep != 0 on the same dims, cu_seqlens, inputs and
 *                   S0, left unchanged since: its packed inputs, summaries and
 *                   chunk-start states are read instead of formed again
 *                   (results equal bit for bit).  16-byte aligned.  (The
 *                   padded form ignores it.)
 */
size_t muir_chunk_varlen_bwd_workspace(const muir_dims_t* dims);

muir_status_t muir_chunk_varlen_bwd(const muir_dims_t* dims, const int32_t* cu_seqlens,
                                    const void* q, const void* k, const void* v,
                                    const void* log_a, const void* erase,
                                    const void* write, const void* gamma,
                                    const float* S0, const void* dO, const float* dS_T,
                                    void* dq, void* dk, void* dv, void* dlog_a,
                                    void* derase, void* dwrite, void* dgamma, float* dS0,
                                    const void* fwd_workspace,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step of the recurrence for N independent streams (abstract:
 * constant-memory inference; the state stays fp32).
 *
 *   q, k, log_a, erase : [N, H, dk] dtype
 *   gamma              : by gamma_mode (muir_gamma_mode_t): [N, H, dk] or
 *                        [H, dk] dtype, or unused (NULL allowed)
 *   v, write           : [N, H, dv] dtype
 *   S : [N, H, dk, dv] fp32, read and updated in place (S_{t-1} -> S_t)
 *   o : [N, H, dv] dtype, output o_t
 * Supported sizes: dk in {64, 128}, dv a multiple of 64.
 */
muir_status_t muir_step(int32_t N, int32_t H, int32_t dk, int32_t dv, int32_t dtype,
                        int32_t gamma_mode, const void* q, const void* k, const void* v,
                        const void* log_a, const void* erase,
                        const void* write, const void* gamma,
                        float* S, void* o, void* stream);

/*
 * Gate prologue (wolonglab summary page, §Methodology and fig:arch (b), (c)):
 * the five per-token gates come from ONE low-rank projection of the
 * token's input x -- a shared down-projection to 512 channels, split into
 * rank slices (64, 64, 128, 128, 128) for the gates (f, b, g, w, q) in that
 * order, each slice up-projected to its gate's width plus a per-channel bias:
 *
 *   z      = x W_down^T                                 [M, 512]
 *   pre_i  = z[:, slice_i] U_i^T + c_i
 *   log_a  = log sigmoid(pre_f)   [M, H, dk]   (decay; <= 0)
 *   erase  = sigmoid(pre_b)       [M, H, dk]
 *   g      = sigmoid(pre_g)       [M, H, dv]   (output gate, used after the operator)
 *   write  = sigmoid(pre_w)       [M, H, dv]
 *   gamma  = 2 sigmoid(pre_q)     [M, H, dk]   (readout gain)
 *
 * The activations are readings (the pages name the gates, not their
 * nonlinearities).  Layouts (row-major, dtype unless stated; weights in a
 * linear layer's [out, in] layout):
 *   x      : [M, d] tokens (M = B * T)
 *   W_down : [512, d]
 *   W_up   : the five U_i back to back: U_f [H*dk, 64], U_b [H*dk, 64],
 *            U_g [H*dv, 128], U_w [H*dv, 128], U_q [H*dk, 128]
 *   bias   : the five c_i back to back: [H*dk], [H*dk], [H*dv], [H*dv], [H*dk]
 * Supported sizes: d a multiple of 64 up to 65536; dk, dv in {64, 128}.
 */
typedef struct {
  int32_t M;      /* tokens */
  int32_t d;      /* width of x */
  int32_t H;      /* heads */
  int32_t dk, dv; /* key / value channels per head */
  int32_t dtype;  /* muir_dtype_t of x, the weights, z, the gates and their gradients */
} muir_gate_dims_t;

/*
 * Forward: writes z (kept for the backward) and the five gates.  All
 * pointers are required.  M == 0 launches nothing.
 *
 * For bf16, the two plain products z = x W_down^T (here, and in the
 * backward when z is NULL) and dx = dz W_down run through hipBLASLt.  The
 * first such call on a device creates that device's hipBLASLt handle, and
 * the first call of each shape its plan (descriptors and the algorithm the
 * library's heuristic picks); both are kept until the process ends, and
 * hipBLASLt makes its own host allocations and loads its kernels for them.
 * Later calls of a known shape allocate nothing, so a caller that captures
 * these calls into a graph makes one call of each shape first.  A shape
 * for which hipBLASLt has no algorithm needing no workspace runs this
 * library's own GEMM kernel.
 */
muir_status_t muir_gate_proj_fwd(const muir_gate_dims_t* dims, const void* x, const void* W_down,
                                 const void* W_up, const void* bias, void* z, void* log_a,
                                 void* erase, void* g, void* write, void* gamma, void* stream);

/* Bytes of workspace muir_gate_proj_bwd needs (0 if dims are invalid). */
size_t muir_gate_proj_bwd_workspace(const muir_gate_dims_t* dims);

/*
 * Backward: from the gradients of the five gates (shaped like the gates,
 * dtype) to dx [M, d] (dtype, overwritten), and dW_down [512, d], dW_up
 * and dbias (fp32, packed like W_up and bias, overwritten; sums over tokens
 * in a fixed order).  z is the forward's z, or NULL to recompute it.  Every
 * other pointer is required; the workspace is clobbered.
 */
muir_status_t muir_gate_proj_bwd(const muir_gate_dims_t* dims, const void* x, const void* W_down,
                                 const void* W_up, const void* bias, const void* z,
                                 const void* dlog_a, const void* derase, const void* dg,
                                 const void* dwrite, const void* dgamma, void* dx, float* dW_down,
                                 float* dW_up, float* dbias, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * End of the q / k pathways (fig:arch (b); the operator takes unit keys and
 * queries): for each of `rows` vectors u of D values (one head),
 *   y = s / sqrt(sum s^2 + 1e-6),  s = u * sigmoid(u)  (SiLU).
 * u, y, dy, du: [rows, D] dtype; D in {64, 128}.  muir_qk_norm_bwd writes
 * du, the gradient of sum(dy * y) with respect to u.
 */
muir_status_t muir_qk_norm_fwd(int64_t rows, int32_t D, int32_t dtype, const void* u, void* y,
                               void* stream);
muir_status_t muir_qk_norm_bwd(int64_t rows, int32_t D, int32_t dtype, const void* u, const void* dy,
                               void* du, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MUIR_H_ */
