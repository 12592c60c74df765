/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 chunked-SSD forward.
 *
 * Pages cited (by title):
 *   P1 = "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
 *         Tensor Cores with cuTile" (disconfirmai.com digest of the NVIDIA
 *         Developer Blog post on Mamba-2 forward kernels in cuTile).
 *   P3 = "Jane Street and NVIDIA optimize three Mamba-2 forward-pass kernels in
 *         cuTile" (genainews.tech).
 *
 * The operation.  Per batch b and head h, with group g = h / (H/G), the state
 * h_t (N x P) and output y_t (P) follow
 *     h_t = exp(dt[b,t,h] A[h]) h_{t-1} + dt[b,t,h] B[b,t,g,:] x[b,t,h,:]^T
 *     y_t = C[b,t,g,:]^T h_t + D[h] x[b,t,h,:]
 * evaluated chunk by chunk (chunk length Q, nc = ceil(L/Q) chunks) in the three
 * steps P1 describes in its paragraph on the three kernels: a log-space
 * cumulative sum of the decay term, the jump-formula state advance across
 * chunks, and the fused output (carried-state term, decayed causally masked
 * C.B^T interaction applied to x, skip connection).  The state advance is
 * exported as two calls here: the per-chunk states (parallel over chunks) and
 * the sequential pass that carries them across chunks.
 *
 * Conventions for every call:
 *   - Every tensor pointer is a DEVICE pointer to dense row-major memory,
 *     16-byte aligned.  The caller owns all memory; the library allocates
 *     nothing, keeps no mutable global state and is safe to call from several
 *     host threads.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Calls are asynchronous: they enqueue kernels and return without
 *     synchronising.  Buffers must stay valid until the stream reaches them.
 *   - Every argument check runs on the host BEFORE any HIP call; a failed
 *     check returns its status and enqueues nothing.  A launch failure is
 *     reported as SSD_ERR_HIP.  Values are not validated: NaN/Inf propagate.
 *   - dt, A, D, dA_cumsum, dt_bhl, initial and final states are float32; the
 *     chunk states and the carried states are F32 or BF16 (the caller's
 *     choice, `states_dtype` and `carried_dtype`; BF16 values are the fp32
 *     results rounded to nearest even).  x, B and C share one input dtype `in` (F32
 *     or BF16).
 *   - Shape limits of this version (else SSD_ERR_UNSUPPORTED): headdim P and
 *     dstate N multiples of 16 with N <= 256 and P <= 256; chunk Q in
 *     {32, 64, 128, 256}.  L need not be a multiple of Q: the last chunk is
 *     then ragged (L - (nc-1) Q tokens).  The per-chunk layouts keep Q
 *     positions per chunk; positions past the end of the sequence count as
 *     tokens with dt = 0 (dt_bhl 0, dA_cumsum constant at its last value),
 *     which adds nothing to any state or output.
 *
 * Precision modes (ssd_mma): SSD_MMA_BF16 rounds the matrix-core operands
 * (the decay-scaled x rows, the decayed interaction tile, the carried state)
 * to bfloat16, round-to-nearest-even, and accumulates in float32;
 * SSD_MMA_F32 keeps every operand in float32 (fp32 matrix instructions).
 */
#ifndef MAMBA_SSD_H
#define MAMBA_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 4

typedef enum {
  SSD_OK = 0,
  SSD_ERR_NULL = 1,         /* a required pointer is NULL */
  SSD_ERR_SHAPE = 2,        /* a size is <= 0, or nheads % ngroups != 0 */
  SSD_ERR_DTYPE = 3,        /* unknown dtype / mma enum value */
  SSD_ERR_UNSUPPORTED = 4,  /* valid shape outside this version's limits */
  SSD_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than ssd_workspace_bytes */
  SSD_ERR_ALIGN = 6,        /* a pointer is not 16-byte aligned */
  SSD_ERR_HIP = 7,          /* a kernel launch failed */
  SSD_ERR_SCRATCH = 8       /* ssd_forward_noalloc: the shape needs more than SSD_NOALLOC_SCRATCH_BYTES */
} ssd_status;

/* The *_MAX_ENUM members are not valid arguments: they give the enums the
 * range of a 32-bit int, so that an out-of-range value from a C caller is a
 * representable value that the calls reject with SSD_ERR_DTYPE. */
typedef enum { SSD_F32 = 0, SSD_BF16 = 1, SSD_DTYPE_MAX_ENUM = 0x7fffffff } ssd_dtype;
typedef enum { SSD_MMA_BF16 = 0, SSD_MMA_F32 = 1, SSD_MMA_MAX_ENUM = 0x7fffffff } ssd_mma;

/* B, L, H, P, N, G, Q in the notation above. */
typedef struct {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
} ssd_shape;

/*
 * Log-space decay cumulative sum (P1, paragraph on the three kernels: per
 * token and per head, the running sum of the decay term inside each chunk;
 * P1, Blackwell-optimisation paragraph and P3: stored token-contiguous per
 * (batch, head)).
 *   dA_cumsum[b,h,c,i] = sum_{k<=i} dt[b,cQ+k,h] * A[h]   (inclusive, fp32)
 *   dt_bhl[b,h,c,i]    = dt[b,cQ+i,h]                      (optional: NULL skips it)
 * dt [B,L,H], A [H]  ->  dA_cumsum, dt_bhl [B,H,nc,Q].
 */
ssd_status ssd_chunk_cumsum(const ssd_shape* shape, const float* dt, const float* A,
                            float* dA_cumsum, float* dt_bhl, void* stream);

/*
 * Per-chunk states by the jump formula with decay (P1, jump-formula
 * paragraph: with stacked b and x rows the state advance over a chunk is one
 * matrix product, and pre-multiplying rows by exponentials of the log-space
 * sums keeps that form):
 *   states[b,c,h] = sum_{j<Q} exp(G_{Q-1} - G_j) dt_j B_j x_j^T    (N x P)
 * with G = dA_cumsum[b,h,c,:], dt_j = dt_bhl[b,h,c,j].
 * x [B,L,H,P], Bm [B,L,G,N] (dtype `in`)  ->  states [B,nc,H,N,P], stored as
 * fp32 (states_dtype = SSD_F32) or rounded from the fp32 accumulators to
 * bf16, nearest even (SSD_BF16).
 */
ssd_status ssd_chunk_state(const ssd_shape* shape, const void* x, const void* Bm, ssd_dtype in,
                           const float* dt_bhl, const float* dA_cumsum, void* states, ssd_dtype states_dtype,
                           ssd_mma mma, void* stream);

/*
 * ssd_chunk_cumsum followed by ssd_chunk_state, as one call (the first two
 * steps of ssd_forward): dA_cumsum and dt_bhl [B,H,nc,Q] (both required here)
 * and the chunk states, bit-identical to the two calls.  Where the chunk
 * states have a head-group kernel (bf16 inputs and operands; (Q, N) in
 * {(64,128), (128,128), (256,128), (64,256), (128,256)}; P a multiple of 64)
 * that kernel computes the cumulative sums itself, in one launch.  Arguments
 * and errors as for the two calls.
 */
ssd_status ssd_chunk_cumsum_state(const ssd_shape* shape, const void* x, const void* Bm, ssd_dtype in,
                                  const float* dt, const float* A, float* dA_cumsum, float* dt_bhl, void* states,
                                  ssd_dtype states_dtype, ssd_mma mma, void* stream);

/*
 * Inter-chunk state advance (P1, paragraph on the three kernels: a sequential
 * loop over chunks advancing the hidden state).  Per (b,h):
 *   run = initial_states[b,h] (zeros when NULL)
 *   for c in 0..nc-1:  carried[b,c,h] = run;  run = exp(G_{Q-1}(c)) run + chunk_states[b,c,h]
 *   final_states[b,h] = run
 * The recurrence runs in fp32 whatever the storage dtypes: chunk_states
 * (states_dtype F32, or BF16 widened exactly) are added to an fp32 running
 * state.  carried is written as fp32 (carried_dtype = SSD_F32) or rounded to
 * bf16, nearest even (SSD_BF16).  carried may equal chunk_states (in place)
 * when the two dtypes match; aliasing with different dtypes returns
 * SSD_ERR_UNSUPPORTED.  chunk_states, carried [B,nc,H,N,P];
 * initial_states, final_states [B,H,N,P] fp32.
 */
ssd_status ssd_state_passing(const ssd_shape* shape, const void* chunk_states, ssd_dtype states_dtype,
                             void* carried, ssd_dtype carried_dtype, const float* dA_cumsum,
                             const float* initial_states, float* final_states, void* stream);

/*
 * Fused state path (P1, paragraph on the three kernels: the state pass walks
 * the chunks in order with one matrix product per chunk and the running state
 * on chip): ssd_chunk_state and ssd_state_passing in one call, without
 * writing the chunk states anywhere.  Per (b,h):
 *   run = initial_states[b,h] (zeros when NULL)
 *   for c in 0..nc-1:  carried[b,c,h] = run;
 *                      run = exp(G_{Q-1}(c)) run + sum_{j<Q} exp(G_{Q-1} - G_j) dt_j B_j x_j^T
 *   final_states[b,h] = run   (final_states may be NULL: not written)
 * Where ssd_chunk_state uses its head-group kernel (bf16, chunk 256 with
 * N = 128 or chunk 128 with N = 256) the results are bit-identical to
 * ssd_chunk_state with fp32 states followed by ssd_state_passing with the
 * same carried_dtype; elsewhere they differ from it only by the order of the
 * fp32 sums.
 * x [B,L,H,P], Bm [B,L,G,N]
 * (dtype `in`), dt_bhl and dA_cumsum [B,H,nc,Q], carried [B,nc,H,N,P] in
 * carried_dtype, initial/final states [B,H,N,P] fp32.  Supported: in = BF16,
 * mma = SSD_MMA_BF16, N and P multiples of 64 (else SSD_ERR_UNSUPPORTED).
 */
ssd_status ssd_chunk_state_passing(const ssd_shape* shape, const void* x, const void* Bm, ssd_dtype in,
                                   const float* dt_bhl, const float* dA_cumsum,
                                   const float* initial_states, void* carried, ssd_dtype carried_dtype,
                                   float* final_states, ssd_mma mma, void* stream);

/*
 * Fused chunk output (P1, compute_out paragraph: carried-state term, decayed
 * and causally masked interaction matrix C.B^T, skip connection, in one
 * kernel with the interaction tile kept on chip and the mask applied as a
 * register-level select).  For token i of chunk c (t = cQ+i):
 *   y[b,t,h,:] = exp(G_i) C_i^T carried[b,c,h]
 *              + sum_{j<=i} (C_i . B_j) exp(G_i - G_j) dt_j x[b,cQ+j,h,:]
 *              + D[h] x[b,t,h,:]
 * x [B,L,H,P], Bm/Cm [B,L,G,N] (dtype `in`), carried [B,nc,H,N,P] in
 * `carried_dtype`, D [H] fp32  ->  y [B,L,H,P] in `y_dtype` (F32 or BF16,
 * rounded to nearest even).  With SSD_MMA_BF16 the carried state is rounded
 * to bf16 as a matrix operand anyway, so BF16 carried states written by
 * ssd_state_passing give bit-identical results with half the traffic.
 */
ssd_status ssd_chunk_scan(const ssd_shape* shape, const void* x, const void* Bm, const void* Cm,
                          ssd_dtype in, const float* dt_bhl, const float* dA_cumsum,
                          const void* carried, ssd_dtype carried_dtype, const float* D, void* y,
                          ssd_dtype y_dtype, ssd_mma mma, void* stream);

/*
 * Single-token recurrent step, the decode form of the same recurrence (P1,
 * opening paragraph: a fixed-size hidden state updated once per token, so
 * each new token costs the same; jump-formula paragraph: the update is a
 * decay of the state plus the outer product of b and x).  Per (b,h), with
 * g = h / (H/G):
 *   r = exp(dt[b,h] A[h])
 *   state[b,h] = r state[b,h] + dt[b,h] Bm[b,g,:] x[b,h,:]^T      (N x P, fp32, in place)
 *   y[b,h,:]   = Cm[b,g,:]^T state[b,h] + D[h] x[b,h,:]
 * i.e. ssd_forward over one token with initial_states = state, final_states
 * written back into state.  shape->seqlen must be 1; shape->chunk is not
 * used.  x [B,H,P] and Bm, Cm [B,G,N] in `in`; dt [B,H], A [H], D [H] fp32;
 * state [B,H,N,P] fp32 (read, then overwritten: caller-owned, must not
 * alias the other arguments); y [B,H,P] in y_dtype (bf16 rounded to nearest
 * even).  Supported: P a multiple of 4, P <= 1024 (else
 * SSD_ERR_UNSUPPORTED); other shape errors as for the other calls.  All
 * pointers 16-byte aligned.  Asynchronous on `stream`.
 */
ssd_status ssd_decode_step(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                           const void* Bm, const void* Cm, const float* D, ssd_dtype in, float* state,
                           void* y, ssd_dtype y_dtype, void* stream);

/*
 * Bytes of device workspace ssd_forward needs for `shape` on either precision
 * path: dA_cumsum and dt_bhl (fp32 [B,H,nc,Q] each) and one state area
 * [B,nc,H,N,P] sized for fp32, each 256-byte aligned.  The bf16-operand path
 * uses half of the state area (bf16 chunk states with the bf16 carried states
 * written over them, or the fused state path's bf16 carried states).
 * Returns 0 for an invalid or NULL shape.  Pure host computation.
 */
size_t ssd_workspace_bytes(const ssd_shape* shape);

/*
 * One-call forward of the whole recurrence (P1, paragraph on the three
 * kernels: the forward is the log-space cumulative sum, then the state pass
 * over the chunks, then the fused output, each step reusing what the previous
 * one stored; P1 compute_out paragraph for the output).  For every (b,h),
 * with the recurrence at the top of this header:
 *   y[b,t,h,:] = C_t^T h_t + D[h] x[b,t,h,:]   for t < L
 *   final_states[b,h] = h_{L-1},  h_{-1} = initial_states[b,h] (zeros when NULL)
 * computed as ssd_chunk_cumsum -> ssd_chunk_state -> ssd_state_passing
 * -> ssd_chunk_scan on one stream, no host synchronisation.  With
 * SSD_MMA_BF16 the chunk states are stored as bf16 (states_dtype = SSD_BF16)
 * and the state passing writes the carried states in place over them as bf16
 * (the matrix-operand values the chunk scan uses either way); the recurrence
 * and the final states stay fp32.  With SSD_MMA_F32 everything is fp32 and
 * the state passing runs in place on the chunk states.
 * Where ssd_chunk_state_passing supports the shape and launches at least two
 * blocks per compute unit of the current device (B*H*(N/R)*(P/64) >= 2 x
 * units, with R = 128 state rows per block when N % 128 == 0 and Q <= 128,
 * else R = 64), the two middle steps are that fused call instead (chunk states
 * never stored, so no bf16 rounding of them).  Results are bit-identical to
 * the separate calls of the path taken, with those state and carried dtypes.
 * The path and the heads per block of the head-group kernels follow a table
 * measured per benchmark shape (rules elsewhere); the environment variable
 * SSD_TUNE, read at every call, overrides them for sweeps (comma-separated
 * path=fused|split|fwd, scan_hg=<n>, state_hg=<n>; choices that do not apply
 * are ignored).  path=fwd takes the fused forward kernel (bf16 inputs and
 * operands, Q = 128, N = 256, P % 64 == 0): chunk states, state advance and
 * output in one kernel per (batch, head, 64 columns); its final states are
 * bit-identical to the fused state path, its y equal within the bf16 bar,
 * not bit for bit, to either composition.
 * initial_states [B,H,N,P] may be NULL (zeros); final_states [B,H,N,P] may be
 * NULL (not written).  workspace: device memory of at least
 * ssd_workspace_bytes(shape) bytes, owned by the caller, contents undefined
 * after the call.
 */
ssd_status ssd_forward(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                       const void* Bm, const void* Cm, const float* D, ssd_dtype in,
                       const float* initial_states, void* y, ssd_dtype y_dtype,
                       float* final_states, void* workspace, size_t workspace_bytes,
                       ssd_mma mma, void* stream);

/* Bytes of the static device scratch array ssd_forward_noalloc works in (one
 * copy per GPU, held from library load until the process ends). */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)192 << 20)

/*
 * ssd_forward for callers that cannot allocate device memory: code under
 * HIP stream capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, computation and results as ssd_forward (bit
 * for bit), without the workspace: the forward works in the library's own
 * static device array of SSD_NOALLOC_SCRATCH_BYTES bytes per GPU instead.
 * It calls no hipMalloc / hipFree and allocates nothing; the first call on a
 * device looks up that device's copy of the array once.  Shapes whose
 * workspace (dA_cumsum and dt_bhl, 4 B*H*nc*Q bytes each, plus 2 (bf16
 * operands) or 4 (fp32 operands) B*nc*H*N*P bytes of states, each part
 * rounded up to 256 bytes) exceeds the array return SSD_ERR_SCRATCH before
 * any launch; other errors as for ssd_forward.  The 192 MiB hold the
 * Mamba-2 2.7B-layer shape (B=2, L=8192, H=80, P=64, N=128, Q=256) on both
 * precision paths.  Every call on one GPU uses that GPU's one array: calls
 * that overlap on one GPU (different streams, or several host threads
 * without ordering) race and give wrong results; calls ordered on one
 * stream are safe.  Nothing in the array needs clearing between calls.
 */
ssd_status ssd_forward_noalloc(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                               const void* Bm, const void* Cm, const float* D, ssd_dtype in,
                               const float* initial_states, void* y, ssd_dtype y_dtype,
                               float* final_states, ssd_mma mma, void* stream);

/*
 * Packed sequences.  Several sequences share a batch row: seq_idx [B,L]
 * (int32, device) names each token's sequence, and the recurrence restarts
 * from a zero state wherever seq_idx[b,t] != seq_idx[b,t-1].  This follows
 * from the recurrence's definition applied to each sequence on its own (the
 * pages speak of one sequence at a time): every output is that of its own
 * sequence run alone; initial_states[b] (may be NULL: zeros) applies to the
 * first sequence of row b, and final_states[b] (may be NULL) is the state
 * after the last token of row b (its last sequence).  For s < nseq,
 * seq_states[s] ([nseq,H,N,P] fp32) receives the state after token
 * seq_last[s] (int64 device array of flattened indices b*L + t) of that
 * token's sequence -- for serving, each sequence's last token, to continue
 * it with ssd_decode_step; an index outside [0, B*L) leaves its entry
 * untouched.  nseq = 0 allows seq_last, seq_states NULL.  Same arguments and
 * support as ssd_forward otherwise, always through the two-kernel state
 * path (with SSD_MMA_BF16 bf16 chunk states and bf16 carried states, as in
 * ssd_forward -- the per-sequence states then start from the bf16 carried
 * state of their chunk; fp32 throughout with SSD_MMA_F32); the workspace
 * must hold ssd_workspace_bytes_varlen(shape) bytes.
 * Implementation: per chunk position, the start of its sequence inside the
 * chunk masks the interaction tile and the carried-state term; each chunk
 * state collects the chunk's last sequence only, and the state passing
 * restarts where that sequence began inside the chunk.  With bf16 inputs and
 * SSD_MMA_BF16 the sequence starts, the cumulative sums and both masks are
 * computed inside the chunk-state kernel (three launches, as ssd_forward).
 */
ssd_status ssd_forward_varlen(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                              const void* Bm, const void* Cm, const float* D, ssd_dtype in,
                              const int32_t* seq_idx, const float* initial_states, void* y,
                              ssd_dtype y_dtype, float* final_states, int64_t nseq,
                              const int64_t* seq_last, float* seq_states, void* workspace,
                              size_t workspace_bytes, ssd_mma mma, void* stream);

/* Workspace bytes ssd_forward_varlen needs (0 for an invalid or NULL shape). */
size_t ssd_workspace_bytes_varlen(const ssd_shape* shape);

/*
 * Gradients of ssd_forward (the same recurrence; no packed sequences) for a
 * loss whose derivative is dy (dL/dy, [B,L,H,P], dtype dy_dtype) and dfinal
 * (dL/d final_states, [B,H,N,P] fp32, or NULL: zero).  The pages only preview
 * a backward pass, without its formulas: what is computed is the derivative
 * of the recurrence (page "Jane Street ML Engineers Map Mamba-2 Recurrent
 * State Computation to Tensor Cores with cuTile", opening and jump-formula
 * paragraphs) with the adjoint state g_t = dL/dh_t, which obeys the same
 * recurrence backwards in time (g_t = C_t dy_t^T + exp(dt_{t+1} A) g_{t+1}):
 *   dx_t  = D dy_t + dt_t B_t^T g_t          dB_t = sum over the group's heads of dt_t g_t x_t
 *   dC_t  = sum over the group's heads of h_t dy_t
 *   ddt_t = A exp(dt_t A) <g_t, h_{t-1}> + B_t^T g_t x_t
 *   dA    = sum_t dt_t exp(dt_t A) <g_t, h_{t-1}>,  dD = sum_t dy_t . x_t
 *   dinitial = exp(dt_0 A) g_0
 * ddt is the derivative with respect to the dt given to the forward.
 * Inputs as for ssd_forward (x, Bm, Cm of dtype `in`; initial_states may be
 * NULL).  Outputs, all fp32 and device: dx like x, ddt [B,L,H], dA [H],
 * dB and dC [B,L,G,N], dD [H], dinitial [B,H,N,P] (may be NULL: not written).
 * The adjoint runs as a chunked pass of this library's forward kernels in
 * reversed time, the forward is recomputed, dB and dC come from per-chunk
 * matrix-core kernels summed over each group's heads, and elementwise kernels
 * combine the rest.  mma selects the matrix-core operands as for ssd_forward:
 *   SSD_MMA_F32: fp32 operands, fp32 intermediates.  Every output is within
 *     1e-4 of its oracle value (max |err| / max |ref| per tensor; for ddt
 *     and dA, relative to the summed magnitude of their terms), and dA within
 *     about 1e-3 of |dA| itself at the Mamba-2 2.7B-layer shape.
 *   SSD_MMA_BF16: operands and intermediates (chunk and carried states, the
 *     recomputed outputs) rounded to bf16, nearest even; fp32 accumulation
 *     and sums; about 2.4x faster.  dx, dB, dC, dD and dinitial are within
 *     1e-2 (max |err| / max |ref|), ddt and dA within 2e-2 of the summed
 *     magnitude of their terms (each term carries several bf16-rounded
 *     intermediates; measured up to ~1e-2).  ddt_t and dA are sums of terms of both signs
 *     that can cancel to far below their size (at the 2.7B-layer shape |dA_h|
 *     is 1e-4 to 6e-3 of that sum), and bf16 rounding of each term is not
 *     small against such a sum: there, bf16 dA was measured off by 0.2 to 2
 *     times |dA|.  Use SSD_MMA_F32 where the decay gradients matter.
 * workspace (device, 16-byte aligned) of at least
 * ssd_backward_workspace_bytes(shape) bytes.  Errors as for ssd_forward.
 */
ssd_status ssd_backward(const ssd_shape* shape, const void* x, const float* dt, const float* A, const void* Bm,
                        const void* Cm, const float* D, ssd_dtype in, const float* initial_states, const void* dy,
                        ssd_dtype dy_dtype, const float* dfinal, float* dx, float* ddt, float* dA, float* dB,
                        float* dC, float* dD, float* dinitial, void* workspace, size_t workspace_bytes,
                        ssd_mma mma, void* stream);

/* Workspace bytes ssd_backward needs (0 for an invalid or NULL shape). */
size_t ssd_backward_workspace_bytes(const ssd_shape* shape);

/* Static, NUL-terminated description of a status code. */
const char* ssd_status_string(ssd_status status);

/* SSD_ABI_VERSION of the built library. */
int ssd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SSD_H */
