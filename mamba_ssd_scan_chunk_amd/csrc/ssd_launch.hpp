// ssd_launch.hpp -- host-side launchers of the gfx950 SSD kernels.
// Shapes are validated by the C ABI layer (ssd_api.cpp) before any of these
// is called; each launcher only picks the kernel instance, sets its LDS size
// and enqueues it on `stream`, returning the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

struct Dims {
  int64_t B, L, H, P, N, G, Q, nc;
};

// Per-shape launch choices (tuning.cpp): path 0 = rule, 1 = fused state
// walk, 2 = chunk states + state passing, 3 = fused forward (state walk and
// chunk output in one kernel); heads per block of the head-group
// chunk-scan / chunk-state kernels, 0 = rule.
struct Tuning {
  int path, scan_hg, state_hg;
};
Tuning tuning_for(const Dims& d, bool f32_mma);

// Dynamic LDS bytes each kernel needs for the given shape (0 = unsupported).
size_t chunk_state_lds_bytes(const Dims& d, bool f32_mma);
size_t chunk_scan_lds_bytes(const Dims& d, bool f32_mma);

// Compute units of the current device (cached per device, thread-safe; 256
// when the query fails).  Used to size grids and pick kernel variants.
int device_cu_count();

hipError_t launch_chunk_cumsum(const Dims& d, const float* dt, const float* A, float* dA_cumsum,
                               float* dt_bhl, hipStream_t stream);
// Packed sequences: seq_start [B,nc,Q] int32 from seq_idx [B,L] (see chunk_cumsum.hip).
hipError_t launch_seq_start(const Dims& d, const int* seq_idx, int* seq_start, hipStream_t stream);
// Packed sequences: dt masked to each chunk's last sequence (for the chunk
// states) and dA_cumsum with -inf at a chunk's last position where the state
// restarts inside the chunk (for the state passing).
hipError_t launch_varlen_prep(const Dims& d, const float* dA_cumsum, const float* dt_bhl, const int* seq_start,
                              float* dA_pass, float* dt_last, hipStream_t stream);

hipError_t launch_chunk_state(const Dims& d, const void* x, const void* Bm, bool in_bf16,
                              const float* dt_bhl, const float* dA_cumsum, float* states,
                              bool f32_mma, hipStream_t stream);
// The same with the states stored as fp32 or (states_bf16) rounded to bf16,
// nearest even.
hipError_t launch_chunk_state_any(const Dims& d, const void* x, const void* Bm, bool in_bf16,
                                  const float* dt_bhl, const float* dA_cumsum, void* states, bool states_bf16,
                                  bool f32_mma, hipStream_t stream);

// Head-group variant of the chunk states (bf16 inputs; bf16 or, with
// f32_mma, fp32 matrix operands; (chunk, N) in {(64,128), (128,128),
// (256,128), (64,256), (128,256)}, P a multiple of 64); launch_chunk_state
// picks it when supported.
bool chunk_state_hg_supported(const Dims& d, bool in_bf16, bool f32_mma);
hipError_t launch_chunk_state_hg(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                                 const float* dA_cumsum, void* states, bool states_bf16, bool f32_mma,
                                 hipStream_t stream);
// The same kernel with the cumulative-sum step fused in front: it reads dt and
// A, writes dA_cumsum and dt_bhl (bit-identical to launch_chunk_cumsum) and
// the chunk states.  Same support as chunk_state_hg_supported.
hipError_t launch_chunk_state_cumsum_hg(const Dims& d, const void* x, const void* Bm, const float* dt,
                                        const float* A, float* dA_cumsum, float* dt_bhl, void* states,
                                        bool states_bf16, bool f32_mma, hipStream_t stream);

// Packed sequences (bf16 inputs, operands and states; the shapes of
// chunk_state_hg_varlen_supported): the fused instance above with the
// sequence steps folded in.  From seq_idx [B,L] it also writes seq_start
// [B,nc,Q] (as launch_seq_start), weights each chunk's state by the rows of
// its last sequence only, and writes dA_pass at position Q-1 of every
// (b, h, c) row (the only entries the state passing reads): -inf where the
// chunk's last sequence starts inside it, else dA_cumsum there.
bool chunk_state_hg_varlen_supported(const Dims& d);
hipError_t launch_chunk_state_cumsum_hg_varlen(const Dims& d, const void* x, const void* Bm, const float* dt,
                                               const float* A, const int* seq_idx, float* dA_cumsum, float* dt_bhl,
                                               int* seq_start, float* dA_pass, void* states, hipStream_t stream);

hipError_t launch_state_passing(const Dims& d, const float* chunk_states, float* carried,
                                const float* dA_cumsum, const float* initial_states,
                                float* final_states, hipStream_t stream);
// Same recurrence; the carried states are written rounded to bf16 (RNE) into a
// separate buffer (same [B,nc,H,N,P] layout); final states stay fp32.
hipError_t launch_state_passing_bf16(const Dims& d, const float* chunk_states, uint16_t* carried_bf16,
                                     const float* dA_cumsum, const float* initial_states,
                                     float* final_states, hipStream_t stream);
// Any combination of chunk-state and carried dtypes (fp32 or bf16 bits); the
// recurrence runs in fp32.  carried may equal chunk_states when both dtypes
// match.
hipError_t launch_state_passing_any(const Dims& d, const void* chunk_states, bool states_bf16, void* carried,
                                    bool carried_bf16, const float* dA_cumsum, const float* initial_states,
                                    float* final_states, hipStream_t stream);

// Fused state path: chunk states and the inter-chunk advance in one pass (the
// chunk states stay on chip); carried and final states are bit-identical to
// launch_chunk_state + launch_state_passing.  bf16 inputs and operands,
// N and P multiples of 64, chunk in {32, 64, 128, 256}.
bool state_fused_supported(const Dims& d, bool in_bf16, bool f32_mma);
// Independent chunk walks of the fused state kernel for the shape, one per
// (head, state-row block, 64-column slice); a block runs one or two of them.
int64_t state_fused_blocks(const Dims& d);
hipError_t launch_state_fused(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                              const float* dA_cumsum, const float* initial_states, void* carried, bool carried_bf16,
                              float* final_states, hipStream_t stream);

// Fused forward (forward_fused.hip): chunk states, state advance and chunk
// output in one pass per (batch, head, 64-column slice), the running state on
// chip; reads dA_cumsum / dt_bhl of launch_chunk_cumsum.  bf16 inputs and
// operands, chunk 128, N = 256, P a multiple of 64.
bool fwd_fused_supported(const Dims& d, bool in_bf16, bool f32_mma);
hipError_t launch_fwd_fused(const Dims& d, const void* x, const void* Bm, const void* Cm, const float* dt_bhl,
                            const float* dA_cumsum, const float* D, const float* initial_states, void* y, bool y_bf16,
                            float* final_states, hipStream_t stream);

// Head-group variant of the fused chunk output (bf16 inputs; bf16 or, with
// f32_mma, fp32 operands for M.X and C.H_in; (chunk, N) in {(128,64),
// (128,128), (128,256), (256,64), (256,128)}, P a multiple of 64);
// launch_chunk_scan picks it when supported.  `carried` holds fp32 values, or
// bf16 bits (already rounded to nearest even) when carried_bf16 is set.
bool chunk_scan_hg_supported(const Dims& d, bool in_bf16, bool f32_mma);
hipError_t launch_chunk_scan_hg(const Dims& d, const void* x, const void* Bm, const void* Cm, bool in_bf16,
                                const float* dt_bhl, const float* dA_cumsum, const void* carried, bool carried_bf16,
                                const float* D, void* y, bool y_bf16, bool f32_mma, hipStream_t stream,
                                const int* seq_start = nullptr);

// The backward's adjoint pass, run over reversed time (d.L = nc*Q steps),
// reading the forward arrays directly: step s of the pass reads forward token
// d.L-1-s of the lin-token inputs (d.L - Q < lin <= d.L), clamped to lin-1 --
// the steps past the forward sequence must have input scale (dt_bhl) 0.  The
// states / y are written in the pass's own order.  Shapes of the head-group
// kernels; bf16 states / y with bf16 operands, fp32 with fp32.
hipError_t launch_chunk_state_hg_rev(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                                     const float* dA_cumsum, void* states, bool states_bf16, bool f32_mma,
                                     int64_t lin, hipStream_t stream);
hipError_t launch_chunk_scan_hg_rev(const Dims& d, const void* x, const void* Bm, const void* Cm, const float* dt_bhl,
                                    const float* dA_cumsum, const void* carried, bool carried_bf16, const float* D,
                                    void* y, bool f32_mma, int64_t lin, hipStream_t stream);

// `carried` holds fp32 values, or bf16 bits when carried_bf16 is set.
// seq_start (packed sequences, [B,nc,Q] from launch_seq_start, or NULL):
// interaction and carried-state terms are masked to each row's sequence.
hipError_t launch_chunk_scan(const Dims& d, const void* x, const void* Bm, const void* Cm, bool in_bf16,
                             const float* dt_bhl, const float* dA_cumsum, const void* carried, bool carried_bf16,
                             const float* D, void* y, bool y_bf16, bool f32_mma, hipStream_t stream,
                             const int* seq_start = nullptr);

// Packed sequences: the state after token last_token[s] (flattened b*L+t) of
// its sequence, for s < nseq -> out [nseq,H,N,P] fp32; carried = the states
// entering each chunk [B,nc,H,N,P], fp32 or (carried_bf16) bf16 bits.  On
// the matrix cores (bf16 or, with f32_mma, fp32 operands) for bf16 inputs
// with N and P multiples of 64, else in fp32 on the vector ALUs.
hipError_t launch_varlen_states(const Dims& d, const void* x, const void* Bm, bool in_bf16, const float* dt_bhl,
                                const float* dA_cumsum, const int* seq_start, const void* carried, bool carried_bf16,
                                int64_t nseq, const int64_t* last_token, float* out, bool f32_mma,
                                hipStream_t stream);

// Single-token recurrent step: state [Bn,H,N,P] fp32 updated in place, y
// [Bn,H,P].  Supported for P a multiple of 4 up to 1024.
bool decode_step_supported(int64_t P);
hipError_t launch_decode_step(int64_t Bn, int64_t H, int64_t P, int64_t N, int64_t G, const void* x,
                              const float* dt, const float* A, const void* Bm, const void* Cm, const float* D,
                              bool in_bf16, float* state, void* y, bool y_bf16, hipStream_t stream);

// Gradients of B and C of the chunked forward, summed over each group's heads
// (bwd_dbc.hip): dA_cumsum / dt_bhl of the forward [B,H,nc,Q], the states
// entering each chunk [B,nc,H,N,P], and the adjoint's carried states in
// reversed chunk order (entry k' is the gradient at the first token
// of chunk nc-k', or dL/dfinal for k' = 0), both fp32 or (st_bf16) bf16
// bits.  ws: bwd_dbc_ws_bytes of scratch.
// Q in {32, 64, 128, 256}, N and P multiples of 16 with N <= 256.
bool bwd_dbc_supported(const Dims& d);
size_t bwd_dbc_ws_bytes(const Dims& d);
// Largest dynamic LDS any of its kernels takes for the shape and mode.
size_t bwd_dbc_lds_bytes(const Dims& d, bool f32_mma);
hipError_t launch_bwd_dbc(const Dims& d, const void* x, bool x_bf16, const void* dy, bool dy_bf16, const void* Bm,
                          const void* Cm, bool in_bf16, const float* dA_cumsum, const float* dt_bhl,
                          const void* fwd_carried, const void* adj_carried_rev, bool st_bf16, const float* A,
                          float* ws, float* dB, float* dC, bool f32_mma, hipStream_t stream);

// Gradients of the forward (see backward.hip); fp32 outputs and accumulation.
size_t backward_workspace_bytes(const Dims& d);
hipError_t launch_backward(const Dims& d, const void* x, const float* dt, const float* A, const void* Bm,
                           const void* Cm, const float* D, bool in_bf16, const float* initial_states,
                           const void* dy, bool dy_bf16, const float* dfinal, float* dx, float* ddt, float* dA,
                           float* dB, float* dC, float* dD, float* dinit, bool f32_mma, void* workspace,
                           hipStream_t stream);

}  // namespace ssd
