// chunk_cumsum.hip -- log-space decay cumulative sum: one segmented wave64 scan
// per (batch, chunk, head).
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), paragraph on the three kernels
// (per-token, per-head cumulative sums of the decay term inside each chunk,
// stored for the two later kernels) and the Blackwell-optimisation paragraph
// (the sums and dt are re-laid out token-contiguous per (batch, head)).
//
//   dA_cumsum[b,h,c,i] = sum_{k<=i} dt[b,cQ+k,h] * A[h]      (fp32, inclusive)
//   dt_bhl[b,h,c,i]    = dt[b,cQ+i,h]
// with dt = 0 for tokens cQ+i >= L (ragged last chunk).
//
// One 512-thread block owns (b, c, up to 32 heads).  The dt tile of the chunk
// (Q tokens x 32 heads = one 128-byte row per token when H % 4 == 0) is read
// with 16-byte loads, 8 consecutive threads per row (whole lines), and
// transposed through LDS to head-major rows.  Each wave then scans its heads
// one at a time: lane l holds the E = Q/64 consecutive tokens lE..lE+E-1, sums
// them serially, and the 64 lane totals are combined by a log-depth (6-step)
// shuffle scan (chunk_cumsum_lane); every output row (one head, one chunk) is
// written as Q contiguous floats.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kCsThreads = 512;
constexpr int kCsHeads = 32;  // heads per block

template <bool VEC>
__global__ __launch_bounds__(kCsThreads) void chunk_cumsum_kernel(
    const float* __restrict__ dt, const float* __restrict__ A, float* __restrict__ dA_cumsum,
    float* __restrict__ dt_bhl, int L, int H, int Q, int nc, int nhb) {
  // [head][token]; the pitch keeps every row 16-byte aligned for the scan's
  // vector reads
  __shared__ __align__(16) float Ds[kCsHeads][256 + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hb = blockIdx.x % nhb;
  const int bc = blockIdx.x / nhb;
  const int c = bc % nc, b = bc / nc;
  const int h0 = hb * kCsHeads;
  const int nh = min(kCsHeads, H - h0);  // heads in this block
  // tokens past the end of the sequence (a ragged last chunk) count as dt = 0:
  // dt_bhl is 0 there and dA_cumsum stays at its last value
  const int nvalid = min(Q, L - c * Q);
  const float* src = dt + ((int64_t)b * L + (int64_t)c * Q) * H + h0;

  if (VEC) {
    // 16-byte pieces: piece = token * 8 + q4 (heads 4q4 .. 4q4+3)
    for (int idx = tid; idx < Q * (kCsHeads / 4); idx += kCsThreads) {
      const int tok = idx >> 3, q4 = idx & 7;
      if (4 * q4 >= nh) continue;
      const float4 v = tok < nvalid ? *reinterpret_cast<const float4*>(src + (int64_t)tok * H + 4 * q4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
      Ds[4 * q4 + 0][tok] = v.x;
      Ds[4 * q4 + 1][tok] = v.y;
      Ds[4 * q4 + 2][tok] = v.z;
      Ds[4 * q4 + 3][tok] = v.w;
    }
  } else {
    for (int idx = tid; idx < Q * kCsHeads; idx += kCsThreads) {
      const int tok = idx / kCsHeads, k = idx % kCsHeads;
      if (k >= nh) continue;
      Ds[k][tok] = tok < nvalid ? src[(int64_t)tok * H + k] : 0.f;
    }
  }
  __syncthreads();

  const int E = Q >= 64 ? Q / 64 : 1;  // tokens per lane (<= 4 for Q <= 256)
  const int active = Q / E;            // lanes that hold tokens
  for (int k = wave; k < nh; k += kCsThreads / 64) {
    float d4[4], g4[4];
    if (E == 4) {
      const float4 v = *reinterpret_cast<const float4*>(&Ds[k][4 * lane]);
      d4[0] = v.x; d4[1] = v.y; d4[2] = v.z; d4[3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) d4[e] = (e < E && lane < active) ? Ds[k][lane * E + e] : 0.f;
    }
    chunk_cumsum_lane(d4, E, A[h0 + k], lane, g4);
    if (lane < active) {
      const int64_t orow = (((int64_t)b * H + h0 + k) * nc + c) * Q + lane * E;
      if (E == 4) {
        *reinterpret_cast<float4*>(dA_cumsum + orow) = make_float4(g4[0], g4[1], g4[2], g4[3]);
        if (dt_bhl) *reinterpret_cast<float4*>(dt_bhl + orow) = make_float4(d4[0], d4[1], d4[2], d4[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < E) {
            dA_cumsum[orow + e] = g4[e];
            if (dt_bhl) dt_bhl[orow + e] = d4[e];
          }
      }
    }
  }
}

// Packed sequences: seq_idx[b, t] (int32, non-decreasing along t) names the
// sequence of each token, and the recurrence restarts from a zero state where
// it changes.  Per (b, chunk, position i) this writes
//     seq_start[b, c, i] = the largest k <= i with a sequence start at cQ + k,
//                          or -1 when token cQ + i continues the sequence that
//                          was running before the chunk (the first sequence of
//                          a row counts as running: it starts from the
//                          initial state)
// (positions past the end of a ragged last chunk repeat the last valid one).
// The later kernels read it as masks: token j reaches token i in the chunk
// iff j >= seq_start[i], and only tokens with seq_start = -1 see the carried
// state.  One wave per (b, c); lane l holds positions E l .. E l + E - 1 and
// an inclusive max-scan across the lanes completes the running maximum.
__global__ __launch_bounds__(64) void seq_start_kernel(const int* __restrict__ seq_idx, int* __restrict__ seq_start,
                                                       int L, int Q, int nc) {
  const int lane = threadIdx.x;
  const int c = blockIdx.x % nc, b = blockIdx.x / nc;
  const int E = Q >= 64 ? Q / 64 : 1;
  const int active = Q / E;
  const int nvalid = min(Q, L - c * Q);
  const int* sq = seq_idx + (int64_t)b * L + (int64_t)c * Q;
  int run = -1;
  int loc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = lane * E + e;
    if (e < E && lane < active && i < nvalid) {
      const int t = c * Q + i;
      if (t > 0 && sq[i] != (i > 0 ? sq[i - 1] : sq[-1])) run = i;
    }
    loc[e] = run;
  }
  // inclusive max-scan of the lane maxima (log-depth)
  int tot = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(tot, off, 64);
    if (lane >= off) tot = max(tot, o);
  }
  int excl = __shfl_up(tot, 1, 64);
  if (lane == 0) excl = -1;
  int out[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = max(excl, loc[e]);
  // positions past nvalid: the running maximum already stops growing there
  // (no boundary is recorded past nvalid), so they repeat the last valid value
  if (lane < active) {
    int* o = seq_start + ((int64_t)b * nc + c) * Q + lane * E;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < E) o[e] = out[e];
  }
}

hipError_t launch_seq_start(const Dims& d, const int* seq_idx, int* seq_start, hipStream_t stream) {
  hipLaunchKernelGGL(seq_start_kernel, dim3((unsigned)(d.B * d.nc)), dim3(64), 0, stream, seq_idx, seq_start,
                     (int)d.L, (int)d.Q, (int)d.nc);
  return hipGetLastError();
}

// Packed sequences, inputs of the state steps (per (b, h, c) row of Q):
//   dt_last[i] = dt_bhl[i] where token i belongs to the chunk's last sequence
//                (i >= seq_start[Q-1]), else 0 -- so the chunk state collects
//                that sequence only;
//   dA_pass    = dA_cumsum, except at i = Q-1 where -inf stands in when the
//                chunk's last sequence started inside the chunk -- so the
//                state passing decays the incoming state to exactly 0 there.
__global__ __launch_bounds__(256) void varlen_prep_kernel(const float* __restrict__ dA_cumsum,
                                                          const float* __restrict__ dt_bhl,
                                                          const int* __restrict__ seq_start,
                                                          float* __restrict__ dA_pass, float* __restrict__ dt_last,
                                                          int H, int Q, int nc, int64_t nrows) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // element of [B,H,nc,Q]
  if (e >= nrows * Q) return;
  const int i = (int)(e % Q);
  const int64_t row = e / Q;  // (b * H + h) * nc + c
  const int c = (int)(row % nc);
  const int64_t b = row / nc / H;
  const int st_last = seq_start[(b * nc + c) * Q + Q - 1];
  dt_last[e] = i >= st_last ? dt_bhl[e] : 0.f;
  dA_pass[e] = (i == Q - 1 && st_last >= 0) ? -INFINITY : dA_cumsum[e];
}

hipError_t launch_varlen_prep(const Dims& d, const float* dA_cumsum, const float* dt_bhl, const int* seq_start,
                              float* dA_pass, float* dt_last, hipStream_t stream) {
  const int64_t nrows = d.B * d.H * d.nc;
  const int64_t n = nrows * d.Q;
  hipLaunchKernelGGL(varlen_prep_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dA_cumsum, dt_bhl,
                     seq_start, dA_pass, dt_last, (int)d.H, (int)d.Q, (int)d.nc, nrows);
  return hipGetLastError();
}

hipError_t launch_chunk_cumsum(const Dims& d, const float* dt, const float* A, float* dA_cumsum,
                               float* dt_bhl, hipStream_t stream) {
  const int nhb = (int)((d.H + kCsHeads - 1) / kCsHeads);
  const int64_t nblk = d.B * d.nc * nhb;
  auto kern = (d.H % 4 == 0) ? chunk_cumsum_kernel<true> : chunk_cumsum_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(kCsThreads), 0, stream, dt, A, dA_cumsum, dt_bhl, (int)d.L,
                     (int)d.H, (int)d.Q, (int)d.nc, nhb);
  return hipGetLastError();
}

}  // namespace ssd
