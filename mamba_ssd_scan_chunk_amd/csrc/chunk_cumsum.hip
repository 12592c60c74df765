// chunk_cumsum.hip -- log-space decay cumulative sum, one segmented wave64 scan
// per (batch, chunk, 4 heads).
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
// One wave owns (b, c, heads 4q..4q+3).  Lane l holds the E = Q/64
// consecutive tokens lE..lE+E-1 of all four heads (16-byte loads of dt when
// H % 4 == 0), sums them serially, and the 64 lane totals are combined with a
// log-depth (6-step) shuffle scan per head.  Each lane then writes its E
// values of each head as one contiguous run, so every output row (one head,
// one chunk) is written as Q contiguous floats.  No LDS is used.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kCsThreads = 256;

__global__ __launch_bounds__(kCsThreads) void chunk_cumsum_kernel(
    const float* __restrict__ dt, const float* __restrict__ A, float* __restrict__ dA_cumsum,
    float* __restrict__ dt_bhl, int L, int H, int Q, int nc, int nq, int64_t nwaves) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * (kCsThreads / 64) + (threadIdx.x >> 6);
  if (wid >= nwaves) return;  // whole wave exits together
  const int q = (int)(wid % nq);
  const int64_t bc = wid / nq;
  const int c = (int)(bc % nc);
  const int b = (int)(bc / nc);
  const int h0 = 4 * q;
  const int E = Q >= 64 ? Q / 64 : 1;  // tokens per lane (<= 4 for Q <= 256)
  const int active = Q / E;            // lanes that hold tokens
  const bool vec = (H % 4 == 0);       // 16-byte aligned head quadruples

  float A4[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) A4[k] = (h0 + k < H) ? A[h0 + k] : 0.f;

  float dv[4][4];  // [token e][head k]
  const int64_t row0 = (int64_t)b * L + (int64_t)c * Q;
  // tokens past the end of the sequence (a ragged last chunk) count as dt = 0:
  // dt_bhl is 0 there and dA_cumsum stays at its last value
  const int nvalid = L - c * Q;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool ok = e < E && lane < active && lane * E + e < nvalid;
    const int64_t row = row0 + lane * E + e;
    if (ok && vec) {
      const float4 v = *reinterpret_cast<const float4*>(dt + row * H + h0);
      dv[e][0] = v.x; dv[e][1] = v.y; dv[e][2] = v.z; dv[e][3] = v.w;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) dv[e][k] = (ok && h0 + k < H) ? dt[row * H + h0 + k] : 0.f;
    }
  }
  // per head: running sum inside the lane, then the lane offsets by a shuffle scan
  float gv[4][4];  // [head k][token e]
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float d4[4] = {dv[0][k], dv[1][k], dv[2][k], dv[3][k]};
    chunk_cumsum_lane(d4, E, A4[k], lane, gv[k]);
  }
  if (lane < active) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (h0 + k >= H) continue;
      const int64_t orow = (((int64_t)b * H + h0 + k) * nc + c) * Q + lane * E;
      if (E == 4) {
        *reinterpret_cast<float4*>(dA_cumsum + orow) = make_float4(gv[k][0], gv[k][1], gv[k][2], gv[k][3]);
        if (dt_bhl) *reinterpret_cast<float4*>(dt_bhl + orow) = make_float4(dv[0][k], dv[1][k], dv[2][k], dv[3][k]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < E) {
            dA_cumsum[orow + e] = gv[k][e];
            if (dt_bhl) dt_bhl[orow + e] = dv[e][k];
          }
      }
    }
  }
}

hipError_t launch_chunk_cumsum(const Dims& d, const float* dt, const float* A, float* dA_cumsum,
                               float* dt_bhl, hipStream_t stream) {
  const int nq = (int)((d.H + 3) / 4);
  const int64_t nwaves = d.B * d.nc * nq;
  const unsigned blocks = (unsigned)((nwaves + kCsThreads / 64 - 1) / (kCsThreads / 64));
  hipLaunchKernelGGL(chunk_cumsum_kernel, dim3(blocks), dim3(kCsThreads), 0, stream, dt, A, dA_cumsum, dt_bhl,
                     (int)d.L, (int)d.H, (int)d.Q, (int)d.nc, nq, nwaves);
  return hipGetLastError();
}

}  // namespace ssd
