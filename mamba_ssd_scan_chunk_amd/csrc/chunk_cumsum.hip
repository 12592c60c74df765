// chunk_cumsum.hip -- log-space decay cumulative sum, one segmented wave64 scan
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
//
// Layout work: dt arrives [B,L,H] (head fastest).  A block reads a Q x 16-head
// tile with head-contiguous (coalesced) loads, transposes it through LDS, and
// each wave scans one head's Q values: Q/64 consecutive values per lane are
// summed serially, then the 64 lane totals are combined with a log-depth
// (6-step) shuffle scan.  Every output row (one head, one chunk) is written as
// Q contiguous floats.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kCsHeads = 16;
constexpr int kCsThreads = 256;

__global__ __launch_bounds__(kCsThreads) void chunk_cumsum_kernel(
    const float* __restrict__ dt, const float* __restrict__ A, float* __restrict__ dA_cumsum,
    float* __restrict__ dt_bhl, int L, int H, int Q, int nc) {
  extern __shared__ float cs_lds[];
  const int pitch = Q + 1;
  float* sa = cs_lds;                     // [16][Q+1]  dt*A
  float* sd = cs_lds + kCsHeads * pitch;  // [16][Q+1]  dt
  const int hb = blockIdx.x * kCsHeads;
  const int c = blockIdx.y;
  const int b = blockIdx.z;
  const int nh = min(kCsHeads, H - hb);
  const int tid = threadIdx.x;

  const int64_t row0 = (int64_t)b * L + (int64_t)c * Q;
  for (int idx = tid; idx < Q * kCsHeads; idx += kCsThreads) {
    const int i = idx / kCsHeads, hh = idx % kCsHeads;
    float v = 0.f, av = 0.f;
    if (hh < nh) {
      v = dt[(row0 + i) * H + hb + hh];
      av = v * A[hb + hh];
    }
    sa[hh * pitch + i] = av;
    sd[hh * pitch + i] = v;
  }
  __syncthreads();

  const int wave = tid / 64, lane = tid % 64;
  const int E = Q >= 64 ? Q / 64 : 1;  // values per lane (<= 4 for Q <= 256)
  const int active = Q / E;            // lanes that hold values
  for (int hh = wave; hh < nh; hh += kCsThreads / 64) {
    float part[4];
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (e < E && lane < active) run += sa[hh * pitch + lane * E + e];
      part[e] = run;
    }
    // inclusive scan of the lane totals, then shift by one lane -> exclusive prefix
    float tot = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(tot, off, 64);
      if (lane >= off) tot += o;
    }
    float excl = __shfl_up(tot, 1, 64);
    if (lane == 0) excl = 0.f;
    if (lane < active) {
      const int64_t orow = (((int64_t)b * H + hb + hh) * nc + c) * Q + lane * E;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < E) dA_cumsum[orow + e] = excl + part[e];
      if (dt_bhl) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < E) dt_bhl[orow + e] = sd[hh * pitch + lane * E + e];
      }
    }
  }
}

hipError_t launch_chunk_cumsum(const Dims& d, const float* dt, const float* A, float* dA_cumsum,
                               float* dt_bhl, hipStream_t stream) {
  const dim3 grid((unsigned)((d.H + kCsHeads - 1) / kCsHeads), (unsigned)d.nc, (unsigned)d.B);
  const size_t lds = sizeof(float) * 2 * kCsHeads * (d.Q + 1);
  hipLaunchKernelGGL(chunk_cumsum_kernel, grid, dim3(kCsThreads), lds, stream, dt, A, dA_cumsum, dt_bhl,
                     (int)d.L, (int)d.H, (int)d.Q, (int)d.nc);
  return hipGetLastError();
}

}  // namespace ssd
