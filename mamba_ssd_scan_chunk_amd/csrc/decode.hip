// decode.hip -- single-token recurrent step (decode).
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), opening paragraph (the model
// keeps a fixed-size hidden state and updates it once per token, so each new
// token costs the same work and memory) and jump-formula paragraph (one update
// is a decay of the state plus the outer product of b and x).  Per (b, h),
// with g = h / (H/G):
//     r         = exp(dt[b,h] A[h])
//     h[n, p]   = r h[n, p] + dt[b,h] B[b,g,n] x[b,h,p]          (fp32, in place)
//     y[b,h,p]  = sum_n C[b,g,n] h[n, p] + D[h] x[b,h,p]
//
// The step is bound by the state: 8 N P bytes per (b, h) read and written,
// against 2 N + P input elements.  One 256-thread block per (b, h) (an
// XCD-aware remap keeps neighbouring heads of one sequence, which share B and
// C, on one L2).  Thread t owns the four columns 4 (t % CG) .. +3 (one float4,
// CG = P/4 column groups) of the rows rg, rg + RG, ... (rg = t / CG, RG =
// 256 / CG row groups): a wave's float4 accesses cover whole consecutive state
// rows.  All of a thread's state loads are issued before the first update.
// The partial sums of y over each thread's rows meet in LDS and are added in
// row-group order by the CG threads of the first row group (deterministic).
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 8;  // state rows whose loads are in flight together per thread

template <bool IN_BF16, bool Y_BF16>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(
    const void* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const void* __restrict__ Bm, const void* __restrict__ Cm, const float* __restrict__ D,
    float* __restrict__ state, void* __restrict__ y, int H, int P, int N, int G, int remap) {
  __shared__ float4 red[kDecThreads];
  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  if (remap) bid = (bid & 7u) * (nblk >> 3) + (bid >> 3);
  const int h = bid % H;
  const int b = bid / H;
  const int g = h / (H / G);
  const int CG = P >> 2, RG = kDecThreads / CG;
  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const bool active = rg < RG;
  const int64_t bh = (int64_t)b * H + h;

  const float dtv = dt[bh];
  const float r = expf(dtv * A[h]);
  // x[b,h,4cg .. 4cg+3] in fp32
  float4 xv;
  if constexpr (IN_BF16) {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + bh * P + 4 * cg);
    xv = make_float4(bf16_bits_to_f32(q.x & 0xffffu), bf16_bits_to_f32(q.x >> 16), bf16_bits_to_f32(q.y & 0xffffu),
                     bf16_bits_to_f32(q.y >> 16));
  } else {
    xv = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + bh * P + 4 * cg);
  }
  const int64_t bg = ((int64_t)b * G + g) * N;  // B[b,g,0], C[b,g,0]
  auto bc_at = [&](const void* base, int n) -> float {
    if constexpr (IN_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[bg + n]);
    else return static_cast<const float*>(base)[bg + n];
  };

  float4* st = reinterpret_cast<float4*>(state + bh * (int64_t)N * P) + cg;  // row n at st[n * CG]
  float4 yp = make_float4(0.f, 0.f, 0.f, 0.f);
  if (active) {
    for (int n0 = rg; n0 < N; n0 += kDecUnroll * RG) {
      float4 hv[kDecUnroll];
      float bv[kDecUnroll], cv[kDecUnroll];
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) {
        const int n = n0 + u * RG;
        if (n < N) {
          hv[u] = st[(int64_t)n * CG];
          bv[u] = bc_at(Bm, n);
          cv[u] = bc_at(Cm, n);
        }
      }
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) {
        const int n = n0 + u * RG;
        if (n < N) {
          const float s = dtv * bv[u];
          float4 v;
          v.x = fmaf(r, hv[u].x, s * xv.x);
          v.y = fmaf(r, hv[u].y, s * xv.y);
          v.z = fmaf(r, hv[u].z, s * xv.z);
          v.w = fmaf(r, hv[u].w, s * xv.w);
          st[(int64_t)n * CG] = v;
          yp.x = fmaf(cv[u], v.x, yp.x);
          yp.y = fmaf(cv[u], v.y, yp.y);
          yp.z = fmaf(cv[u], v.z, yp.z);
          yp.w = fmaf(cv[u], v.w, yp.w);
        }
      }
    }
  }
  red[tid] = yp;
  __syncthreads();
  if (tid < CG) {
    float4 acc = red[tid];
    for (int k = 1; k < RG; ++k) {
      const float4 o = red[k * CG + tid];
      acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
    }
    const float dh = D[h];
    acc.x = fmaf(dh, xv.x, acc.x);
    acc.y = fmaf(dh, xv.y, acc.y);
    acc.z = fmaf(dh, xv.z, acc.z);
    acc.w = fmaf(dh, xv.w, acc.w);
    if constexpr (Y_BF16)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + bh * P + 4 * tid) =
          make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
    else
      *reinterpret_cast<float4*>(static_cast<float*>(y) + bh * P + 4 * tid) = acc;
  }
}

bool decode_step_supported(int64_t P) { return P % 4 == 0 && P / 4 <= kDecThreads; }

hipError_t launch_decode_step(int64_t Bn, int64_t H, int64_t P, int64_t N, int64_t G, const void* x,
                              const float* dt, const float* A, const void* Bm, const void* Cm, const float* D,
                              bool in_bf16, float* state, void* y, bool y_bf16, hipStream_t stream) {
  const int64_t nblk = Bn * H;
  const int remap = (nblk % 8 == 0) ? 1 : 0;
  auto kern = in_bf16 ? (y_bf16 ? decode_step_kernel<true, true> : decode_step_kernel<true, false>)
                      : (y_bf16 ? decode_step_kernel<false, true> : decode_step_kernel<false, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(kDecThreads), 0, stream, x, dt, A, Bm, Cm, D, state, y, (int)H,
                     (int)P, (int)N, (int)G, remap);
  return hipGetLastError();
}

}  // namespace ssd
