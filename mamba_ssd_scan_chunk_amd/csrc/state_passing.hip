// state_passing.hip -- inter-chunk state advance, an HBM-bound elementwise scan.
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), paragraph on the three kernels
// (a sequential loop over chunks carries the hidden state forward) and the
// jump-formula paragraph (each chunk adds its own state to the decayed
// previous one).  Per (b, h) and state element e:
//     run = h0[b,h,e] (or 0)
//     for c:  carried[b,c,h,e] = run;  run = exp(G_last(b,h,c)) * run + S[b,c,h,e]
//     final[b,h,e] = run
//
// One thread owns 4 consecutive state elements (one float4).  Consecutive
// threads own consecutive float4s of the same (b, h), so every load and store
// is a fully coalesced 1 KB wave access.  The chain over chunks is serial per
// thread, but the S loads do not depend on it: the loop is unrolled by 8 with
// all 8 loads issued before the 8 dependent updates, keeping 8 x 16 B per
// thread in flight, and the next 8 loads are issued before the current 8
// stores.  carried may alias S: each location is read before it is written,
// by the same thread.
//
// A second instantiation writes the carried states rounded to bf16 (round to
// nearest even, 8-byte stores) into a separate buffer: the bf16-operand chunk
// scan rounds them to exactly these values anyway, so the one-call forward
// uses it to halve the carried-state traffic without changing any result.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kSpThreads = 256;
constexpr int kSpUnroll = 8;

// carried element type: float (may alias S) or bf16 bits (separate buffer)
template <bool CBF16>
__global__ __launch_bounds__(kSpThreads) void state_passing_kernel(
    const float* S, void* carried_v, const float* __restrict__ dA_cumsum,
    const float* __restrict__ init, float* __restrict__ fin, int H, int nc, int Q, int64_t np4,
    int64_t total) {
  const int64_t id = (int64_t)blockIdx.x * kSpThreads + threadIdx.x;
  if (id >= total) return;
  const int64_t bh = id / np4;
  const int64_t e4 = id - bh * np4;
  const int64_t b = bh / H, h = bh - b * H;

  float4 run = make_float4(0.f, 0.f, 0.f, 0.f);
  if (init) run = reinterpret_cast<const float4*>(init)[bh * np4 + e4];

  const float* glast = dA_cumsum + bh * nc * Q + (Q - 1);  // chunk c at glast[c*Q]
  const int64_t cstride = (int64_t)H * np4;                // float4s between chunks
  const float4* sp = reinterpret_cast<const float4*>(S) + (b * nc * H + h) * np4 + e4;
  const int64_t coff = (b * nc * H + h) * np4 + e4;  // in units of 4 elements
  auto put = [&](int64_t c, const float4& v) {
    if constexpr (CBF16)
      reinterpret_cast<uint2*>(carried_v)[coff + c * cstride] = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    else
      reinterpret_cast<float4*>(carried_v)[coff + c * cstride] = v;
  };

  // Software pipeline: the loads of chunks c+8..c+15 are issued before the
  // stores of chunks c..c+7 (distinct addresses, so this also holds in place).
  float4 s[kSpUnroll], sn[kSpUnroll];
  float dec[kSpUnroll], decn[kSpUnroll];
  const int nfull = nc / kSpUnroll;  // full batches
  if (nfull > 0) {
#pragma unroll
    for (int u = 0; u < kSpUnroll; ++u) {
      s[u] = sp[(int64_t)u * cstride];
      dec[u] = expf(glast[(int64_t)u * Q]);
    }
  }
  for (int bt = 0; bt < nfull; ++bt) {
    const int c = bt * kSpUnroll;
    if (bt + 1 < nfull) {
#pragma unroll
      for (int u = 0; u < kSpUnroll; ++u) {
        sn[u] = sp[(int64_t)(c + kSpUnroll + u) * cstride];
        decn[u] = expf(glast[(int64_t)(c + kSpUnroll + u) * Q]);
      }
    }
#pragma unroll
    for (int u = 0; u < kSpUnroll; ++u) {
      put(c + u, run);
      run.x = fmaf(dec[u], run.x, s[u].x);  // explicit fused multiply-add: the fused
      run.y = fmaf(dec[u], run.y, s[u].y);  // state path repeats these bits exactly
      run.z = fmaf(dec[u], run.z, s[u].z);
      run.w = fmaf(dec[u], run.w, s[u].w);
    }
#pragma unroll
    for (int u = 0; u < kSpUnroll; ++u) {
      s[u] = sn[u];
      dec[u] = decn[u];
    }
  }
  for (int c = nfull * kSpUnroll; c < nc; ++c) {
    const float4 sv = sp[(int64_t)c * cstride];
    const float d1 = expf(glast[(int64_t)c * Q]);
    put(c, run);
    run.x = fmaf(d1, run.x, sv.x);
    run.y = fmaf(d1, run.y, sv.y);
    run.z = fmaf(d1, run.z, sv.z);
    run.w = fmaf(d1, run.w, sv.w);
  }
  if (fin) reinterpret_cast<float4*>(fin)[bh * np4 + e4] = run;
}

template <bool CBF16>
static hipError_t launch_sp(const Dims& d, const float* chunk_states, void* carried, const float* dA_cumsum,
                            const float* initial_states, float* final_states, hipStream_t stream) {
  const int64_t np4 = d.N * d.P / 4;
  const int64_t total = d.B * d.H * np4;
  const unsigned blocks = (unsigned)((total + kSpThreads - 1) / kSpThreads);
  hipLaunchKernelGGL(state_passing_kernel<CBF16>, dim3(blocks), dim3(kSpThreads), 0, stream, chunk_states, carried,
                     dA_cumsum, initial_states, final_states, (int)d.H, (int)d.nc, (int)d.Q, np4, total);
  return hipGetLastError();
}

hipError_t launch_state_passing(const Dims& d, const float* chunk_states, float* carried,
                                const float* dA_cumsum, const float* initial_states,
                                float* final_states, hipStream_t stream) {
  return launch_sp<false>(d, chunk_states, carried, dA_cumsum, initial_states, final_states, stream);
}

hipError_t launch_state_passing_bf16(const Dims& d, const float* chunk_states, uint16_t* carried_bf16,
                                     const float* dA_cumsum, const float* initial_states,
                                     float* final_states, hipStream_t stream) {
  return launch_sp<true>(d, chunk_states, carried_bf16, dA_cumsum, initial_states, final_states, stream);
}

}  // namespace ssd
