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
// One thread owns 4 consecutive state elements (one float4 of fp32 chunk
// states) or 8 (one 16-byte piece of bf16 chunk states).  Consecutive threads
// own consecutive pieces of the same (b, h), so every load and store is a
// fully coalesced wave access.  The chain over chunks is serial per thread,
// but the S loads do not depend on it: the loop is unrolled by 8 with all 8
// loads issued before the 8 dependent updates, keeping 8 x 16 B per thread in
// flight, and the next 8 loads are issued before the current 8 stores.
// carried may alias S: each location is read before it is written, by the
// same thread.
//
// Instantiations write the carried states rounded to bf16 (round to nearest
// even): the bf16-operand chunk scan rounds them to exactly these values
// anyway, so the one-call forward uses it to halve the carried-state traffic
// without changing any result.  The chunk states may arrive as bf16 too
// (widened exactly to fp32); the recurrence itself always runs in fp32.
// carried may alias S when both have the same element size.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kSpThreads = 256;

// EPT consecutive state elements of one thread in fp32 or bf16 storage:
// the raw vector moved by one load or store (16 bytes, except 4 fp32 -> 16 and
// 4 bf16 -> 8 bytes), widened exactly to fp32 and narrowed by rounding to
// nearest even.
template <int EPT, bool BF16>
struct SpVec;
template <>
struct SpVec<4, false> {
  using raw = float4;
  __device__ __forceinline__ static raw load(const void* p, int64_t e) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + e);
  }
  __device__ __forceinline__ static void widen(const raw& v, float* f) { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
  __device__ __forceinline__ static void store(void* p, int64_t e, const float* f) {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + e) = make_float4(f[0], f[1], f[2], f[3]);
  }
};
template <>
struct SpVec<4, true> {
  using raw = uint2;
  __device__ __forceinline__ static raw load(const void* p, int64_t e) {
    return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + e);
  }
  __device__ __forceinline__ static void widen(const raw& v, float* f) {
    f[0] = bf16_bits_to_f32(v.x & 0xffffu); f[1] = bf16_bits_to_f32(v.x >> 16);
    f[2] = bf16_bits_to_f32(v.y & 0xffffu); f[3] = bf16_bits_to_f32(v.y >> 16);
  }
  __device__ __forceinline__ static void store(void* p, int64_t e, const float* f) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + e) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
  }
};
template <>
struct SpVec<8, true> {
  using raw = uint4;
  __device__ __forceinline__ static raw load(const void* p, int64_t e) {
    return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p) + e);
  }
  __device__ __forceinline__ static void widen(const raw& v, float* f) {
    f[0] = bf16_bits_to_f32(v.x & 0xffffu); f[1] = bf16_bits_to_f32(v.x >> 16);
    f[2] = bf16_bits_to_f32(v.y & 0xffffu); f[3] = bf16_bits_to_f32(v.y >> 16);
    f[4] = bf16_bits_to_f32(v.z & 0xffffu); f[5] = bf16_bits_to_f32(v.z >> 16);
    f[6] = bf16_bits_to_f32(v.w & 0xffffu); f[7] = bf16_bits_to_f32(v.w >> 16);
  }
  __device__ __forceinline__ static void store(void* p, int64_t e, const float* f) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p) + e) =
        make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
};
template <>
struct SpVec<8, false> {
  struct raw { float4 a, b; };
  __device__ __forceinline__ static raw load(const void* p, int64_t e) {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + e);
    return raw{q[0], q[1]};
  }
  __device__ __forceinline__ static void widen(const raw& v, float* f) {
    f[0] = v.a.x; f[1] = v.a.y; f[2] = v.a.z; f[3] = v.a.w; f[4] = v.b.x; f[5] = v.b.y; f[6] = v.b.z; f[7] = v.b.w;
  }
  __device__ __forceinline__ static void store(void* p, int64_t e, const float* f) {
    float4* q = reinterpret_cast<float4*>(static_cast<float*>(p) + e);
    q[0] = make_float4(f[0], f[1], f[2], f[3]);
    q[1] = make_float4(f[4], f[5], f[6], f[7]);
  }
};

// One thread owns EPT consecutive state elements: 4 with fp32 chunk states
// (16-byte loads), 8 with bf16 chunk states (16-byte loads as well).
// U chunks per batch: U loads per thread are in flight while the previous
// batch's updates run.
template <bool SBF16, bool CBF16, int EPT, int TPB, int U>
__global__ __launch_bounds__(TPB) void state_passing_kernel(
    const void* S, void* carried_v, const float* __restrict__ dA_cumsum,
    const float* __restrict__ init, float* __restrict__ fin, int H, int nc, int Q, int64_t npv,
    int64_t total) {
  using In = SpVec<EPT, SBF16>;
  using Out = SpVec<EPT, CBF16>;
  using F32 = SpVec<EPT, false>;
  using Raw = typename In::raw;
  const int64_t id = (int64_t)blockIdx.x * TPB + threadIdx.x;
  if (id >= total) return;
  const int64_t bh = id / npv;
  const int64_t ev = id - bh * npv;
  const int64_t b = bh / H, h = bh - b * H;
  const int64_t np = npv * EPT;  // N * P

  float run[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) run[k] = 0.f;
  if (init) F32::widen(F32::load(init, bh * np + ev * EPT), run);

  const float* glast = dA_cumsum + bh * nc * Q + (Q - 1);  // chunk c at glast[c*Q]
  const int64_t cstride = (int64_t)H * np;                 // elements between chunks
  const int64_t e0 = (b * nc * H + h) * np + ev * EPT;     // element offset of chunk 0
  auto step = [&](const Raw& r, float d) __attribute__((always_inline)) {
    float sv[EPT];
    In::widen(r, sv);
#pragma unroll
    for (int k = 0; k < EPT; ++k) run[k] = fmaf(d, run[k], sv[k]);  // explicit fused multiply-add: the
  };                                                                    // fused state path repeats these bits

  // Software pipeline: the loads of chunks c+U..c+2U-1 are issued before the
  // stores of chunks c..c+U-1 (distinct addresses, so this also holds in place).
  Raw s[U], sn[U];
  float dec[U], decn[U];
  const int nfull = nc / U;  // full batches
  if (nfull > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[u] = In::load(S, e0 + (int64_t)u * cstride);
      dec[u] = expf(glast[(int64_t)u * Q]);
    }
  }
  for (int bt = 0; bt < nfull; ++bt) {
    const int c = bt * U;
    if (bt + 1 < nfull) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        sn[u] = In::load(S, e0 + (int64_t)(c + U + u) * cstride);
        decn[u] = expf(glast[(int64_t)(c + U + u) * Q]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Out::store(carried_v, e0 + (int64_t)(c + u) * cstride, run);
      step(s[u], dec[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s[u] = sn[u];
      dec[u] = decn[u];
    }
  }
  for (int c = nfull * U; c < nc; ++c) {
    const Raw sv = In::load(S, e0 + (int64_t)c * cstride);
    const float d1 = expf(glast[(int64_t)c * Q]);
    Out::store(carried_v, e0 + (int64_t)c * cstride, run);
    step(sv, d1);
  }
  if (fin) F32::store(fin, bh * np + ev * EPT, run);
}

template <bool SBF16, bool CBF16>
static hipError_t launch_sp(const Dims& d, const void* chunk_states, void* carried, const float* dA_cumsum,
                            const float* initial_states, float* final_states, hipStream_t stream) {
  // 8 elements per thread for bf16 chunk states (N * P is a multiple of 256),
  // in blocks of half the size, so the grid has as many blocks as with 4.
  // With fewer than 4 waves per compute unit (long sequences of few heads)
  // the parallelism sets the rate: batches of 16 chunks instead of 8, and
  // bf16 chunk states at 4 elements per thread (twice the waves, the same
  // bytes in flight).
  const int cus = device_cu_count();
  const int64_t waves8 = (d.B * d.H * (d.N * d.P / (SBF16 ? 8 : 4)) + 63) / 64;
  const bool deep = waves8 < 4 * (int64_t)cus && d.nc >= 32;
  if (deep) {
    constexpr int EPT = 4, TPB = kSpThreads;
    const int64_t npv = d.N * d.P / EPT;
    const int64_t total = d.B * d.H * npv;
    const unsigned blocks = (unsigned)((total + TPB - 1) / TPB);
    hipLaunchKernelGGL((state_passing_kernel<SBF16, CBF16, EPT, TPB, 16>), dim3(blocks), dim3(TPB), 0, stream,
                       chunk_states, carried, dA_cumsum, initial_states, final_states, (int)d.H, (int)d.nc, (int)d.Q,
                       npv, total);
  } else {
    constexpr int EPT = SBF16 ? 8 : 4;
    constexpr int TPB = SBF16 ? kSpThreads / 2 : kSpThreads;
    const int64_t npv = d.N * d.P / EPT;
    const int64_t total = d.B * d.H * npv;
    const unsigned blocks = (unsigned)((total + TPB - 1) / TPB);
    hipLaunchKernelGGL((state_passing_kernel<SBF16, CBF16, EPT, TPB, 8>), dim3(blocks), dim3(TPB), 0, stream,
                       chunk_states, carried, dA_cumsum, initial_states, final_states, (int)d.H, (int)d.nc, (int)d.Q,
                       npv, total);
  }
  return hipGetLastError();
}

hipError_t launch_state_passing(const Dims& d, const float* chunk_states, float* carried,
                                const float* dA_cumsum, const float* initial_states,
                                float* final_states, hipStream_t stream) {
  return launch_sp<false, false>(d, chunk_states, carried, dA_cumsum, initial_states, final_states, stream);
}

hipError_t launch_state_passing_bf16(const Dims& d, const float* chunk_states, uint16_t* carried_bf16,
                                     const float* dA_cumsum, const float* initial_states,
                                     float* final_states, hipStream_t stream) {
  return launch_sp<false, true>(d, chunk_states, carried_bf16, dA_cumsum, initial_states, final_states, stream);
}

hipError_t launch_state_passing_any(const Dims& d, const void* chunk_states, bool states_bf16, void* carried,
                                    bool carried_bf16, const float* dA_cumsum, const float* initial_states,
                                    float* final_states, hipStream_t stream) {
  if (states_bf16)
    return carried_bf16
               ? launch_sp<true, true>(d, chunk_states, carried, dA_cumsum, initial_states, final_states, stream)
               : launch_sp<true, false>(d, chunk_states, carried, dA_cumsum, initial_states, final_states, stream);
  return carried_bf16
             ? launch_sp<false, true>(d, chunk_states, carried, dA_cumsum, initial_states, final_states, stream)
             : launch_sp<false, false>(d, chunk_states, carried, dA_cumsum, initial_states, final_states, stream);
}

}  // namespace ssd
