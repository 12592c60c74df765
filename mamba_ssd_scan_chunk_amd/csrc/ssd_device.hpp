// ssd_device.hpp -- gfx950 device helpers shared by the SSD kernels:
// bf16 conversions, MFMA fragment types and the matrix-core step.
//
// MFMA lane layouts used throughout (wave64, checked on gfx950 hardware):
//   v_mfma_f32_16x16x32_bf16: lane l supplies A[l%16][8*(l/16)+e] and
//     B[8*(l/16)+e][l%16] for e = 0..7; D lane l holds D[4*(l/16)+r][l%16].
//   v_mfma_f32_16x16x4_f32:   lane l supplies A[l%16][l/16], B[l/16][l%16];
//     same D layout.
// A "fragment" is the 8 contraction slots one lane owns for one 32-deep step.
// For bf16 operands one MFMA consumes it; for fp32 operands eight 16x16x4
// MFMAs consume it, the q-th one taking slot q of every lane.  Since the
// slot -> contraction-index map only has to agree between the A and B
// fragments, the kernels are free to choose it (see chunk_scan).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (one
// instruction converts two values).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Low (sel = 0) or high (sel = 1) 16-bit halves of two words, packed as
// (a's half) | (b's half) << 16.
__device__ __forceinline__ uint32_t pick_lo16(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pick_hi16(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// Operand-type traits.  Frag<T>::type holds 8 contraction slots of one lane.
struct OpBF16 {
  static constexpr int kBytes = 2;
  struct Frag { uint4 v; };  // 8 x bf16
  __device__ __forceinline__ static Frag zero() { Frag f; f.v = make_uint4(0, 0, 0, 0); return f; }
  __device__ __forceinline__ static Frag from_f32(const float* s) {
    Frag f;
    f.v.x = pack_bf16x2(s[0], s[1]);
    f.v.y = pack_bf16x2(s[2], s[3]);
    f.v.z = pack_bf16x2(s[4], s[5]);
    f.v.w = pack_bf16x2(s[6], s[7]);
    return f;
  }
  __device__ __forceinline__ static f32x4_t mma(const Frag& a, const Frag& b, f32x4_t acc) {
    bf16x8_t av = __builtin_bit_cast(bf16x8_t, a.v);
    bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b.v);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
  }
};

struct OpF32 {
  static constexpr int kBytes = 4;
  struct Frag { float4 lo, hi; };  // 8 x f32
  __device__ __forceinline__ static Frag zero() {
    Frag f; f.lo = make_float4(0.f, 0.f, 0.f, 0.f); f.hi = f.lo; return f;
  }
  __device__ __forceinline__ static Frag from_f32(const float* s) {
    Frag f;
    f.lo = make_float4(s[0], s[1], s[2], s[3]);
    f.hi = make_float4(s[4], s[5], s[6], s[7]);
    return f;
  }
  __device__ __forceinline__ static f32x4_t mma(const Frag& a, const Frag& b, f32x4_t acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
    return acc;
  }
};

// ---- LDS fragment access (8 consecutive elements of operand type) ----
template <class Op> struct Lds;
template <> struct Lds<OpBF16> {
  __device__ __forceinline__ static OpBF16::Frag load8(const uint16_t* p) {
    OpBF16::Frag f; f.v = *reinterpret_cast<const uint4*>(p); return f;
  }
  // Two runs of 4 consecutive elements -> one fragment (slots 0-3, 4-7).
  __device__ __forceinline__ static OpBF16::Frag load4x2(const uint16_t* p0, const uint16_t* p1) {
    uint2 a = *reinterpret_cast<const uint2*>(p0);
    uint2 b = *reinterpret_cast<const uint2*>(p1);
    OpBF16::Frag f; f.v = make_uint4(a.x, a.y, b.x, b.y); return f;
  }
  __device__ __forceinline__ static void store8(uint16_t* p, const float* s) {
    *reinterpret_cast<uint4*>(p) = OpBF16::from_f32(s).v;
  }
};
template <> struct Lds<OpF32> {
  __device__ __forceinline__ static OpF32::Frag load8(const float* p) {
    OpF32::Frag f;
    f.lo = *reinterpret_cast<const float4*>(p);
    f.hi = *reinterpret_cast<const float4*>(p + 4);
    return f;
  }
  __device__ __forceinline__ static OpF32::Frag load4x2(const float* p0, const float* p1) {
    OpF32::Frag f;
    f.lo = *reinterpret_cast<const float4*>(p0);
    f.hi = *reinterpret_cast<const float4*>(p1);
    return f;
  }
  __device__ __forceinline__ static void store8(float* p, const float* s) {
    *reinterpret_cast<float4*>(p) = make_float4(s[0], s[1], s[2], s[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(s[4], s[5], s[6], s[7]);
  }
};

// ---- transposing fragment reads from row-major LDS tiles (gfx950) ----
// ds_read_b64_tr_b16: in each group of 16 lanes, lane 16g + i receives as its
// element r (r = 0..3) the 16-bit word at offset i % 4 of the 8 bytes that
// lane 16g + 4r + i / 4 addresses (lane layout measured on the hardware).
__device__ __forceinline__ uint2 lds_read_tr16_b64(const uint16_t* p) {
  typedef short v4i16_t __attribute__((ext_vector_type(4)));
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p));
  return __builtin_bit_cast(uint2, v);
}
// MFMA fragment of a tile stored row-major [k][col] in LDS, for the operand
// whose lane index (mod 16) is the column: `tile` points at (row k0, column
// c0); lane (i = lane % 16, g = lane / 16) receives, as slots 4t + r,
// tile[k0 + 16t + 4g + r][c0 + i] for t = 0, 1 and r = 0..3.
__device__ __forceinline__ OpBF16::Frag lds_frag_tr(const uint16_t* tile, int pitch, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const uint16_t* p = tile + (4 * g + (i >> 2)) * pitch + 4 * (i & 3);
  const uint2 a = lds_read_tr16_b64(p);
  const uint2 b = lds_read_tr16_b64(p + 16 * pitch);
  OpBF16::Frag f;
  f.v = make_uint4(a.x, a.y, b.x, b.y);
  return f;
}

template <class Op> struct OpElem;
template <> struct OpElem<OpBF16> { typedef uint16_t type; };
template <> struct OpElem<OpF32> { typedef float type; };

// ---- global loads of 8 consecutive input elements, widened to fp32 ----
// in_bf16 selects the input dtype at run time (uniform branch).
__device__ __forceinline__ void load8_as_f32(const void* base, int64_t elem, bool in_bf16, float* out) {
  if (in_bf16) {
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
    out[0] = bf16_bits_to_f32(v.x & 0xffffu); out[1] = bf16_bits_to_f32(v.x >> 16);
    out[2] = bf16_bits_to_f32(v.y & 0xffffu); out[3] = bf16_bits_to_f32(v.y >> 16);
    out[4] = bf16_bits_to_f32(v.z & 0xffffu); out[5] = bf16_bits_to_f32(v.z >> 16);
    out[6] = bf16_bits_to_f32(v.w & 0xffffu); out[7] = bf16_bits_to_f32(v.w >> 16);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
}

__device__ __forceinline__ float load1_as_f32(const void* base, int64_t elem, bool in_bf16) {
  if (in_bf16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[elem]);
  return reinterpret_cast<const float*>(base)[elem];
}

// exp via the hardware exp2 (v_exp_f32); relative error ~4e-6 worst case over
// the ranges used here, and exact 1 at 0.
__device__ __forceinline__ float fast_exp(float v) { return __expf(v); }
// In-chunk inclusive cumulative sum of dt*A for one head, one wave: lane l
// holds the E (<= 4) consecutive tokens E*l .. E*l+E-1 (d[e], e < E), sums
// them with a running fused multiply-add, and a 6-step inclusive shuffle scan
// of the 64 lane totals supplies each lane's offset.  out[e] = G at token
// E*l + e.  Shared by the cumulative-sum kernel and the fused chunk-state
// prologue, which therefore produce identical bits.
__device__ __forceinline__ void chunk_cumsum_lane(const float (&d)[4], int E, float a, int lane, float (&out)[4]) {
  float part[4];
  float run = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (e < E) run = fmaf(d[e], a, run);
    part[e] = run;
  }
  float tot = run;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(tot, off, 64);
    if (lane >= off) tot += o;
  }
  float excl = __shfl_up(tot, 1, 64);
  if (lane == 0) excl = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = excl + part[e];
}

// 2^v on the hardware exponential (one v_exp_f32): for log-space sums kept in
// base-2 units (pre-multiplied by log2(e)), saving the scaling multiply.
__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }
constexpr float kLog2e = 1.4426950408889634f;

// 16-byte rows from MFMA accumulator tiles.  In the 16x16 accumulator layout
// lane (l16, lg) holds 4 consecutive columns 4lg .. 4lg+3 of row l16 for each
// column tile.  Given two column tiles t0 (columns 0..15) and t1 (16..31) of
// the same rows, packed as 2 dwords each, one v_permlane16_swap per dword
// trades them between the lane-row pairs (lg, lg ^ 1): afterwards each lane
// holds 8 consecutive columns -- lg even: 4lg .. 4lg+7 of t0, lg odd:
// 4(lg-1) .. +7 of t1, i.e. column 4lg + 12 (lg & 1) relative to t0 -- as
// the returned uint4, ready for one 16-byte store.
__device__ __forceinline__ uint4 pair_tiles_16b(uint2 t0, uint2 t1) {
  const auto a = __builtin_amdgcn_permlane16_swap(t0.x, t1.x, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(t0.y, t1.y, false, false);
  return make_uint4(a[0], b[0], a[1], b[1]);
}
__device__ __forceinline__ int pair_tiles_col(int lg) { return 4 * lg + 12 * (lg & 1); }

}  // namespace ssd
