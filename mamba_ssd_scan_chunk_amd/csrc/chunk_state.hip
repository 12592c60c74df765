// chunk_state.hip -- per-chunk states by the decayed jump formula, on MFMA.
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), jump-formula paragraph: with
// the b and x vectors of a chunk stacked as matrices, the state advance over
// the chunk is one matrix product, and pre-multiplying rows by exponentials
// of the log-space sums keeps it one.  For chunk c of (b, h):
//     S[n][p] = sum_j B[j][n] * w_j * x[j][p],   w_j = exp(G_{Q-1} - G_j) dt_j
// The decay weight is folded into the x rows (not the B rows) so that the B
// tile stays the raw input shared by every head of a group; in exact
// arithmetic the two placements are the same product.
//
// Work split: one 256-thread block per (b, c, HPB heads of one group,
// 16/32/64-column slice of P).  The B rows of a step are staged once for the
// block's HPB heads (B does not depend on the head).
// The contraction runs over the chunk's tokens in steps of 32.  Both operands
// arrive token-major from HBM, while an MFMA fragment needs 8 consecutive
// contraction slots per lane, so each step stages them through LDS
// transposed: a thread loads an 8-token x 8-column block with 16-byte loads,
// transposes it in registers (scaling the x rows by w_j on the way, in fp32,
// then rounding to the operand type) and writes 8 16-byte rows of the
// K-contiguous tiles Bt[n][j] and Xt[p][j].  Wave w then owns output row
// tiles n = 16*(w + 4*i) and all column tiles of the slice.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

#include <type_traits>

namespace ssd {

constexpr int kCsThreadsState = 256;
constexpr int kStateKS = 32;  // tokens per contraction step

template <class Op>
struct StateCfg {
  using E = typename OpElem<Op>::type;
  // LDS row pitch (elements) of the K-contiguous tiles; keeps rows 16-byte
  // aligned and spreads the 16 rows one fragment read touches over distinct
  // banks.
  static constexpr int KP = kStateKS + (Op::kBytes == 2 ? 8 : 4);
};

template <class Op, int RW, int CT, int HPB>
__global__ __launch_bounds__(kCsThreadsState) void chunk_state_kernel(
    const void* __restrict__ x, const void* __restrict__ Bm, int in_bf16, const float* __restrict__ dt_bhl,
    const float* __restrict__ dA_cumsum, void* __restrict__ states, int states_bf16, int L, int H, int P, int N,
    int G, int Q, int nc) {
  using E = typename OpElem<Op>::type;
  using Frag = typename Op::Frag;
  constexpr int PT = CT * 16;
  constexpr int KP = StateCfg<Op>::KP;
  extern __shared__ __align__(16) unsigned char st_smem[];
  E* Bt = reinterpret_cast<E*>(st_smem);    // [N][KP]
  E* Xt = Bt + (size_t)N * KP;               // [HPB][PT][KP]
  float* w_s = reinterpret_cast<float*>(Xt + HPB * PT * KP);  // [HPB][Q]

  const int npt = P / PT;
  const int h0 = (blockIdx.x / npt) * HPB, pt = blockIdx.x - (blockIdx.x / npt) * npt;
  const int c = blockIdx.y, b = blockIdx.z;
  const int g = h0 / (H / G);
  const int p0 = pt * PT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const bool bf = in_bf16 != 0;

  for (int idx = tid; idx < HPB * Q; idx += kCsThreadsState) {
    const int hp = idx / Q, j = idx - (idx / Q) * Q;
    const int64_t bhc = ((int64_t)b * H + h0 + hp) * nc + c;
    const float* Gc = dA_cumsum + bhc * Q;
    w_s[idx] = fast_exp(Gc[Q - 1] - Gc[j]) * dt_bhl[bhc * Q + j];
  }

  f32x4_t acc[HPB][RW][CT];
#pragma unroll
  for (int hp = 0; hp < HPB; ++hp)
#pragma unroll
    for (int i = 0; i < RW; ++i)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[hp][i][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int NT = N / 16;
  const int64_t tok0 = (int64_t)b * L + (int64_t)c * Q;
  // rows past the end of the sequence (ragged last chunk) re-read the last
  // one; their weight w = exp(.) * dt is 0
  const int rmax = min(Q, L - c * Q) - 1;
  const int nbB = (kStateKS / 8) * (N / 8);
  const int nbX = (kStateKS / 8) * (PT / 8);

  for (int k0 = 0; k0 < Q; k0 += kStateKS) {
    __syncthreads();  // previous step's fragment reads are done; w_s is visible
    for (int blk = tid; blk < nbB + HPB * nbX; blk += kCsThreadsState) {
      float v[8][8];
      if (blk < nbB) {
        const int jb = blk & 3, cb = blk >> 2;
#pragma unroll
        for (int r = 0; r < 8; ++r)
          load8_as_f32(Bm, ((tok0 + min(k0 + 8 * jb + r, rmax)) * G + g) * N + 8 * cb, bf, v[r]);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float col[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) col[r] = v[r][q];
          Lds<Op>::store8(Bt + (8 * cb + q) * KP + 8 * jb, col);
        }
      } else {
        const int hp = (blk - nbB) / nbX, bx = (blk - nbB) - hp * nbX;
        const int jb = bx & 3, cb = bx >> 2;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          load8_as_f32(x, ((tok0 + min(k0 + 8 * jb + r, rmax)) * H + h0 + hp) * P + p0 + 8 * cb, bf, v[r]);
          const float w = w_s[hp * Q + k0 + 8 * jb + r];
#pragma unroll
          for (int q = 0; q < 8; ++q) v[r][q] *= w;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float col[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) col[r] = v[r][q];
          Lds<Op>::store8(Xt + (hp * PT + 8 * cb + q) * KP + 8 * jb, col);
        }
      }
    }
    __syncthreads();

#pragma unroll
    for (int hp = 0; hp < HPB; ++hp) {
      Frag bfr[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) bfr[ct] = Lds<Op>::load8(Xt + (hp * PT + 16 * ct + l16) * KP + 8 * lg);
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int rt = wave + 4 * i;
        if (rt < NT) {
          const Frag afr = Lds<Op>::load8(Bt + (16 * rt + l16) * KP + 8 * lg);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) acc[hp][i][ct] = Op::mma(afr, bfr[ct], acc[hp][i][ct]);
        }
      }
    }
  }

  // fp32 states, or (states_bf16) rounded to bf16, nearest even
#pragma unroll
  for (int hp = 0; hp < HPB; ++hp) {
    const int64_t so = (((int64_t)b * nc + c) * H + h0 + hp) * (int64_t)N * P;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int rt = wave + 4 * i;
      if (rt < NT) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t e = so + (int64_t)(16 * rt + 4 * lg + r) * P + p0 + 16 * ct + l16;
            if (states_bf16)
              static_cast<uint16_t*>(states)[e] = (uint16_t)f32_to_bf16_bits(acc[hp][i][ct][r]);
            else
              static_cast<float*>(states)[e] = acc[hp][i][ct][r];
          }
      }
    }
  }
}

static int state_ct(int64_t P) { return (P % 64 == 0) ? 4 : (P % 32 == 0) ? 2 : 1; }
static int state_rw(int64_t N) {
  const int64_t nt = N / 16;
  const int64_t rw = (nt + 3) / 4;
  return rw <= 1 ? 1 : rw <= 2 ? 2 : 4;
}

static size_t state_lds_bytes_hpb(const Dims& d, bool f32_mma, int hpb) {
  const int PT = 16 * state_ct(d.P);
  const size_t eb = f32_mma ? 4 : 2;
  const size_t KP = f32_mma ? StateCfg<OpF32>::KP : StateCfg<OpBF16>::KP;
  return eb * KP * (size_t)(d.N + hpb * PT) + sizeof(float) * (size_t)(hpb * d.Q);
}

// the one-head form; the launcher takes HPB = 4 only where that also fits
size_t chunk_state_lds_bytes(const Dims& d, bool f32_mma) { return state_lds_bytes_hpb(d, f32_mma, 1); }

// Heads per block: 4 where they divide the group, the LDS holds their tiles
// and the grid still has two blocks per compute unit, else 1.
static int state_hpb(const Dims& d, bool f32_mma) {
  const int64_t hpg = d.H / d.G;
  const int PT = 16 * state_ct(d.P);
  const int64_t blocks4 = d.B * d.nc * (d.H / 4) * (d.P / PT);
  if (hpg % 4 == 0 && state_lds_bytes_hpb(d, f32_mma, 4) <= 160 * 1024 && blocks4 >= 2 * (int64_t)device_cu_count())
    return 4;
  return 1;
}

template <class Op, int RW, int CT, int HPB>
static hipError_t launch_state_hpb(const Dims& d, const void* x, const void* Bm, bool in_bf16,
                                   const float* dt_bhl, const float* dA_cumsum, void* states,
                                   bool states_bf16, hipStream_t stream) {
  auto kern = chunk_state_kernel<Op, RW, CT, HPB>;
  const size_t lds = state_lds_bytes_hpb(d, std::is_same<Op, OpF32>::value, HPB);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(d.H / HPB * (d.P / (16 * CT))), (unsigned)d.nc, (unsigned)d.B);
  hipLaunchKernelGGL(kern, grid, dim3(kCsThreadsState), lds, stream, x, Bm, (int)in_bf16, dt_bhl, dA_cumsum,
                     states, (int)states_bf16, (int)d.L, (int)d.H, (int)d.P, (int)d.N, (int)d.G, (int)d.Q, (int)d.nc);
  return hipGetLastError();
}

template <class Op, int RW, int CT>
static hipError_t launch_state_inst(const Dims& d, const void* x, const void* Bm, bool in_bf16,
                                    const float* dt_bhl, const float* dA_cumsum, void* states,
                                    bool states_bf16, hipStream_t stream) {
  // four heads' accumulators fit the register budget up to 8 tiles per wave
  if constexpr (RW * CT <= 8) {
    if (state_hpb(d, std::is_same<Op, OpF32>::value) == 4)
      return launch_state_hpb<Op, RW, CT, 4>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
  }
  return launch_state_hpb<Op, RW, CT, 1>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
}

template <class Op, int RW>
static hipError_t launch_state_ct(const Dims& d, const void* x, const void* Bm, bool in_bf16,
                                  const float* dt_bhl, const float* dA_cumsum, void* states,
                                  bool states_bf16, hipStream_t stream) {
  switch (state_ct(d.P)) {
    case 4: return launch_state_inst<Op, RW, 4>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
    case 2: return launch_state_inst<Op, RW, 2>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
    default: return launch_state_inst<Op, RW, 1>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
  }
}

template <class Op>
static hipError_t launch_state_op(const Dims& d, const void* x, const void* Bm, bool in_bf16,
                                  const float* dt_bhl, const float* dA_cumsum, void* states,
                                  bool states_bf16, hipStream_t stream) {
  switch (state_rw(d.N)) {
    case 1: return launch_state_ct<Op, 1>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
    case 2: return launch_state_ct<Op, 2>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
    default: return launch_state_ct<Op, 4>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
  }
}

hipError_t launch_chunk_state(const Dims& d, const void* x, const void* Bm, bool in_bf16,
                              const float* dt_bhl, const float* dA_cumsum, float* states,
                              bool f32_mma, hipStream_t stream) {
  return launch_chunk_state_any(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, false, f32_mma, stream);
}

hipError_t launch_chunk_state_any(const Dims& d, const void* x, const void* Bm, bool in_bf16,
                                  const float* dt_bhl, const float* dA_cumsum, void* states, bool states_bf16,
                                  bool f32_mma, hipStream_t stream) {
  if (chunk_state_hg_supported(d, in_bf16, f32_mma))
    return launch_chunk_state_hg(d, x, Bm, dt_bhl, dA_cumsum, states, states_bf16, f32_mma, stream);
  if (f32_mma) return launch_state_op<OpF32>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
  return launch_state_op<OpBF16>(d, x, Bm, in_bf16, dt_bhl, dA_cumsum, states, states_bf16, stream);
}

}  // namespace ssd
