// bwd_dbc.hip -- gradients of B and C for one chunk, summed over the heads of
// a group, on the matrix cores.
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com): the backward pass is only
// previewed there; what is computed is the derivative of the recurrence of
// its opening and jump-formula paragraphs,
//     h_t = r_t h_{t-1} + dt_t B_t x_t^T,  r_t = exp(dt_t A),  y_t = C_t^T h_t + D x_t.
// Inside chunk c (positions i, j; G = in-chunk cumulative sum of dt A, so that
// the decay from token j to token i >= j is exp(G_i - G_j)), with Hc^h the
// state of head h entering the chunk and dH^h the gradient of the state
// leaving it through the later chunks only:
//   U[i][j] = sum_h exp(G_i - G_j) dt_j (dy_i . x_j)       for j <= i, else 0
//   dC_i    = sum_{j <= i} U[i][j] B_j + sum_h exp(G_i) Hc^h dy_i
//   dB_j    = sum_{i >= j} U[i][j] C_i + sum_h dt_j exp(G_last - G_j) dH^h x_j
// (the heads h run over the group that shares B and C).  U is the per-group
// sum of the heads' decayed dy.x Gram matrices, so the products with B and C
// run once per group instead of once per head.
//
// bwd_part_kernel: one block per (b, c, g, slice of the group's heads); every
//   x, dy and state element is read once.  The loop over (head, slice of the
//   head dimension) accumulates in registers, as transposed 16x16 tiles:
//     U^T[j][i]   (DO_U)  the raw dy.x Gram tile of the head (one matrix-core
//                 product per 32-deep step), scaled per element by its decay
//                 and added: below the diagonal tile the decay is split at the
//                 last row E of j's tile, exp(G_i - G_E) exp(G_E - G_j), both
//                 factors <= 1; on the diagonal tile exp(G_i - G_j) is taken
//                 per element with the exponent selected before exp (j > i
//                 gives 0);
//     S^T[n][k]   (DO_S)  the carried-state part, sum_p St[n][p] col_k[p]
//                 scaled per column k: dC: col = dy, St = Hc, factor
//                 exp(G_k); dB: col = x, St = dH, factor r dt_k exp(G_last -
//                 G_k) with r the decay step to the next chunk's first token.
//   Partial sums per head slice go to the workspace (fp32).
// bwd_fin_kernel: one block per (b, c, g, tile T of TI = min(64, Q) rows):
//   sums the slices, then dC^T += B^T U^T over U's row panel of T and
//   dB^T += C^T U over its column panel.
//
// Operands are bf16 (rounded to nearest even) or, with fp32 matrix operands,
// fp32; accumulation is fp32.  Products are 16x16x32 steps of the matrix cores
// (eight 16x16x4 steps for fp32 operands).  An accumulator tile holds, in lane
// (i = lane % 16, q = lane / 16), rows 4q .. 4q+3 of column i: since the
// products are stored transposed, each lane owns 4 consecutive output columns
// of one row, written with 16-byte stores.
#include <algorithm>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

// Transposing fragment read for either operand type: lane (i = lane % 16,
// q = lane / 16) receives as slots 4t + r the element
// tile[(16t + 4q + r) * pitch + i], t = 0, 1, r = 0..3.
template <class Op> struct FragTr;
template <> struct FragTr<OpBF16> {
  __device__ __forceinline__ static OpBF16::Frag load(const uint16_t* tile, int pitch, int lane) {
    return lds_frag_tr(tile, pitch, lane);
  }
};
template <> struct FragTr<OpF32> {
  __device__ __forceinline__ static OpF32::Frag load(const float* tile, int pitch, int lane) {
    const float* p = tile + 4 * (lane >> 4) * pitch + (lane & 15);
    OpF32::Frag f;
    f.lo = make_float4(p[0], p[pitch], p[2 * pitch], p[3 * pitch]);
    p += 16 * pitch;
    f.hi = make_float4(p[0], p[pitch], p[2 * pitch], p[3 * pitch]);
    return f;
  }
};

// One 16-byte piece of an input row: 8 bf16 or 4 fp32 elements, widened.
__device__ __forceinline__ int unpack16(const uint4 v, bool bf16, float* out) {
  if (bf16) {
    out[0] = bf16_bits_to_f32(v.x & 0xffffu); out[1] = bf16_bits_to_f32(v.x >> 16);
    out[2] = bf16_bits_to_f32(v.y & 0xffffu); out[3] = bf16_bits_to_f32(v.y >> 16);
    out[4] = bf16_bits_to_f32(v.z & 0xffffu); out[5] = bf16_bits_to_f32(v.z >> 16);
    out[6] = bf16_bits_to_f32(v.w & 0xffffu); out[7] = bf16_bits_to_f32(v.w >> 16);
    return 8;
  }
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
  return 4;
}

__device__ __forceinline__ uint4 load16(const void* base, int64_t elem, bool bf16) {
  const char* p = static_cast<const char*>(base) + elem * (bf16 ? 2 : 4);
  return *reinterpret_cast<const uint4*>(p);
}

// n (4 or 8) values into LDS in the operand type
__device__ __forceinline__ void store_vals(uint16_t* p, const float* v, int n) {
  if (n == 8)
    *reinterpret_cast<uint4*>(p) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
  else
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ void store_vals(float* p, const float* v, int n) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  if (n == 8) *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
// A 16-byte input piece into LDS: bf16 bits are copied as they are when the
// operand type is bf16, anything else goes through fp32.
__device__ __forceinline__ void store_piece(uint16_t* p, const uint4 v, bool bf16) {
  if (bf16) {
    *reinterpret_cast<uint4*>(p) = v;
  } else {
    float f[8];
    unpack16(v, false, f);
    store_vals(p, f, 4);
  }
}
__device__ __forceinline__ void store_piece(float* p, const uint4 v, bool bf16) {
  float f[8];
  const int n = unpack16(v, bf16, f);
  store_vals(p, f, n);
}

template <class Op> struct DbcPitch {
  typedef typename OpElem<Op>::type E;
  static constexpr bool kB = sizeof(E) == 2;
  // rows read 16 bytes per lane (operand rows), and rows read by the
  // transposing reads of the final products (bf16: ds_read_b64_tr_b16; fp32:
  // 4-byte reads)
  __host__ __device__ static constexpr int op(int ps) { return ps + (kB ? 16 : 8); }
  __host__ __device__ static constexpr int tr(int cols) { return cols + (kB ? 16 : 4); }
};

// ---------------------------------------------------------------- partial sums
struct PartArgs {
  const void* col;     // [B, L, H, P]: dy (U and dC) or x (dB) -- the column operand
  const void* x;       // [B, L, H, P]: x, the row operand of U
  const void* st;      // dC: forward carried states [B, nc, H, N, P];
                       // dB: adjoint carried states in reversed chunk order
                       // (fp32, or bf16 bits when st_bf16)
  const float* dA;     // dA_cumsum [B, H, nc, Q]
  const float* dtb;    // dt_bhl   [B, H, nc, Q]
  const float* A;      // [H]
  float* uout;         // [S, B*nc*G, Q, Q] (tiles on and below the diagonal)
  float* sout;         // [S, B*nc*G, Q, N]
  int L, H, P, N, G, Q, nc, S, hps;
  int col_bf16, x_bf16, st_bf16;
};

template <class Op>
size_t part_lds_bytes(int Q, int N, int PS, bool do_u, bool do_s) {
  const size_t e = sizeof(typename OpElem<Op>::type);
  const int PP = DbcPitch<Op>::op(PS);
  const size_t rows = (size_t)Q + (do_u ? Q : 0) + (do_s ? N : 0);
  return rows * PP * e + 2 * 4 * (size_t)Q * sizeof(float);
}

// NW waves; CPW column tiles (16 positions each) per wave: wave w owns
// column w and, with CPW = 2, column 2 NW - 1 - w (so that the causal U work,
// (w + 1) + (2 NW - w) tiles, is the same on every wave).
// KIND_DB: the state part is dB's (column operand x, adjoint states, factor
// r dt_k exp(G_last - G_k)), else dC's (column operand dy, forward states,
// factor exp(G_k)).
template <class Op, int PS, int NW, int CPW, bool DO_U, bool DO_S, bool KIND_DB, int NTS>
__global__ __launch_bounds__(64 * NW) void bwd_part_kernel(PartArgs a) {
  typedef typename OpElem<Op>::type E;
  typedef typename Op::Frag Frag;
  constexpr int T = 64 * NW;
  constexpr int PP = DbcPitch<Op>::op(PS);
  constexpr int KS = PS / 32;
  constexpr int KP = NW == 8 ? 4 : 2;      // 16-byte pieces per thread: Q rows of one slice
  constexpr int KSP = NW == 8 ? 4 : 8;     // ... and N state rows
  constexpr int UT0 = NW == 8 ? 8 : 4;     // U tiles of the first column (<= w + 1)
  constexpr int UT1 = CPW == 2 ? 2 * NW : 1;
  constexpr int NT16MAX = NTS;              // state tiles per column, N <= 16 NTS
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lg = lane >> 4;
  const int Q = a.Q, P = a.P, N = a.N, H = a.H, T16 = Q / 16, NT16 = N / 16;
  const int s = blockIdx.x % a.S;
  const int bcg = blockIdx.x / a.S;
  const int g = bcg % a.G, c = (bcg / a.G) % a.nc, b = bcg / a.G / a.nc;
  const int hpg = H / a.G, h_lo = g * hpg + s * a.hps, nh = min(a.hps, hpg - s * a.hps);
  const int NPS = (P + PS - 1) / PS, NU = nh * NPS;
  const int64_t tok0 = (int64_t)b * a.L + (int64_t)c * Q;
  const int nvalid = min(Q, a.L - c * Q);
  const bool cb16 = a.col_bf16 != 0, xb16 = a.x_bf16 != 0;

  E* sCol = reinterpret_cast<E*>(smem);       // [Q][PP] column operand
  E* sX = sCol + Q * PP;                      // [Q][PP] x (DO_U)
  E* sSt = sX + (DO_U ? Q * PP : 0);          // [N][PP] states (DO_S)
  float* sSc = reinterpret_cast<float*>(sSt + (DO_S ? N * PP : 0));
  // per buffer: G [Q], the below-diagonal factor exp(G_E - G_j) dt_j [Q],
  // dt [Q], the state factor per column [Q]
  auto scb = [&](int buf) { return sSc + buf * 4 * Q; };

  const int ccpr = PS / (cb16 ? 8 : 4), cepc = cb16 ? 8 : 4;
  const int xcpr = PS / (xb16 ? 8 : 4), xepc = xb16 ? 8 : 4;
  const bool sb16 = a.st_bf16 != 0;
  const int scpr = PS / (sb16 ? 8 : 4), sepc = sb16 ? 8 : 4;

  uint4 pc[KP], px[KP], pst[KSP];
  float pg[4];
  float rho_e = 0.f;  // dB: exponent of r (dt of the next chunk's first token times A)
  auto issue = [&](int u) {
    const int hh = u / NPS, p0 = (u - hh * NPS) * PS, h = h_lo + hh;
    const int64_t cb = ((int64_t)(b * H + h) * a.nc + c) * Q;
    pg[0] = tid < Q ? a.dA[cb + tid] : 0.f;
    pg[1] = tid < Q ? a.dtb[cb + tid] : 0.f;
    pg[2] = tid < Q ? a.dA[cb + (tid | 15)] : 0.f;
    pg[3] = a.dA[cb + Q - 1];
    if (KIND_DB) rho_e = c + 1 < a.nc ? a.dtb[cb + Q] * a.A[h] : 0.f;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int q = tid + T * k;
      pc[k] = make_uint4(0, 0, 0, 0);
      if (q < Q * ccpr) {
        const int j = q / ccpr, p = p0 + (q - j * ccpr) * cepc;
        if (j < nvalid && p < P) pc[k] = load16(a.col, ((tok0 + j) * H + h) * P + p, cb16);
      }
      if (DO_U) {
        px[k] = make_uint4(0, 0, 0, 0);
        if (q < Q * xcpr) {
          const int j = q / xcpr, p = p0 + (q - j * xcpr) * xepc;
          if (j < nvalid && p < P) px[k] = load16(a.x, ((tok0 + j) * H + h) * P + p, xb16);
        }
      }
    }
    if (DO_S) {
      const int64_t sc = KIND_DB ? ((int64_t)b * a.nc + (a.nc - 1 - c)) : ((int64_t)b * a.nc + c);
      const int64_t st0 = (sc * H + h) * N * P;
#pragma unroll
      for (int k = 0; k < KSP; ++k) {
        const int q = tid + T * k;
        pst[k] = make_uint4(0, 0, 0, 0);
        if (q < N * scpr) {
          const int n = q / scpr, p = p0 + (q - n * scpr) * sepc;
          if (p < P) pst[k] = load16(a.st, st0 + (int64_t)n * P + p, sb16);
        }
      }
    }
  };
  auto commit_scales = [&](int buf) {
    float* sc = scb(buf);
    if (tid < Q) {
      sc[tid] = pg[0];
      sc[Q + tid] = fast_exp(pg[2] - pg[0]) * pg[1];
      sc[2 * Q + tid] = pg[1];
      sc[3 * Q + tid] = KIND_DB ? fast_exp(pg[3] - pg[0] + rho_e) * pg[1] : fast_exp(pg[0]);
    }
  };
  auto commit_ops = [&]() {
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int q = tid + T * k;
      if (q < Q * ccpr) {
        const int j = q / ccpr;
        store_piece(sCol + j * PP + (q - j * ccpr) * cepc, pc[k], cb16);
      }
      if (DO_U && q < Q * xcpr) {
        const int j = q / xcpr;
        store_piece(sX + j * PP + (q - j * xcpr) * xepc, px[k], xb16);
      }
    }
    if (DO_S) {
#pragma unroll
      for (int k = 0; k < KSP; ++k) {
        const int q = tid + T * k;
        if (q < N * scpr) {
          const int n = q / scpr;
          store_piece(sSt + n * PP + (q - n * scpr) * sepc, pst[k], sb16);
        }
      }
    }
  };

  const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t accU0[DO_U ? UT0 : 1], accU1[DO_U ? UT1 : 1], accS[DO_S ? CPW : 1][DO_S ? NT16MAX : 1];
#pragma unroll
  for (int k = 0; k < (DO_U ? UT0 : 1); ++k) accU0[k] = z4;
#pragma unroll
  for (int k = 0; k < (DO_U ? UT1 : 1); ++k) accU1[k] = z4;
#pragma unroll
  for (int cc = 0; cc < (DO_S ? CPW : 1); ++cc)
#pragma unroll
    for (int k = 0; k < (DO_S ? NT16MAX : 1); ++k) accS[cc][k] = z4;

  // the wave's columns
  const int I0 = w, I1 = CPW == 2 ? 2 * NW - 1 - w : 0;
  const bool active = I0 < T16;

  // decayed Gram tile (I, J) of the current head added into acc
  auto u_tile = [&](f32x4_t& acc, const Frag (&bd)[KS], int I, int J, const float* sc) {
    f32x4_t t = z4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      t = Op::mma(Lds<Op>::load8(sX + (16 * J + l16) * PP + 32 * ks + 8 * lg), bd[ks], t);
    const int i = 16 * I + l16;
    const float gi = sc[i];
    if (J < I) {
      const float fa = fast_exp(gi - sc[16 * J + 15]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = fmaf(t[r], fa * sc[Q + 16 * J + 4 * lg + r], acc[r]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * J + 4 * lg + r;
        acc[r] = fmaf(t[r], fast_exp(j <= i ? gi - sc[j] : -INFINITY) * sc[2 * Q + j], acc[r]);
      }
    }
  };

  auto compute = [&](int buf) {
    if (!active) return;
    const float* sc = scb(buf);
    Frag bd0[KS], bd1[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bd0[ks] = Lds<Op>::load8(sCol + (16 * I0 + l16) * PP + 32 * ks + 8 * lg);
      bd1[ks] = CPW == 2 ? Lds<Op>::load8(sCol + (16 * I1 + l16) * PP + 32 * ks + 8 * lg) : bd0[ks];
    }
    if (DO_U) {
#pragma unroll
      for (int J = 0; J < UT0; ++J)
        if (J <= I0) u_tile(accU0[J], bd0, I0, J, sc);
      if (CPW == 2) {
#pragma unroll
        for (int J = 0; J < UT1; ++J)
          if (J <= I1) u_tile(accU1[J], bd1, I1, J, sc);
      }
    }
    if (DO_S) {
      const float f0 = sc[3 * Q + 16 * I0 + l16];
      const float f1 = CPW == 2 ? sc[3 * Q + 16 * I1 + l16] : 0.f;
#pragma unroll
      for (int k = 0; k < NT16MAX; ++k) {
        if (k >= NT16) continue;
        f32x4_t t0 = z4, t1 = z4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const Frag af = Lds<Op>::load8(sSt + (16 * k + l16) * PP + 32 * ks + 8 * lg);
          t0 = Op::mma(af, bd0[ks], t0);
          if (CPW == 2) t1 = Op::mma(af, bd1[ks], t1);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          accS[0][k][r] = fmaf(t0[r], f0, accS[0][k][r]);
          if (CPW == 2) accS[CPW - 1][k][r] = fmaf(t1[r], f1, accS[CPW - 1][k][r]);
        }
      }
    }
  };

  issue(0);
  commit_scales(0);
  commit_ops();
  __syncthreads();
  for (int u = 0; u < NU; ++u) {
    const int cur = u & 1;
    const bool more = u + 1 < NU;
    if (more) issue(u + 1);
    compute(cur);
    if (more) commit_scales(cur ^ 1);
    __syncthreads();
    if (more) {
      commit_ops();
      __syncthreads();
    }
  }

  // ---- partial sums of this head slice
  if (!active) return;
  const int64_t pidx = (int64_t)s * (gridDim.x / a.S) + bcg;
  if (DO_U) {
    float* U = a.uout + pidx * Q * Q;
    auto put = [&](const f32x4_t& v, int I, int J) {
      *reinterpret_cast<float4*>(U + (int64_t)(16 * I + l16) * Q + 16 * J + 4 * lg) =
          make_float4(v[0], v[1], v[2], v[3]);
    };
#pragma unroll
    for (int J = 0; J < UT0; ++J)
      if (J <= I0) put(accU0[J], I0, J);
    if (CPW == 2) {
#pragma unroll
      for (int J = 0; J < UT1; ++J)
        if (J <= I1) put(accU1[J], I1, J);
    }
  }
  if (DO_S) {
    float* Sp = a.sout + pidx * Q * N;
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int i = 16 * (cc == 0 ? I0 : I1) + l16;
#pragma unroll
      for (int k = 0; k < NT16MAX; ++k)
        if (k < NT16)
          *reinterpret_cast<float4*>(Sp + (int64_t)i * N + 16 * k + 4 * lg) =
              make_float4(accS[cc][k][0], accS[cc][k][1], accS[cc][k][2], accS[cc][k][3]);
    }
  }
}

// ---------------------------------------------------------------- final products
struct FinArgs {
  const float* upart;  // [S, B*nc*G, Q, Q]
  const float* cpart;  // [S, B*nc*G, Q, N] dC's carried-state part
  const float* bpart;  // [S, B*nc*G, Q, N] dB's carried-state part
  const void* Bm;      // [B, L, G, N]
  const void* Cm;
  float* dB;           // [B, L, G, N]
  float* dC;
  int L, N, G, Q, nc, S, TI, NT;
  int in_bf16;
};

constexpr int kFinThreads = 256;
constexpr int kNSlice = 64;  // B / C columns staged at a time

template <class Op>
size_t fin_lds_bytes(int Q, int TI) {
  const size_t e = sizeof(typename OpElem<Op>::type);
  const int UP = DbcPitch<Op>::tr(TI), BP = DbcPitch<Op>::tr(kNSlice);
  return (size_t)(Q + TI) * UP * e + (size_t)Q * BP * e;
}

template <class Op, int NS4>
__global__ __launch_bounds__(kFinThreads) void bwd_fin_kernel(FinArgs a) {
  typedef typename OpElem<Op>::type E;
  typedef typename Op::Frag Frag;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lg = lane >> 4;
  const int t = blockIdx.x % a.NT;
  const int bcg = blockIdx.x / a.NT;
  const int g = bcg % a.G, c = (bcg / a.G) % a.nc, b = bcg / a.G / a.nc;
  const int Q = a.Q, N = a.N, TI = a.TI, R = t * TI, J = R + TI, NI = Q - R;
  const int CT = TI / 16, NT16 = N / 16;
  const int64_t tok0 = (int64_t)b * a.L + (int64_t)c * Q;
  const int nvalid = min(Q, a.L - c * Q);
  const int64_t nbcg = (int64_t)(gridDim.x / a.NT);
  const int UP = DbcPitch<Op>::tr(TI), BP = DbcPitch<Op>::tr(kNSlice);
  E* sUt = reinterpret_cast<E*>(smem);  // [J][UP]: U^T of the row panel, sUt[j][i] = U[R + i][j]
  E* sU = sUt + J * UP;                 // [NI][UP]: column panel, sU[i][j] = U[R + i][R + j]
  E* sBC = sU + NI * UP;                // [J or NI][BP]: B or C rows, kNSlice columns

  // U[i][j .. j+3] summed over the head slices (in slice order); zero above
  // the diagonal (those entries of the slices' tiles on the diagonal are zero
  // already, the tiles right of it are never written).  A thread sums UQ
  // pieces at a time with the loads of US slices in flight together before
  // any add: a load-then-add or load-then-store sequence per piece would wait
  // out one memory latency each (loads complete in order).
  constexpr int UQ = 4, US = 4;
  auto usum_batch = [&](int q0, int nq, int cols, int ioff, int joff, float4 (&v)[UQ], int (&ii)[UQ],
                        int (&jj)[UQ]) {
    bool ok[UQ];
#pragma unroll
    for (int u = 0; u < UQ; ++u) {
      const int q = q0 + u * kFinThreads;
      ok[u] = q < nq;
      ii[u] = ok[u] ? q / (cols / 4) : 0;
      jj[u] = ok[u] ? (q - ii[u] * (cols / 4)) * 4 : 0;
      ok[u] = ok[u] && joff + jj[u] <= ioff + ii[u];
      v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int s0 = 0; s0 < a.S; s0 += US) {
      float4 p[US][UQ];
#pragma unroll
      for (int sv = 0; sv < US; ++sv)
#pragma unroll
        for (int u = 0; u < UQ; ++u)
          p[sv][u] = ok[u] && s0 + sv < a.S
                         ? *reinterpret_cast<const float4*>(a.upart + (((s0 + sv) * nbcg + bcg) * Q + ioff + ii[u]) *
                                                                          (int64_t)Q + joff + jj[u])
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int sv = 0; sv < US; ++sv)
#pragma unroll
        for (int u = 0; u < UQ; ++u)
          if (s0 + sv < a.S) {
            v[u].x += p[sv][u].x; v[u].y += p[sv][u].y; v[u].z += p[sv][u].z; v[u].w += p[sv][u].w;
          }
    }
#pragma unroll
    for (int u = 0; u < UQ; ++u) {
      const int i = ioff + ii[u], j = joff + jj[u];
      if (j + 1 > i) v[u].y = 0.f;
      if (j + 2 > i) v[u].z = 0.f;
      if (j + 3 > i) v[u].w = 0.f;
    }
  };
  for (int q0 = tid; q0 < TI * (J / 4); q0 += UQ * kFinThreads) {
    float4 v[UQ];
    int ii[UQ], jj[UQ];
    usum_batch(q0, TI * (J / 4), J, R, 0, v, ii, jj);
#pragma unroll
    for (int u = 0; u < UQ; ++u) {
      if (q0 + u * kFinThreads >= TI * (J / 4)) continue;
      const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (sizeof(E) == 2) sUt[(jj[u] + r) * UP + ii[u]] = (E)f32_to_bf16_bits(vv[r]);
        else sUt[(jj[u] + r) * UP + ii[u]] = vv[r];
      }
    }
  }
  for (int q0 = tid; q0 < NI * (TI / 4); q0 += UQ * kFinThreads) {
    float4 v[UQ];
    int ii[UQ], jj[UQ];
    usum_batch(q0, NI * (TI / 4), TI, R, R, v, ii, jj);
#pragma unroll
    for (int u = 0; u < UQ; ++u) {
      if (q0 + u * kFinThreads >= NI * (TI / 4)) continue;
      const float vv[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      store_vals(sU + ii[u] * UP + jj[u], vv, 4);
    }
  }

  // accumulators start from the carried-state parts: lane (i, q) of tile
  // (k, ct) holds rows n = 16k + 4q .. +3 of column (position) R + 16ct + i
  // (summed in slice order; per slice, the loads of all the thread's tiles
  // are issued before the adds)
  f32x4_t accC[NS4][4], accB[NS4][4];
#pragma unroll
  for (int k = 0; k < NS4; ++k)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      accC[k][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      accB[k][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  // (tiles of KB state-row groups at a time: 16 KB loads in flight)
  constexpr int KB = NS4 < 2 ? NS4 : 2;
#pragma unroll
  for (int k0 = 0; k0 < NS4; k0 += KB)
    for (int s = 0; s < a.S; ++s) {
      float4 pc[KB][4], pb[KB][4];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int s16 = w + 4 * (k0 + kk);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          pc[kk][ct] = pb[kk][ct] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (s16 < NT16 && ct < CT) {
            const int64_t row = R + 16 * ct + l16;
            const int64_t off = ((s * nbcg + bcg) * Q + row) * N + 16 * s16 + 4 * lg;
            pc[kk][ct] = *reinterpret_cast<const float4*>(a.cpart + off);
            pb[kk][ct] = *reinterpret_cast<const float4*>(a.bpart + off);
          }
        }
      }
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          if (w + 4 * (k0 + kk) < NT16 && ct < CT) {
            f32x4_t& c4 = accC[k0 + kk][ct];
            f32x4_t& b4 = accB[k0 + kk][ct];
            c4[0] += pc[kk][ct].x; c4[1] += pc[kk][ct].y; c4[2] += pc[kk][ct].z; c4[3] += pc[kk][ct].w;
            b4[0] += pb[kk][ct].x; b4[1] += pb[kk][ct].y; b4[2] += pb[kk][ct].z; b4[3] += pb[kk][ct].w;
          }
        }
    }

  const bool ib = a.in_bf16 != 0;
  const int epc = ib ? 8 : 4, cpr = kNSlice / epc;
  // stage rows [r0, r0 + nr) of B or C, columns [ns0, ns0 + kNSlice): UQ
  // pieces per thread at a time, their loads issued before the stores
  auto stage = [&](const void* src, int r0, int nr, int ns0) {
    for (int q0 = tid; q0 < nr * cpr; q0 += UQ * kFinThreads) {
      uint4 raw[UQ];
      bool ok[UQ];
#pragma unroll
      for (int u = 0; u < UQ; ++u) {
        const int q = q0 + u * kFinThreads;
        const int j = q / cpr, n = ns0 + (q - j * cpr) * epc;
        ok[u] = q < nr * cpr && r0 + j < nvalid && n < N;
        raw[u] = ok[u] ? load16(src, ((tok0 + r0 + j) * a.G + g) * N + n, ib) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < UQ; ++u) {
        const int q = q0 + u * kFinThreads;
        if (q >= nr * cpr) continue;
        const int j = q / cpr, e0 = (q - j * cpr) * epc;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        int cnt = epc;
        if (ok[u]) cnt = unpack16(raw[u], ib, v);
        store_vals(sBC + j * BP + e0, v, cnt);
      }
    }
  };
  for (int ns0 = 0; ns0 < N; ns0 += kNSlice) {
    // dC^T += B^T U^T over the rows j < J
    stage(a.Bm, 0, J, ns0);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NS4; ++k) {
      const int s16 = w + 4 * k;
      if (s16 < NT16 && 16 * s16 >= ns0 && 16 * s16 < ns0 + kNSlice) {
        for (int kj = 0; kj < J; kj += 32) {
          const Frag af = FragTr<Op>::load(sBC + kj * BP + 16 * s16 - ns0, BP, lane);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            if (ct < CT) accC[k][ct] = Op::mma(af, FragTr<Op>::load(sUt + kj * UP + 16 * ct, UP, lane), accC[k][ct]);
        }
      }
    }
    __syncthreads();
    // dB^T += C^T U over the rows i >= R
    stage(a.Cm, R, NI, ns0);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NS4; ++k) {
      const int s16 = w + 4 * k;
      if (s16 < NT16 && 16 * s16 >= ns0 && 16 * s16 < ns0 + kNSlice) {
        for (int ki = 0; ki < NI; ki += 32) {
          const Frag af = FragTr<Op>::load(sBC + ki * BP + 16 * s16 - ns0, BP, lane);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            if (ct < CT) accB[k][ct] = Op::mma(af, FragTr<Op>::load(sU + ki * UP + 16 * ct, UP, lane), accB[k][ct]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < NS4; ++k) {
    const int s16 = w + 4 * k;
    if (s16 >= NT16) continue;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int i = R + 16 * ct + l16;
      if (ct < CT && i < nvalid) {
        const int64_t off = ((tok0 + i) * a.G + g) * N + 16 * s16 + 4 * lg;
        *reinterpret_cast<float4*>(a.dC + off) =
            make_float4(accC[k][ct][0], accC[k][ct][1], accC[k][ct][2], accC[k][ct][3]);
        *reinterpret_cast<float4*>(a.dB + off) =
            make_float4(accB[k][ct][0], accB[k][ct][1], accB[k][ct][2], accB[k][ct][3]);
      }
    }
  }
}

// ---------------------------------------------------------------- host side
// Head slices per (b, c, g): enough blocks for the 256 compute units of the
// target device (a shape-only rule, so that the workspace size is too).
int dbc_slices(const Dims& d) {
  const int64_t bcg = d.B * d.nc * d.G, hpg = d.H / d.G;
  const int64_t s = (256 + bcg - 1) / bcg;
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, hpg));
}

template <class Op, int PS, int NW, int CPW, bool DO_U, bool DO_S, bool KIND_DB, int NTS>
hipError_t launch_part(const Dims& d, const PartArgs& a, hipStream_t s) {
  const size_t lds = part_lds_bytes<Op>((int)d.Q, (int)d.N, PS, DO_U, DO_S);
  auto kern = &bwd_part_kernel<Op, PS, NW, CPW, DO_U, DO_S, KIND_DB, NTS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(d.B * d.nc * d.G * a.S)), dim3(64 * NW), lds, s, a);
  return hipGetLastError();
}

template <class Op, int PS, int NW, int CPW, bool KIND_DB>
hipError_t launch_state_part(const Dims& d, const PartArgs& a, hipStream_t s) {
  if (d.N <= 64) return launch_part<Op, PS, NW, CPW, false, true, KIND_DB, 4>(d, a, s);
  if (d.N <= 128) return launch_part<Op, PS, NW, CPW, false, true, KIND_DB, 8>(d, a, s);
  return launch_part<Op, PS, NW, CPW, false, true, KIND_DB, 16>(d, a, s);
}

// The partial-sum launches for one operand type, staged slice width and
// chunk-size class: U, dC's carried-state part, dB's.
template <class Op, int PS, int NW, int CPW>
hipError_t launch_parts(const Dims& d, const PartArgs& ac, const PartArgs& ab, hipStream_t s) {
  hipError_t e = launch_part<Op, PS, NW, CPW, true, false, false, 1>(d, ac, s);
  if (e == hipSuccess) e = launch_state_part<Op, PS, NW, CPW, false>(d, ac, s);
  if (e == hipSuccess) e = launch_state_part<Op, PS, NW, CPW, true>(d, ab, s);
  return e;
}

template <class Op, int PS>
hipError_t launch_parts_q(const Dims& d, const PartArgs& ac, const PartArgs& ab, hipStream_t s) {
  if (d.Q == 256) return launch_parts<Op, PS, 8, 2>(d, ac, ab, s);
  if (d.Q == 128) return launch_parts<Op, PS, 8, 1>(d, ac, ab, s);
  return launch_parts<Op, PS, 4, 1>(d, ac, ab, s);
}

template <class Op, int NS4>
hipError_t launch_fin_inst(const Dims& d, const FinArgs& f, hipStream_t s) {
  const size_t lds = fin_lds_bytes<Op>((int)d.Q, f.TI);
  auto kern = &bwd_fin_kernel<Op, NS4>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(d.B * d.nc * d.G * f.NT)), dim3(kFinThreads), lds, s, f);
  return hipGetLastError();
}

template <class Op>
hipError_t launch_fin(const Dims& d, const FinArgs& f, hipStream_t s) {
  if (d.N <= 64) return launch_fin_inst<Op, 1>(d, f, s);
  if (d.N <= 128) return launch_fin_inst<Op, 2>(d, f, s);
  return launch_fin_inst<Op, 4>(d, f, s);
}

}  // namespace

bool bwd_dbc_supported(const Dims& d) {
  return (d.Q == 32 || d.Q == 64 || d.Q == 128 || d.Q == 256) && d.N % 16 == 0 && d.N <= 256 && d.P % 16 == 0 &&
         d.H % d.G == 0;
}

size_t bwd_dbc_lds_bytes(const Dims& d, bool f32_mma) {
  const int Q = (int)d.Q, N = (int)d.N, TI = Q < 64 ? Q : 64;
  if (f32_mma)
    return std::max({part_lds_bytes<OpF32>(Q, N, 32, true, false), part_lds_bytes<OpF32>(Q, N, 32, false, true),
                     fin_lds_bytes<OpF32>(Q, TI)});
  return std::max({part_lds_bytes<OpBF16>(Q, N, 64, true, false), part_lds_bytes<OpBF16>(Q, N, 64, false, true),
                   fin_lds_bytes<OpBF16>(Q, TI)});
}

size_t bwd_dbc_ws_bytes(const Dims& d) {
  const size_t S = (size_t)dbc_slices(d), bcg = (size_t)(d.B * d.nc * d.G);
  return sizeof(float) * S * bcg * (size_t)d.Q * ((size_t)d.Q + 2 * (size_t)d.N);
}

hipError_t launch_bwd_dbc(const Dims& d, const void* x, bool x_bf16, const void* dy, bool dy_bf16, const void* Bm,
                          const void* Cm, bool in_bf16, const float* dA_cumsum, const float* dt_bhl,
                          const void* fwd_carried, const void* adj_carried_rev, bool st_bf16, const float* A,
                          float* ws, float* dB, float* dC, bool f32_mma, hipStream_t s) {
  if (!bwd_dbc_supported(d)) return hipErrorInvalidValue;
  const int S = dbc_slices(d);
  const int64_t bcg = d.B * d.nc * d.G;
  float* upart = ws;
  float* cpart = upart + (size_t)S * bcg * d.Q * d.Q;
  float* bpart = cpart + (size_t)S * bcg * d.Q * d.N;
  PartArgs a;
  a.x = x; a.dA = dA_cumsum; a.dtb = dt_bhl; a.A = A;
  a.L = (int)d.L; a.H = (int)d.H; a.P = (int)d.P; a.N = (int)d.N; a.G = (int)d.G; a.Q = (int)d.Q;
  a.nc = (int)d.nc; a.S = S; a.hps = (int)((d.H / d.G + S - 1) / S);
  a.x_bf16 = x_bf16;
  a.st_bf16 = st_bf16;
  // dC (and U): column operand dy, forward states; dB: column operand x, adjoint states
  PartArgs ac = a, ab = a;
  ac.col = dy; ac.col_bf16 = dy_bf16; ac.st = fwd_carried; ac.uout = upart; ac.sout = cpart;
  ab.col = x; ab.col_bf16 = x_bf16; ab.st = adj_carried_rev; ab.uout = nullptr; ab.sout = bpart;
  hipError_t e;
  // staged head-dimension slice: 64 for bf16 operands from bf16 inputs with
  // N <= 128, else 32 (bounds the prefetch registers and the LDS)
  if (f32_mma) e = launch_parts_q<OpF32, 32>(d, ac, ab, s);
  else if (x_bf16 && dy_bf16 && d.N <= 128) e = launch_parts_q<OpBF16, 64>(d, ac, ab, s);
  else e = launch_parts_q<OpBF16, 32>(d, ac, ab, s);
  if (e != hipSuccess) return e;
  FinArgs f;
  f.upart = upart; f.cpart = cpart; f.bpart = bpart; f.Bm = Bm; f.Cm = Cm; f.dB = dB; f.dC = dC;
  f.L = (int)d.L; f.N = (int)d.N; f.G = (int)d.G; f.Q = (int)d.Q; f.nc = (int)d.nc; f.S = S;
  f.TI = d.Q < 64 ? (int)d.Q : 64;
  f.NT = (int)d.Q / f.TI;
  f.in_bf16 = in_bf16;
  return f32_mma ? launch_fin<OpF32>(d, f, s) : launch_fin<OpBF16>(d, f, s);
}

}  // namespace ssd
