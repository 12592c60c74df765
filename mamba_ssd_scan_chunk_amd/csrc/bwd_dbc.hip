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
// bwd_dc_kernel: one block per (b, c, g, tile T of TI = min(64, Q) rows i).
//   The loop over (head, slice of the head dimension) accumulates, in
//   registers, the transposed tiles
//     U^T[j][i] for j < start(T)       = sum x~_j . dy~_i,  with the decay
//                                         split at R = start(T):
//                                         x~_j = exp(G_R - G_j) dt_j x_j,
//                                         dy~_i = exp(G_i - G_R) dy_i (both
//                                         factors <= 1, no overflow);
//     U^T[j][i] for j, i in T          = raw dy.x Gram, decayed and causally
//                                         masked per element (the exponent is
//                                         selected before exp);
//     dC^T[n][i] (carried-state part)  = sum (exp(G_R) Hc)[n] . dy~_i.
//   Then U's rows of T are stored (fp32, for bwd_db_kernel), U^T is staged in
//   LDS and dC^T += B^T U^T completes the tile.
// bwd_db_kernel: one block per (b, c, g, tile T of rows j).  The same loop
//   accumulates dB^T[n][j] = sum (rho dH)[n] . (dt_j exp(G_last - G_j) x_j),
//   then dB^T += C^T U over the rows i >= start(T) of U's column panel.
//
// Operands are bf16 (rounded to nearest even) or, with fp32 matrix operands,
// fp32; accumulation is fp32.  Every product is a 16x16x32 step of the
// matrix cores (eight 16x16x4 steps for fp32 operands).  Accumulator tiles of
// one 16x16 output hold, in lane (i = lane % 16, q = lane / 16), rows
// 4q .. 4q+3 of column i: stored as the transposed products above, each lane
// owns 4 consecutive output columns of one row, written with 16-byte stores.
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

// n (4 or 8) scaled values into LDS in the operand type
__device__ __forceinline__ void store_scaled(uint16_t* p, const float* v, int n, float s) {
  if (n == 8) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0] * s, v[1] * s), pack_bf16x2(v[2] * s, v[3] * s),
                                              pack_bf16x2(v[4] * s, v[5] * s), pack_bf16x2(v[6] * s, v[7] * s));
  } else {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0] * s, v[1] * s), pack_bf16x2(v[2] * s, v[3] * s));
  }
}
__device__ __forceinline__ void store_scaled(float* p, const float* v, int n, float s) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0] * s, v[1] * s, v[2] * s, v[3] * s);
  if (n == 8) *reinterpret_cast<float4*>(p + 4) = make_float4(v[4] * s, v[5] * s, v[6] * s, v[7] * s);
}
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }

struct DbcArgs {
  const void* x;      // [B, L, H, P]
  const void* dy;     // [B, L, H, P]
  const void* bc;     // B (bwd_dc) or C (bwd_db), [B, L, G, N]
  const float* dA;    // dA_cumsum [B, H, nc, Q]
  const float* dtb;   // dt_bhl   [B, H, nc, Q]
  const float* st;    // bwd_dc: states entering each chunk [B, nc, H, N, P];
                      // bwd_db: adjoint carried states in reversed chunk order
  const float* A;     // [H]; bwd_db: with dt of the next chunk's first token, one decay step
  float* U;           // [B, nc, G, Q, Q]
  float* out;         // dC or dB [B, L, G, N]
  int L, H, P, N, G, Q, nc, TI, NT;
  int x_bf16, dy_bf16, in_bf16;
};

constexpr int kDbcThreads = 256;
constexpr int kNSlice = 64;  // B / C columns staged at a time in the final products

template <class Op> struct DbcPitch {
  typedef typename OpElem<Op>::type E;
  static constexpr bool kB = sizeof(E) == 2;
  // operand rows read 16 bytes per lane, and the transposing reads of the
  // final products (bf16: ds_read_b64_tr_b16; fp32: 4-byte reads)
  __host__ __device__ static constexpr int op(int ps) { return ps + (kB ? 16 : 8); }
  __host__ __device__ static constexpr int tr(int cols) { return cols + (kB ? 16 : 4); }
};

template <class Op>
size_t dbc_lds_bytes(int Q, int TI, int N, int PS, bool dc) {
  typedef typename OpElem<Op>::type E;
  const size_t e = sizeof(E);
  const int PP = DbcPitch<Op>::op(PS), UP = DbcPitch<Op>::tr(TI), BP = DbcPitch<Op>::tr(kNSlice);
  const size_t ops = dc ? (size_t)(2 * TI + Q + N) * PP * e : (size_t)(TI + N) * PP * e;
  const size_t fin = (size_t)Q * UP * e + (size_t)Q * BP * e;
  const size_t region = (std::max(ops, fin) + 15) / 16 * 16;
  const size_t scales = dc ? 2 * (size_t)(Q + 3 * TI) * sizeof(float) : 2 * (size_t)TI * sizeof(float);
  return region + scales;
}

// block -> (b, c, g, tile); consecutive logical blocks (the tiles of one
// chunk) on the same XCD so that its L2 serves their shared rows and states
__device__ __forceinline__ void dbc_block(const DbcArgs& a, int& b, int& c, int& g, int& tile) {
  unsigned bid = blockIdx.x;
  const unsigned nb = gridDim.x;
  if ((nb & 7u) == 0) bid = (bid & 7u) * (nb >> 3) + (bid >> 3);
  tile = bid % a.NT;
  unsigned rest = bid / a.NT;
  g = rest % a.G;
  rest /= a.G;
  c = rest % a.nc;
  b = rest / a.nc;
}

// ---------------------------------------------------------------- dC and U
// Per-thread prefetch slots (16-byte pieces): x rows (<= 256 x 128 bytes),
// dy rows (64 x 128 bytes), state rows (<= 256 x 128 bytes).
constexpr int kPX = 8, kPDY = 2, kPH = 8;

template <class Op, int PS, int NS4>
__global__ __launch_bounds__(kDbcThreads) void bwd_dc_kernel(DbcArgs a) {
  typedef typename OpElem<Op>::type E;
  typedef typename Op::Frag Frag;
  constexpr int PP = DbcPitch<Op>::op(PS);
  constexpr int KS = PS / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lg = lane >> 4;
  int b, c, g, it;
  dbc_block(a, b, c, g, it);
  const int Q = a.Q, TI = a.TI, R = it * TI, J = R + TI, P = a.P, N = a.N, H = a.H;
  const int CT = TI / 16, OT = R / 16, NT16 = N / 16;
  const int hpg = H / a.G, NPS = (P + PS - 1) / PS, NU = hpg * NPS;
  const int64_t tok0 = (int64_t)b * a.L + (int64_t)c * Q;
  const int nvalid = min(Q, a.L - c * Q);
  const bool xb = a.x_bf16 != 0, yb = a.dy_bf16 != 0;

  E* sDyS = reinterpret_cast<E*>(smem);
  E* sDyR = sDyS + TI * PP;
  E* sX = sDyR + TI * PP;
  E* sH = sX + Q * PP;
  // the final products reuse the operand area
  const int UP = DbcPitch<Op>::tr(TI), BP = DbcPitch<Op>::tr(kNSlice);
  E* sUt = reinterpret_cast<E*>(smem);
  E* sB = sUt + Q * UP;
  const size_t ops_b = (size_t)(2 * TI + Q + N) * PP * sizeof(E);
  const size_t fin_b = (size_t)Q * (UP + BP) * sizeof(E);
  float* sSc = reinterpret_cast<float*>(smem + ((ops_b > fin_b ? ops_b : fin_b) + 15) / 16 * 16);
  const int SCW = Q + 3 * TI;  // per buffer: x scale [Q], dy scale [TI], G [TI], dt [TI]

  const int xepc = xb ? 8 : 4, xcpr = PS / xepc;  // elements per piece, pieces per row
  const int yepc = yb ? 8 : 4, ycpr = PS / yepc;
  const int hcpr = PS / 4;

  uint4 px[kPX], py[kPDY], ph[kPH];
  float pg[5];
  auto issue = [&](int u) {
    const int hh = u / NPS, p0 = (u - hh * NPS) * PS, h = g * hpg + hh;
    const int64_t cb = ((int64_t)(b * H + h) * a.nc + c) * Q;
    pg[0] = tid < J ? a.dA[cb + tid] : 0.f;
    pg[1] = tid < J ? a.dtb[cb + tid] : 0.f;
    pg[2] = a.dA[cb + R];
    pg[3] = tid < TI ? a.dA[cb + R + tid] : 0.f;
    pg[4] = tid < TI ? a.dtb[cb + R + tid] : 0.f;
#pragma unroll
    for (int k = 0; k < kPX; ++k) {
      const int q = tid + kDbcThreads * k;
      px[k] = make_uint4(0, 0, 0, 0);
      if (q < J * xcpr) {
        const int j = q / xcpr, p = p0 + (q - j * xcpr) * xepc;
        if (j < nvalid && p < P) px[k] = load16(a.x, ((tok0 + j) * H + h) * P + p, xb);
      }
    }
#pragma unroll
    for (int k = 0; k < kPDY; ++k) {
      const int q = tid + kDbcThreads * k;
      py[k] = make_uint4(0, 0, 0, 0);
      if (q < TI * ycpr) {
        const int i = q / ycpr, p = p0 + (q - i * ycpr) * yepc;
        if (R + i < nvalid && p < P) py[k] = load16(a.dy, ((tok0 + R + i) * H + h) * P + p, yb);
      }
    }
    const float* hc = a.st + (((int64_t)b * a.nc + c) * H + h) * N * P;
#pragma unroll
    for (int k = 0; k < kPH; ++k) {
      const int q = tid + kDbcThreads * k;
      ph[k] = make_uint4(0, 0, 0, 0);
      if (q < N * hcpr) {
        const int n = q / hcpr, p = p0 + (q - n * hcpr) * 4;
        if (p < P) ph[k] = *reinterpret_cast<const uint4*>(hc + (int64_t)n * P + p);
      }
    }
  };
  auto commit_scales = [&](int buf) {
    float* sc = sSc + buf * SCW;
    const float gR = pg[2];
    if (tid < J) sc[tid] = tid < R ? fast_exp(gR - pg[0]) * pg[1] : 1.f;
    if (tid < TI) {
      sc[Q + tid] = fast_exp(pg[3] - gR);
      sc[Q + TI + tid] = pg[3];
      sc[Q + 2 * TI + tid] = pg[4];
    }
  };
  auto commit_ops = [&](int buf) {
    const float* sc = sSc + buf * SCW;
    float v[8];
#pragma unroll
    for (int k = 0; k < kPX; ++k) {
      const int q = tid + kDbcThreads * k;
      if (q < J * xcpr) {
        const int j = q / xcpr, e0 = (q - j * xcpr) * xepc;
        const int n = unpack16(px[k], xb, v);
        store_scaled(sX + j * PP + e0, v, n, sc[j]);
      }
    }
#pragma unroll
    for (int k = 0; k < kPDY; ++k) {
      const int q = tid + kDbcThreads * k;
      if (q < TI * ycpr) {
        const int i = q / ycpr, e0 = (q - i * ycpr) * yepc;
        const int n = unpack16(py[k], yb, v);
        store_scaled(sDyS + i * PP + e0, v, n, sc[Q + i]);
        store_scaled(sDyR + i * PP + e0, v, n, 1.f);
      }
    }
    const float hs = fast_exp(pg[2]);
#pragma unroll
    for (int k = 0; k < kPH; ++k) {
      const int q = tid + kDbcThreads * k;
      if (q < N * hcpr) {
        const int n = q / hcpr, e0 = (q - n * hcpr) * 4;
        unpack16(ph[k], false, v);
        store_scaled(sH + n * PP + e0, v, 4, hs);
      }
    }
  };

  f32x4_t accO[3][4], accS[NS4][4], accD[4], tmp[4];
  const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    accD[ct] = z4;
    tmp[ct] = z4;
#pragma unroll
    for (int k = 0; k < 3; ++k) accO[k][ct] = z4;
#pragma unroll
    for (int k = 0; k < NS4; ++k) accS[k][ct] = z4;
  }

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ko = 32 * ks + 8 * lg;
      Frag bs[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (ct < CT) bs[ct] = Lds<Op>::load8(sDyS + (16 * ct + l16) * PP + ko);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int o = w + 4 * k;
        if (o < OT) {
          const Frag af = Lds<Op>::load8(sX + (16 * o + l16) * PP + ko);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            if (ct < CT) accO[k][ct] = Op::mma(af, bs[ct], accO[k][ct]);
        }
      }
#pragma unroll
      for (int k = 0; k < NS4; ++k) {
        const int s = w + 4 * k;
        if (s < NT16) {
          const Frag af = Lds<Op>::load8(sH + (16 * s + l16) * PP + ko);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            if (ct < CT) accS[k][ct] = Op::mma(af, bs[ct], accS[k][ct]);
        }
      }
      if (w < CT) {
        const Frag af = Lds<Op>::load8(sX + (R + 16 * w + l16) * PP + ko);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          if (ct >= w && ct < CT) {
            const Frag br = Lds<Op>::load8(sDyR + (16 * ct + l16) * PP + ko);
            tmp[ct] = Op::mma(af, br, tmp[ct]);
          }
      }
    }
    // the diagonal tile: decay exp(G_i - G_j) dt_j where j <= i, else 0
    if (w < CT) {
      const float* sc = sSc + buf * SCW;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (ct >= w && ct < CT) {
          const int i = 16 * ct + l16;
          const float gi = sc[Q + TI + i];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * w + 4 * lg + r;
            const float f = fast_exp(j <= i ? gi - sc[Q + TI + j] : -INFINITY) * sc[Q + 2 * TI + j];
            accD[ct][r] = fmaf(tmp[ct][r], f, accD[ct][r]);
            tmp[ct][r] = 0.f;
          }
        }
    }
  };

  issue(0);
  commit_scales(0);
  __syncthreads();
  commit_ops(0);
  __syncthreads();
  for (int u = 0; u < NU; ++u) {
    const int cur = u & 1;
    const bool more = u + 1 < NU;
    if (more) issue(u + 1);
    compute(cur);
    if (more) commit_scales(cur ^ 1);
    __syncthreads();
    if (more) {
      commit_ops(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- U's rows of this tile (fp32, row-major [i][j]) for the dB kernel
  float* Ub = a.U + (((int64_t)b * a.nc + c) * a.G + g) * Q * Q;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    if (ct >= CT) continue;
    const int i = R + 16 * ct + l16;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int o = w + 4 * k;
      if (o < OT)
        *reinterpret_cast<float4*>(Ub + (int64_t)i * Q + 16 * o + 4 * lg) =
            make_float4(accO[k][ct][0], accO[k][ct][1], accO[k][ct][2], accO[k][ct][3]);
    }
    if (w < CT)
      *reinterpret_cast<float4*>(Ub + (int64_t)i * Q + R + 16 * w + 4 * lg) =
          make_float4(accD[ct][0], accD[ct][1], accD[ct][2], accD[ct][3]);
  }
  // ---- U^T of this tile into LDS ([j][i], operand type)
  // (the last barrier of the loop ended every read of the operand area)
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    if (ct >= CT) continue;
    const int i = 16 * ct + l16;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int o = w + 4 * k;
      if (o < OT)
#pragma unroll
        for (int r = 0; r < 4; ++r) store_elem(sUt + (16 * o + 4 * lg + r) * UP + i, accO[k][ct][r]);
    }
    if (w < CT)
#pragma unroll
      for (int r = 0; r < 4; ++r) store_elem(sUt + (R + 16 * w + 4 * lg + r) * UP + i, accD[ct][r]);
  }
  // ---- dC^T += B^T U^T, kNSlice columns of B at a time
  const bool ib = a.in_bf16 != 0;
  const int bepc = ib ? 8 : 4, bcpr = kNSlice / bepc;
  for (int ns0 = 0; ns0 < N; ns0 += kNSlice) {
    for (int q = tid; q < J * bcpr; q += kDbcThreads) {
      const int j = q / bcpr, e0 = (q - j * bcpr) * bepc, n = ns0 + e0;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      int cnt = bepc;
      if (j < nvalid && n < N) cnt = unpack16(load16(a.bc, ((tok0 + j) * a.G + g) * N + n, ib), ib, v);
      store_scaled(sB + j * BP + e0, v, cnt, 1.f);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NS4; ++k) {
      const int s = w + 4 * k;
      if (s < NT16 && 16 * s >= ns0 && 16 * s < ns0 + kNSlice) {
        for (int kj = 0; kj < J; kj += 32) {
          const Frag af = FragTr<Op>::load(sB + kj * BP + 16 * s - ns0, BP, lane);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            if (ct < CT) accS[k][ct] = Op::mma(af, FragTr<Op>::load(sUt + kj * UP + 16 * ct, UP, lane), accS[k][ct]);
        }
      }
    }
    __syncthreads();
  }
  // ---- dC rows of this tile: lane (i, q) holds dC[i][16s + 4q .. +3]
#pragma unroll
  for (int k = 0; k < NS4; ++k) {
    const int s = w + 4 * k;
    if (s >= NT16) continue;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int i = R + 16 * ct + l16;
      if (ct < CT && i < nvalid)
        *reinterpret_cast<float4*>(a.out + ((tok0 + i) * a.G + g) * N + 16 * s + 4 * lg) =
            make_float4(accS[k][ct][0], accS[k][ct][1], accS[k][ct][2], accS[k][ct][3]);
    }
  }
}

// ---------------------------------------------------------------- dB
constexpr int kQX = 2, kQH = 8;

template <class Op, int PS, int NS4>
__global__ __launch_bounds__(kDbcThreads) void bwd_db_kernel(DbcArgs a) {
  typedef typename OpElem<Op>::type E;
  typedef typename Op::Frag Frag;
  constexpr int PP = DbcPitch<Op>::op(PS);
  constexpr int KS = PS / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, l16 = lane & 15, lg = lane >> 4;
  int b, c, g, jt;
  dbc_block(a, b, c, g, jt);
  const int Q = a.Q, TI = a.TI, R = jt * TI, P = a.P, N = a.N, H = a.H;
  const int CT = TI / 16, NT16 = N / 16;
  const int hpg = H / a.G, NPS = (P + PS - 1) / PS, NU = hpg * NPS;
  const int64_t tok0 = (int64_t)b * a.L + (int64_t)c * Q;
  const int nvalid = min(Q, a.L - c * Q);
  const bool xb = a.x_bf16 != 0;

  E* sXh = reinterpret_cast<E*>(smem);
  E* sdH = sXh + TI * PP;
  const int UP = DbcPitch<Op>::tr(TI), BP = DbcPitch<Op>::tr(kNSlice);
  E* sU = reinterpret_cast<E*>(smem);
  E* sC = sU + Q * UP;
  const size_t ops_b = (size_t)(TI + N) * PP * sizeof(E);
  const size_t fin_b = (size_t)Q * (UP + BP) * sizeof(E);
  float* sSc = reinterpret_cast<float*>(smem + ((ops_b > fin_b ? ops_b : fin_b) + 15) / 16 * 16);

  const int xepc = xb ? 8 : 4, xcpr = PS / xepc;
  const int hcpr = PS / 4;
  // adjoint carried states are stored in reversed chunk order: the one that
  // enters reversed chunk nc-1-c is the gradient at the first token of chunk
  // c+1, one decay step r = exp(dt A) after the state leaving chunk c
  const float* dh_base = a.st + (((int64_t)b * a.nc + (a.nc - 1 - c)) * H) * N * P;

  uint4 px[kQX], ph[kQH];
  float pg[3], rho = 1.f;
  auto issue = [&](int u) {
    const int hh = u / NPS, p0 = (u - hh * NPS) * PS, h = g * hpg + hh;
    const int64_t cb = ((int64_t)(b * H + h) * a.nc + c) * Q;
    pg[0] = tid < TI ? a.dA[cb + R + tid] : 0.f;
    pg[1] = tid < TI ? a.dtb[cb + R + tid] : 0.f;
    pg[2] = a.dA[cb + Q - 1];
    rho = c + 1 < a.nc ? a.dtb[cb + Q] * a.A[h] : 0.f;  // exponent; dt of the next chunk's first token
#pragma unroll
    for (int k = 0; k < kQX; ++k) {
      const int q = tid + kDbcThreads * k;
      px[k] = make_uint4(0, 0, 0, 0);
      if (q < TI * xcpr) {
        const int j = q / xcpr, p = p0 + (q - j * xcpr) * xepc;
        if (R + j < nvalid && p < P) px[k] = load16(a.x, ((tok0 + R + j) * H + h) * P + p, xb);
      }
    }
    const float* dh = dh_base + (int64_t)h * N * P;
#pragma unroll
    for (int k = 0; k < kQH; ++k) {
      const int q = tid + kDbcThreads * k;
      ph[k] = make_uint4(0, 0, 0, 0);
      if (q < N * hcpr) {
        const int n = q / hcpr, p = p0 + (q - n * hcpr) * 4;
        if (p < P) ph[k] = *reinterpret_cast<const uint4*>(dh + (int64_t)n * P + p);
      }
    }
  };
  auto commit_scales = [&](int buf) {
    if (tid < TI) sSc[buf * TI + tid] = fast_exp(pg[2] - pg[0]) * pg[1];
  };
  auto commit_ops = [&](int buf) {
    const float* sc = sSc + buf * TI;
    float v[8];
#pragma unroll
    for (int k = 0; k < kQX; ++k) {
      const int q = tid + kDbcThreads * k;
      if (q < TI * xcpr) {
        const int j = q / xcpr, e0 = (q - j * xcpr) * xepc;
        const int n = unpack16(px[k], xb, v);
        store_scaled(sXh + j * PP + e0, v, n, sc[j]);
      }
    }
    const float hs = fast_exp(rho);
#pragma unroll
    for (int k = 0; k < kQH; ++k) {
      const int q = tid + kDbcThreads * k;
      if (q < N * hcpr) {
        const int n = q / hcpr, e0 = (q - n * hcpr) * 4;
        unpack16(ph[k], false, v);
        store_scaled(sdH + n * PP + e0, v, 4, hs);
      }
    }
  };

  f32x4_t acc[NS4][4];
  const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < NS4; ++k)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[k][ct] = z4;

  auto compute = [&]() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ko = 32 * ks + 8 * lg;
      Frag bx[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (ct < CT) bx[ct] = Lds<Op>::load8(sXh + (16 * ct + l16) * PP + ko);
#pragma unroll
      for (int k = 0; k < NS4; ++k) {
        const int s = w + 4 * k;
        if (s < NT16) {
          const Frag af = Lds<Op>::load8(sdH + (16 * s + l16) * PP + ko);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            if (ct < CT) acc[k][ct] = Op::mma(af, bx[ct], acc[k][ct]);
        }
      }
    }
  };

  issue(0);
  commit_scales(0);
  __syncthreads();
  commit_ops(0);
  __syncthreads();
  for (int u = 0; u < NU; ++u) {
    const int cur = u & 1;
    const bool more = u + 1 < NU;
    if (more) issue(u + 1);
    compute();
    if (more) commit_scales(cur ^ 1);
    __syncthreads();
    if (more) {
      commit_ops(cur ^ 1);
      __syncthreads();
    }
  }

  // ---- U's column panel: rows i in [R, Q), columns of this tile
  const float* Ub = a.U + (((int64_t)b * a.nc + c) * a.G + g) * Q * Q;
  const int NI = Q - R;
  for (int q = tid; q < NI * (TI / 4); q += kDbcThreads) {
    const int i = q / (TI / 4), e0 = (q - i * (TI / 4)) * 4;
    const float4 v4 = *reinterpret_cast<const float4*>(Ub + (int64_t)(R + i) * Q + R + e0);
    const float v[4] = {v4.x, v4.y, v4.z, v4.w};
    store_scaled(sU + i * UP + e0, v, 4, 1.f);
  }
  // ---- dB^T += C^T U over the rows i >= R
  const bool ib = a.in_bf16 != 0;
  const int cepc = ib ? 8 : 4, ccpr = kNSlice / cepc;
  for (int ns0 = 0; ns0 < N; ns0 += kNSlice) {
    for (int q = tid; q < NI * ccpr; q += kDbcThreads) {
      const int i = q / ccpr, e0 = (q - i * ccpr) * cepc, n = ns0 + e0;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      int cnt = cepc;
      if (R + i < nvalid && n < N) cnt = unpack16(load16(a.bc, ((tok0 + R + i) * a.G + g) * N + n, ib), ib, v);
      store_scaled(sC + i * BP + e0, v, cnt, 1.f);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NS4; ++k) {
      const int s = w + 4 * k;
      if (s < NT16 && 16 * s >= ns0 && 16 * s < ns0 + kNSlice) {
        for (int ki = 0; ki < NI; ki += 32) {
          const Frag af = FragTr<Op>::load(sC + ki * BP + 16 * s - ns0, BP, lane);
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            if (ct < CT) acc[k][ct] = Op::mma(af, FragTr<Op>::load(sU + ki * UP + 16 * ct, UP, lane), acc[k][ct]);
        }
      }
    }
    __syncthreads();
  }
  // ---- dB rows of this tile
#pragma unroll
  for (int k = 0; k < NS4; ++k) {
    const int s = w + 4 * k;
    if (s >= NT16) continue;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int j = R + 16 * ct + l16;
      if (ct < CT && j < nvalid)
        *reinterpret_cast<float4*>(a.out + ((tok0 + j) * a.G + g) * N + 16 * s + 4 * lg) =
            make_float4(acc[k][ct][0], acc[k][ct][1], acc[k][ct][2], acc[k][ct][3]);
    }
  }
}

// Slice of the head dimension staged per step: 64 for bf16 operands from
// bf16 inputs with N <= 128, else 32 (bounds the prefetch registers and LDS).
int dbc_slice(const Dims& d, bool bf16_ops, bool all_bf16) { return bf16_ops && all_bf16 && d.N <= 128 ? 64 : 32; }

template <class Op, int PS, int NS4>
hipError_t launch_dbc_inst(const Dims& d, const DbcArgs& ac, const DbcArgs& ab, hipStream_t s) {
  const unsigned nblk = (unsigned)(d.B * d.nc * d.G * ac.NT);
  const size_t lds_c = dbc_lds_bytes<Op>((int)d.Q, ac.TI, (int)d.N, PS, true);
  const size_t lds_b = dbc_lds_bytes<Op>((int)d.Q, ac.TI, (int)d.N, PS, false);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dc_kernel<Op, PS, NS4>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_c);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_db_kernel<Op, PS, NS4>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_b);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dc_kernel<Op, PS, NS4>), dim3(nblk), dim3(kDbcThreads), lds_c, s, ac);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the dB kernel reads the U rows that every tile of the chunk stored
  hipLaunchKernelGGL((bwd_db_kernel<Op, PS, NS4>), dim3(nblk), dim3(kDbcThreads), lds_b, s, ab);
  return hipGetLastError();
}

template <class Op, int PS>
hipError_t launch_dbc_ns(const Dims& d, const DbcArgs& ac, const DbcArgs& ab, hipStream_t s) {
  if (d.N <= 64) return launch_dbc_inst<Op, PS, 1>(d, ac, ab, s);
  if (d.N <= 128) return launch_dbc_inst<Op, PS, 2>(d, ac, ab, s);
  return launch_dbc_inst<Op, PS, 4>(d, ac, ab, s);
}

}  // namespace

bool bwd_dbc_supported(const Dims& d) {
  return (d.Q == 32 || d.Q == 64 || d.Q == 128 || d.Q == 256) && d.N % 16 == 0 && d.N <= 256 && d.P % 16 == 0 &&
         d.H % d.G == 0;
}

size_t bwd_dbc_u_bytes(const Dims& d) { return sizeof(float) * (size_t)(d.B * d.nc * d.G) * d.Q * d.Q; }

hipError_t launch_bwd_dbc(const Dims& d, const void* x, bool x_bf16, const void* dy, bool dy_bf16, const void* Bm,
                          const void* Cm, bool in_bf16, const float* dA_cumsum, const float* dt_bhl,
                          const float* fwd_carried, const float* adj_carried_rev, const float* A, float* U,
                          float* dB, float* dC, bool f32_mma, hipStream_t s) {
  if (!bwd_dbc_supported(d)) return hipErrorInvalidValue;
  DbcArgs a;
  a.x = x; a.dy = dy; a.dA = dA_cumsum; a.dtb = dt_bhl; a.A = A; a.U = U;
  a.L = (int)d.L; a.H = (int)d.H; a.P = (int)d.P; a.N = (int)d.N; a.G = (int)d.G; a.Q = (int)d.Q;
  a.nc = (int)d.nc;
  a.TI = d.Q < 64 ? (int)d.Q : 64;
  a.NT = (int)d.Q / a.TI;
  a.x_bf16 = x_bf16; a.dy_bf16 = dy_bf16; a.in_bf16 = in_bf16;
  const int ps = dbc_slice(d, !f32_mma, x_bf16 && dy_bf16 && in_bf16);
  DbcArgs ac = a, ab = a;  // the dC kernel: B and the forward states; the dB kernel: C and the adjoint's
  ac.bc = Bm;
  ac.st = fwd_carried;
  ac.out = dC;
  ab.bc = Cm;
  ab.st = adj_carried_rev;
  ab.out = dB;
  if (f32_mma) return launch_dbc_ns<OpF32, 32>(d, ac, ab, s);
  return ps == 64 ? launch_dbc_ns<OpBF16, 64>(d, ac, ab, s) : launch_dbc_ns<OpBF16, 32>(d, ac, ab, s);
}

}  // namespace ssd
