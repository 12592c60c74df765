// forward_fused.hip -- the whole chunked forward in one pass per (batch, head,
// 64-column slice): chunk states, the inter-chunk advance and the chunk
// output, with the running state on chip.  Neither the chunk states nor the
// carried states reach memory.
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), paragraph on the three
// kernels: the state pass walks the chunks in order with the running state on
// chip, and compute_out combines the interaction tile (C.B^T, decayed and
// causally masked), the carried-state term and the skip.  This kernel runs
// both inside one chunk loop.  Per (b, h), with G = dA_cumsum[b,h,c,:] and
// dt = dt_bhl[b,h,c,:] of chunk c (tokens i, j of the chunk):
//     y_i     = exp(G_i) C_i . H_c + sum_{j<=i} (C_i . B_j) exp(G_i - G_j) dt_j x_j + D x_i
//     S_c     = sum_j exp(G_{Q-1} - G_j) dt_j B_j x_j^T
//     H_{c+1} = exp(G_{Q-1}) H_c + S_c,   H_0 = initial state (or 0), final = H_nc
//
// Shape: chunk Q = 128, N = 256 state rows, bf16 x/B/C and bf16 matrix
// operands (fp32 accumulation).  Block = (b, h, 64 columns p), 16 waves; one
// block per compute unit (LDS), so it pays where the carried states are the
// largest tensor of the split path (N = 256, few heads per B/C group).
//
// The fp32 running state H (256 x 64) lives in registers in the MFMA
// accumulator layout: wave w owns rows 128 half + 16 (w % 8) + l16 and the
// columns 32 (w / 8) + 16 q + 4 lg .. +3 (half, q in {0, 1}).  Per chunk the
// x rows, G, dt and w_j = exp(G_{Q-1} - G_j) dt_j are staged once; the B and
// C rows and H_c (rounded to bf16) are staged by halves of the state index
// (the LDS holds one half of each at a time), and every contraction over n
// (C.B^T, C.H_c) accumulates over the two halves:
//   half 0: stage B, C, H_c rows 0..127 | S_c rows 0..127 (and their H
//           update), C.B^T and C.H_c over n < 128
//   half 1: the same for rows 128..255; then the decayed, masked
//           interaction matrix M (bf16) goes to LDS
//   output: y = exp(G_i) C.H_c + M.X + D x, stored.
// S_c is accumulated from the same operands in the same order as the fused
// state walk and the head-group chunk-state kernel (x rows scaled by w_j in
// fp32 and rounded to bf16, token-major fragments from the transposing LDS
// read), and the update is the same fused multiply-add, so the final states
// are bit-identical to theirs.  The loads of the next half (and of the next
// chunk's first half and x rows) are in flight in registers while the
// current one computes.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

namespace {

constexpr int FQ = 128;        // chunk tokens
constexpr int FN = 256;        // state rows
constexpr int FNH = 128;       // state rows staged per half
constexpr int FPT = 64;        // columns per block
constexpr int FW = 16;         // waves per block
constexpr int FT = 64 * FW;
constexpr int NSUB = (FQ / 16) * (FQ / 16 + 1) / 2;  // causal 16x16 sub-tiles of C.B^T (36)
constexpr int SPW = (NSUB + FW - 1) / FW;            // sub-tiles per wave, at most (3)
// Row pitches (elements).  n- or j-indexed rows (Bs, Cs, Ms; read 16 bytes at
// a time by 16 rows x 4 lane groups, Bs also by the transposing read) are 16
// elements past a multiple of 64 dwords; p-indexed rows (Xn, Hn; transposing
// reads of 8 rows x 32 bytes per half wave) an odd multiple of 8 dwords
// modulo 64: both conflict-free.
constexpr int XP = FPT + 16;
constexpr int BP = FNH + 16;
constexpr int MP = FQ + 16;
constexpr size_t kOffXn = 0;                                // [FQ][XP]  x rows of the chunk (bf16)
constexpr size_t kOffBs = kOffXn + (size_t)FQ * XP * 2;     // [FQ][BP]  B rows, one half of n
constexpr size_t kOffCs = kOffBs + (size_t)FQ * BP * 2;     // [FQ][BP]  C rows, one half of n
constexpr size_t kOffHn = kOffCs + (size_t)FQ * BP * 2;     // [FNH][XP] H_c rows of the half (bf16, permuted)
constexpr size_t kOffMs = kOffHn + (size_t)FNH * XP * 2;    // [FQ][MP]  M[i][fpos(j)] (bf16)
constexpr size_t kOffGs = kOffMs + (size_t)FQ * MP * 2;     // [FQ] G in base-2 units
constexpr size_t kOffDt = kOffGs + sizeof(float) * FQ;      // [FQ] dt
constexpr size_t kOffWl = kOffDt + sizeof(float) * FQ;      // [FQ] w_j
constexpr size_t kLdsBytes = kOffWl + sizeof(float) * FQ;

// Slot maps.  The transposing LDS read hands lane group lg, as slots
// 4t + r, the contraction indices 16t + 4lg + r of a 32-block; a 16-byte read
// of a row hands it the stored positions 8lg + 4t + r.  fpos maps an index to
// the stored position that makes the two agree: M rows store j at fpos(j)
// (so the row read of M matches the transposing read of x), and the H_c tile
// stores state index n in row fpos_inv(n) (so its transposing read matches
// the row read of C).
__device__ __forceinline__ int fpos(int n) { return (n & ~31) | ((n & 12) << 1) | ((n & 16) >> 2) | (n & 3); }
__device__ __forceinline__ int fpos_inv(int m) { return (m & ~31) | ((m & 4) << 2) | ((m & 24) >> 1) | (m & 3); }

// causal sub-tile k (row-major over is >= js) -> (is, js)
__device__ __forceinline__ void sub_tile(int k, int& is, int& js) {
  int i = 0;
  while ((i + 1) * (i + 2) / 2 <= k) ++i;
  is = i;
  js = k - i * (i + 1) / 2;
}

}  // namespace

template <bool RAGGED, bool Y_BF16>
__global__ __launch_bounds__(FT) void fwd_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ Cm,
    const float* __restrict__ dt_bhl, const float* __restrict__ dA_cumsum, const float* __restrict__ D,
    const float* __restrict__ init, void* __restrict__ y, float* __restrict__ fin, int L, int H, int P, int G,
    int nc, int npt, int remap) {
  using Op = OpBF16;
  using Frag = Op::Frag;
  extern __shared__ __align__(16) unsigned char ff_smem[];
  uint16_t* Xn = reinterpret_cast<uint16_t*>(ff_smem + kOffXn);
  uint16_t* Bs = reinterpret_cast<uint16_t*>(ff_smem + kOffBs);
  uint16_t* Cs = reinterpret_cast<uint16_t*>(ff_smem + kOffCs);
  uint16_t* Hn = reinterpret_cast<uint16_t*>(ff_smem + kOffHn);
  uint16_t* Ms = reinterpret_cast<uint16_t*>(ff_smem + kOffMs);
  float* Gs = reinterpret_cast<float*>(ff_smem + kOffGs);
  float* Dts = reinterpret_cast<float*>(ff_smem + kOffDt);
  float* Wl = reinterpret_cast<float*>(ff_smem + kOffWl);

  // block -> (b, h, column slice).  Logical blocks run over (b, h, slice) with
  // the heads of a group consecutive; with remap they land on one XCD, whose
  // L2 then serves the group's B and C rows to all of them.
  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  if (remap) bid = (bid & 7u) * (nblk >> 3) + (bid >> 3);
  const int pt = bid % npt;
  const unsigned rest = bid / npt;
  const int h = rest % H;
  const int b = rest / H;
  const int g = h / (H / G);
  const int p0 = pt * FPT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t bh = (int64_t)b * H + h;
  const int64_t NP = (int64_t)FN * P;
  const float dsk = D[h];

  // ---- running state: rows 128 half + 16 nt + l16, columns 32 pp + 16 q + 4 lg
  const int nt = wave & 7, pp = wave >> 3;
  float4 hs[2][2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int q = 0; q < 2; ++q)
      hs[hf][q] = init ? *reinterpret_cast<const float4*>(init + bh * NP + (int64_t)(FNH * hf + 16 * nt + l16) * P +
                                                          p0 + 32 * pp + 16 * q + 4 * lg)
                       : make_float4(0.f, 0.f, 0.f, 0.f);

  // ---- output tiles: token row tiles ta = w % 4 and tb = 7 - ta (together
  // five 32-token steps of M.X, whatever the pair), 16 columns 16 yp ..
  const int ta = wave & 3, tb = 7 - ta, yp = wave >> 2;
  // ---- C.B^T sub-tiles of this wave: k = wave + 16 s
  int sis[SPW], sjs[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    const int k = wave + FW * s;
    sub_tile(k < NSUB ? k : 0, sis[s], sjs[s]);
  }

  // ---- register prefetch.  x: thread t takes the 16-byte piece t % 8 of row
  // t / 8; B and C halves: pieces q = t and t + FT, row q / 16, 8 state
  // indices 8 (q % 16); G and dt: token t % 128 (all threads load, branch-free,
  // so the memory-counter waits stay exact).
  uint4 xv, bv[2], cv[2];
  float gv = 0.f, dv = 0.f, glv = 0.f;
  // Global addresses: a wave-uniform base per chunk (scalar registers) plus a
  // 32-bit per-lane offset (row offsets within a chunk fit in 32 bits).
  auto row = [&](int c, int r) -> int {
    const int rmax = RAGGED ? min(FQ, L - c * FQ) - 1 : FQ - 1;
    return RAGGED ? min(r, rmax) : r;
  };
  const int GN = G * FN, HP = H * P;
  auto issue_bc = [&](int c, int hf) __attribute__((always_inline)) {
    const int64_t cb0 = (((int64_t)b * L + (int64_t)c * FQ) * G + g) * FN + FNH * hf;
    const uint16_t* bsrc = Bm + cb0;
    const uint16_t* csrc = Cm + cb0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + FT * u;
      const unsigned off = (unsigned)(row(c, q >> 4) * GN + 8 * (q & 15));
      bv[u] = *reinterpret_cast<const uint4*>(bsrc + off);
      cv[u] = *reinterpret_cast<const uint4*>(csrc + off);
    }
  };
  auto issue_x = [&](int c) __attribute__((always_inline)) {
    const uint16_t* xsrc = x + (((int64_t)b * L + (int64_t)c * FQ) * H + h) * (int64_t)P + p0;
    xv = *reinterpret_cast<const uint4*>(xsrc + (unsigned)(row(c, tid >> 3) * HP + 8 * (tid & 7)));
    const float* gsrc = dA_cumsum + (bh * nc + c) * FQ;
    const float* dsrc = dt_bhl + (bh * nc + c) * FQ;
    gv = gsrc[tid & (FQ - 1)];
    dv = dsrc[tid & (FQ - 1)];
    glv = gsrc[FQ - 1];
  };
  auto commit_bc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + FT * u;
      const int o = (q >> 4) * BP + 8 * (q & 15);
      const uint4 bq = bv[u], cq = cv[u];
      *reinterpret_cast<uint4*>(Bs + o) = make_uint4(bq.x, bq.y, bq.z, bq.w);
      *reinterpret_cast<uint4*>(Cs + o) = make_uint4(cq.x, cq.y, cq.z, cq.w);
    }
  };
  // x rows raw; G (base 2), dt and w_j (the fused state walk's expression)
  auto commit_x = [&]() __attribute__((always_inline)) {
    const uint4 q = xv;
    *reinterpret_cast<uint4*>(Xn + (tid >> 3) * XP + 8 * (tid & 7)) = make_uint4(q.x, q.y, q.z, q.w);
    if (tid < FQ) {
      Gs[tid] = gv * kLog2e;
      Dts[tid] = dv;
      Wl[tid] = fast_exp(glv - gv) * dv;
    }
  };
  // H_c rows of one half -> Hn (bf16, row fpos_inv(n)), from the owning lanes
  auto commit_h = [&](int hf) __attribute__((always_inline)) {
    const int row = fpos_inv(16 * nt + l16);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float4 v = hs[hf][q];
      *reinterpret_cast<uint2*>(Hn + row * XP + 32 * pp + 16 * q + 4 * lg) =
          make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    }
  };

  f32x4_t cbacc[SPW];  // C.B^T sub-tiles (transposed: lane holds j = 16 js + 4 lg + r of row i = 16 is + l16)
  f32x4_t ya, yb;      // y^T tiles of rows ta, tb (lane: i = 16 t + l16, p = 16 yp + 4 lg + r)

  // S_c rows of one half and the state update: S^T = (w x)^T B, fragments
  // from the transposing reads of Xn (scaled by w_j in fp32, rounded to bf16)
  // and Bs; H_{c+1} = exp(G_{Q-1}) H_c + S_c.
  auto state_half = [&](int hf, float glast, int ln) __attribute__((always_inline)) {
    const int lgl = ln >> 4;
    f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < FQ / 32; ++kk) {
      const Frag bf = lds_frag_tr(Bs + 32 * kk * BP + 16 * nt, BP, ln);
      const float4 w0 = *reinterpret_cast<const float4*>(Wl + 32 * kk + 4 * lgl);
      const float4 w1 = *reinterpret_cast<const float4*>(Wl + 32 * kk + 16 + 4 * lgl);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const Frag xf = lds_frag_tr(Xn + 32 * kk * XP + 32 * pp + 16 * q, XP, ln);
        Frag xw;
        xw.v.x = pack_bf16x2(bf16_bits_to_f32(xf.v.x & 0xffffu) * w0.x, bf16_bits_to_f32(xf.v.x >> 16) * w0.y);
        xw.v.y = pack_bf16x2(bf16_bits_to_f32(xf.v.y & 0xffffu) * w0.z, bf16_bits_to_f32(xf.v.y >> 16) * w0.w);
        xw.v.z = pack_bf16x2(bf16_bits_to_f32(xf.v.z & 0xffffu) * w1.x, bf16_bits_to_f32(xf.v.z >> 16) * w1.y);
        xw.v.w = pack_bf16x2(bf16_bits_to_f32(xf.v.w & 0xffffu) * w1.z, bf16_bits_to_f32(xf.v.w >> 16) * w1.w);
        acc[q] = Op::mma(xw, bf, acc[q]);
      }
    }
    const float dec = expf(glast);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float4& hv = hs[hf][q];
      hv.x = fmaf(dec, hv.x, acc[q][0]);
      hv.y = fmaf(dec, hv.y, acc[q][1]);
      hv.z = fmaf(dec, hv.z, acc[q][2]);
      hv.w = fmaf(dec, hv.w, acc[q][3]);
    }
  };
  // C.B^T and C.H_c over the staged half of n (row reads of Bs / Cs, the
  // transposing read of Hn)
  auto contract_half = [&](int ln) __attribute__((always_inline)) {
    const int l16l = ln & 15, lgl = ln >> 4;
#pragma unroll 1
    for (int kk = 0; kk < FNH / 32; ++kk) {
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        if (wave + FW * s < NSUB) {
          const Frag bf = Lds<Op>::load8(Bs + (16 * sjs[s] + l16l) * BP + 32 * kk + 8 * lgl);
          const Frag cf = Lds<Op>::load8(Cs + (16 * sis[s] + l16l) * BP + 32 * kk + 8 * lgl);
          cbacc[s] = Op::mma(bf, cf, cbacc[s]);
        }
      }
      const Frag hf = lds_frag_tr(Hn + 32 * kk * XP + 16 * yp, XP, ln);
      const Frag ca = Lds<Op>::load8(Cs + (16 * ta + l16l) * BP + 32 * kk + 8 * lgl);
      const Frag cb = Lds<Op>::load8(Cs + (16 * tb + l16l) * BP + 32 * kk + 8 * lgl);
      ya = Op::mma(hf, ca, ya);
      yb = Op::mma(hf, cb, yb);
    }
  };

  // Ms: the sub-tiles above the diagonal pairs are never written; zero once
  for (int e = tid; e < FQ * MP / 8; e += FT) reinterpret_cast<uint4*>(Ms)[e] = make_uint4(0, 0, 0, 0);

  issue_x(0);
  issue_bc(0, 0);
  for (int c = 0; c < nc; ++c) {
    const int64_t tok0 = (int64_t)b * L + (int64_t)c * FQ;
    const int rmax = RAGGED ? min(FQ, L - c * FQ) - 1 : FQ - 1;
    // ---- half 0 staged (the previous chunk's last barrier ended all reads)
    const float glast = glv;
    commit_x();
    commit_bc();
    commit_h(0);
    __syncthreads();
    issue_bc(c, 1);
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int s = 0; s < SPW; ++s) cbacc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    ya = f32x4_t{0.f, 0.f, 0.f, 0.f};
    yb = f32x4_t{0.f, 0.f, 0.f, 0.f};
    state_half(0, glast, ln);
    contract_half(ln);
    __syncthreads();
    // ---- half 1 (H_c rows 128.. are not yet advanced)
    commit_bc();
    commit_h(1);
    __syncthreads();
    const int cn = c + 1 < nc ? c + 1 : c;  // past the end: this chunk again, unused
    issue_x(cn);
    state_half(1, glast, ln);
    contract_half(ln);
    // ---- M = C.B^T * exp(G_i - G_j) * dt_j on and below the diagonal, 0 above
    {
      const int l16l = ln & 15, lgl = ln >> 4;
#pragma unroll
      for (int s = 0; s < SPW; ++s) {
        if (wave + FW * s < NSUB) {
          const int i = 16 * sis[s] + l16l, j0 = 16 * sjs[s] + 4 * lgl;
          const float gi = Gs[i];
          const float4 gj = *reinterpret_cast<const float4*>(Gs + j0);
          const float4 dj = *reinterpret_cast<const float4*>(Dts + j0);
          const float gjv[4] = {gj.x, gj.y, gj.z, gj.w}, djv[4] = {dj.x, dj.y, dj.z, dj.w};
          float m[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float dec = fast_exp2(j0 + r <= i ? gi - gjv[r] : -INFINITY);
            m[r] = cbacc[s][r] * djv[r] * dec;
          }
          *reinterpret_cast<uint2*>(Ms + i * MP + fpos(j0)) =  // j0 .. j0 + 3 stay consecutive
              make_uint2(pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3]));
        }
      }
      // the carried-state term takes exp(G_i) per row
      const float ea = fast_exp2(Gs[16 * ta + l16l]), eb = fast_exp2(Gs[16 * tb + l16l]);
      ya *= ea;
      yb *= eb;
    }
    issue_bc(cn, 0);
    __syncthreads();
    // ---- M.X (transposed: x^T fragments from the transposing read of Xn, M
    // rows read directly), skip, store
    {
      const int l16l = ln & 15, lgl = ln >> 4;
#pragma unroll
      for (int k = 0; k < FQ / 32; ++k) {
        if (k <= (tb >> 1)) {
          const Frag xf = lds_frag_tr(Xn + 32 * k * XP + 16 * yp, XP, ln);
          if (k <= (ta >> 1)) {
            const Frag ma = Lds<Op>::load8(Ms + (16 * ta + l16l) * MP + 32 * k + 8 * lgl);
            ya = Op::mma(xf, ma, ya);
          }
          const Frag mb = Lds<Op>::load8(Ms + (16 * tb + l16l) * MP + 32 * k + 8 * lgl);
          yb = Op::mma(xf, mb, yb);
        }
      }
      const int64_t ybase = h * (int64_t)P + p0 + 16 * yp + 4 * lgl;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int i = 16 * (t2 ? tb : ta) + l16l;
        const f32x4_t acc = t2 ? yb : ya;
        const uint2 xq = *reinterpret_cast<const uint2*>(Xn + i * XP + 16 * yp + 4 * lgl);
        const float v0 = acc[0] + dsk * bf16_bits_to_f32(xq.x & 0xffffu);
        const float v1 = acc[1] + dsk * bf16_bits_to_f32(xq.x >> 16);
        const float v2 = acc[2] + dsk * bf16_bits_to_f32(xq.y & 0xffffu);
        const float v3 = acc[3] + dsk * bf16_bits_to_f32(xq.y >> 16);
        if (!RAGGED || i <= rmax) {
          const int64_t o = (tok0 + i) * H * (int64_t)P + ybase;
          if constexpr (Y_BF16)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + o) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          else
            *reinterpret_cast<float4*>(static_cast<float*>(y) + o) = make_float4(v0, v1, v2, v3);
        }
      }
    }
    __syncthreads();
  }
  if (fin) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        *reinterpret_cast<float4*>(fin + bh * NP + (int64_t)(FNH * hf + 16 * nt + l16) * P + p0 + 32 * pp + 16 * q +
                                   4 * lg) = hs[hf][q];
  }
}

// ------------------------------------------------------------------ host side
bool fwd_fused_supported(const Dims& d, bool in_bf16, bool f32_mma) {
  return in_bf16 && !f32_mma && d.Q == FQ && d.N == FN && d.P % FPT == 0 &&
         d.B * d.H * (d.P / FPT) <= 0x7fffffff;
}

hipError_t launch_fwd_fused(const Dims& d, const void* x, const void* Bm, const void* Cm, const float* dt_bhl,
                            const float* dA_cumsum, const float* D, const float* initial_states, void* y, bool y_bf16,
                            float* final_states, hipStream_t stream) {
  const bool ragged = d.L % FQ != 0;
  auto kern = ragged ? (y_bf16 ? fwd_fused_kernel<true, true> : fwd_fused_kernel<true, false>)
                     : (y_bf16 ? fwd_fused_kernel<false, true> : fwd_fused_kernel<false, false>);
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (e != hipSuccess) return e;
  const int npt = (int)(d.P / FPT);
  const int64_t nblk = d.B * d.H * npt;
  const int remap = (nblk % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(FT), kLdsBytes, stream, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(Bm), static_cast<const uint16_t*>(Cm), dt_bhl, dA_cumsum, D,
                     initial_states, y, final_states, (int)d.L, (int)d.H, (int)d.P, (int)d.G, (int)d.nc, npt, remap);
  return hipGetLastError();
}

}  // namespace ssd
