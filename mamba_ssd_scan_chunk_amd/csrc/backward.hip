// backward.hip -- gradients of the SSD forward, composed from forward passes.
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com): the backward pass is
// previewed, not published.  What is computed is the derivative of the same
// recurrence (opening and jump-formula paragraphs),
//     h_t = r_t h_{t-1} + dt_t B_t x_t^T,  r_t = exp(dt_t A),  y_t = C_t^T h_t + D x_t,
// for a loss with dL/dy = dy and dL/dh_{L-1} = dfinal.  The adjoint state
// g_t = dL/dh_t satisfies g_t = C_t dy_t^T + r_{t+1} g_{t+1}: read backwards in
// time that is again this recurrence, with the decay of each step taken from
// dt_{t+1} (none at the last token), input scale 1, B-role C, x-role dy and
// initial state dfinal.  So the products below are chunked forward passes of
// the existing kernels, plus one per-chunk kernel for dB and dC
// (bwd_dbc.hip), and the glue here only reverses, combines and reduces:
//   (0) forward:            y0_t = C_t^T h_t, carried states h
//   (1) adjoint, reversed:  y1_t = B_t^T g_t, carried states g
//                           -> dx = dt y1 + D dy,  beta_t = B_t . g_t x_t = y1_t . x_t,  final = g_0
//   (2) dB, dC per (chunk, group) from x, dy, B, C and the carried states of
//       (0) and (1), summed over the group's heads.
// The reversed pass runs over nc*Q steps, the sequence padded at its far end
// (zero inputs, no decay), so that its chunk edges fall on the forward's.
// Matrix operands are bf16 (rounded to nearest even) or fp32.
// The log-decay gradient needs q_t = <g_t, h_t>, since
//   dL/d(dt_t A) = r_t <g_t, h_{t-1}> = q_t - dt_t beta_t,
//   ddt_t = A dL/d(dt_t A) + beta_t,  dA = sum_t dt_t dL/d(dt_t A).
// Within a chunk q follows q_{t+1} = q_t - dy_t . y0_t + dt_{t+1} beta_{t+1};
// that sum has no decay, so its rounding would pile up over a whole sequence.
// Each chunk therefore starts from an exact anchor, the inner product of the
// carried states at its first token, <g_{kQ}, h_{kQ-1}>, which both state
// passes already hold.  dD = sum_t dy_t . x_t and dh0 = r_0 g_0.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// out[b, s, k, e] = in[b, t(s), k / (KO / KI), e] for s < Lout, with t(s) = s,
// or Lout-1-s when reversing; rows with t >= Lin are zero.  KO/KI maps output
// slots to input slots (heads -> groups when expanding B or C per head).  One
// block per output row (b, s); 4-element groups (E is a multiple of 16).
// Output fp32, or bf16 rounded to nearest even (exact for bf16 input).
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gather_rows_kernel(const void* __restrict__ in, int in_bf16,
                                                          void* __restrict__ out, int Lin, int Lout, int KO, int KI,
                                                          int E, int reverse) {
  const int64_t row = blockIdx.x;  // b * Lout + s
  const int64_t b = row / Lout;
  const int s = (int)(row - b * Lout);
  const int t = reverse ? Lout - 1 - s : s;
  const int E4 = E / 4, W4 = KO * E4, per = KO / KI;
  const int64_t src_row = (b * Lin + t) * KI;
  for (int j = threadIdx.x; j < W4; j += 256) {
    const int k = j / E4, e4 = j - k * E4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < Lin) {
      const int64_t src = (src_row + k / per) * E + 4 * e4;
      if (in_bf16) {
        const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(in) + src);
        v[0] = bf16_bits_to_f32(u.x & 0xffffu);
        v[1] = bf16_bits_to_f32(u.x >> 16);
        v[2] = bf16_bits_to_f32(u.y & 0xffffu);
        v[3] = bf16_bits_to_f32(u.y >> 16);
      } else {
        const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(in) + src);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
      }
    }
    const int64_t dst = row * KO * E + 4 * (int64_t)j;
    if constexpr (OUT_BF16)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + dst) =
          make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    else
      *reinterpret_cast<float4*>(static_cast<float*>(out) + dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// dt of the reversed adjoint over Lp steps: step s carries token t = Lp-1-s and
// decays by dt_{t+1}, so dts[b, s, h] = dt[b, Lp - s, h] where Lp - s < L, else 0.
__global__ __launch_bounds__(256) void shift_reverse_dt_kernel(const float* __restrict__ dt, float* __restrict__ dts,
                                                               int L, int Lp, int H, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int h = (int)(i % H);
  const int64_t r = i / H;
  const int s = (int)(r % Lp);
  const int64_t b = r / Lp;
  const int idx = Lp - s;
  dts[i] = idx < L ? dt[(b * L + idx) * H + h] : 0.f;
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// Input scale of the reversed adjoint, [B,H,nc,Q] (the dt_bhl layout): 1 on
// the steps s = cQ + i that carry a forward token (Lp-1-s < L), 0 on the
// padding steps, whose input rows then contribute nothing whatever they hold.
__global__ __launch_bounds__(256) void step_mask_kernel(float* __restrict__ p, int L, int Lp, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = (Lp - 1 - (int)(i % Lp)) < L ? 1.f : 0.f;
}

// 8 consecutive elements (16-byte aligned group) as fp32
__device__ __forceinline__ void load8_f32(const void* base, int64_t elem, bool bf16, float (&o)[8]) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = bf16_bits_to_f32(w[e] & 0xffffu);
      o[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
}

// anc[b, h, k] = <g_{kQ}, h_{kQ-1}> for k < nc: for k >= 1 the adjoint's
// carried state entering its reversed chunk nc-k and the forward's carried
// state entering chunk k; for k = 0 the adjoint's final state (g_0) and the
// initial state (zero when absent).  anc[b, h, nc] = <dL/dfinal, final state>
// (zero when dfinal is absent).  One block per (b, k, h); states are
// [B, nc, H, N*P], anc is [B, H, nc+1].
// Carried states are fp32, or bf16 bits when st_bf16 (final, initial and
// dfinal states are fp32).
__global__ __launch_bounds__(256) void anchor_dot_kernel(const void* __restrict__ fwd_carried,
                                                         const float* __restrict__ fwd_final,
                                                         const void* __restrict__ adj_carried,
                                                         const float* __restrict__ adj_final,
                                                         const float* __restrict__ h0,
                                                         const float* __restrict__ dfinal, float* __restrict__ anc,
                                                         int H, int nc, int64_t NP, int st_bf16) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int h = blockIdx.x % H;
  const int k = (blockIdx.x / H) % (nc + 1);
  const int64_t b = blockIdx.x / H / (nc + 1);
  const int64_t bh = (b * H + h) * NP;
  const void* gp;
  const void* hp;
  bool bf = false;
  if (k == 0) {
    gp = adj_final + bh;
    hp = h0 ? h0 + bh : nullptr;
  } else if (k == nc) {
    gp = dfinal ? dfinal + bh : nullptr;
    hp = fwd_final + bh;
  } else {
    const int64_t ga = ((b * nc + (nc - k)) * H + h) * NP, ha = ((b * nc + k) * H + h) * NP;
    bf = st_bf16 != 0;
    gp = bf ? static_cast<const void*>(static_cast<const uint16_t*>(adj_carried) + ga)
            : static_cast<const void*>(static_cast<const float*>(adj_carried) + ga);
    hp = bf ? static_cast<const void*>(static_cast<const uint16_t*>(fwd_carried) + ha)
            : static_cast<const void*>(static_cast<const float*>(fwd_carried) + ha);
  }
  float sum = 0.f;
  if (gp && hp)
    for (int64_t e = 8 * tid; e < NP; e += 8 * 256) {  // N*P is a multiple of 256
      float gv[8], hv[8];
      load8_f32(gp, e, bf, gv);
      load8_f32(hp, e, bf, hv);
#pragma unroll
      for (int q = 0; q < 8; ++q) sum = fmaf(gv[q], hv[q], sum);
    }
  // wave sums by shuffles, then the four wave partials in order
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0) anc[(b * H + h) * (nc + 1) + k] = (red[0] + red[1]) + (red[2] + red[3]);
}

// Per (b, t, h): dx, beta_t = y1_t . x_t (= B_t . g_t x_t), v_t = dy_t . y0_t,
// u_t = dy_t . x_t.  8 lanes per (b, t, h) row, 8-element groups (P a
// multiple of 16), eight rows per wave; y1 is in reversed time over Lp steps.
// y0 and y1 are fp32, or bf16 bits when y_bf16.
__global__ __launch_bounds__(256) void combine_token_kernel(
    const void* __restrict__ dy, int dy_bf16, const void* __restrict__ x, int in_bf16, const float* __restrict__ dt,
    const float* __restrict__ D, const void* __restrict__ y0, const void* __restrict__ y1, int y_bf16,
    float* __restrict__ dx, float* __restrict__ beta, float* __restrict__ v, float* __restrict__ u, int L, int Lp,
    int H, int P, int64_t nrows) {
  const int64_t row = (int64_t)blockIdx.x * (blockDim.x / 8) + (threadIdx.x >> 3);  // (b * L + t) * H + h
  const int l8 = threadIdx.x & 7;
  if (row >= nrows) return;  // whole 8-lane groups leave together
  const int h = (int)(row % H);
  const int64_t bt = row / H;
  const int t = (int)(bt % L);
  const int64_t b = bt / L;
  const int64_t rrow = (b * Lp + (Lp - 1 - t)) * H + h;  // the same token in reversed time
  const float dtv = dt[row], dh = D[h];
  float sv = 0.f, su = 0.f, sb = 0.f;
  for (int p = 8 * l8; p < P; p += 64) {
    float dyv[8], xv[8], a1[8], a0[8];
    load8_f32(dy, row * P + p, dy_bf16 != 0, dyv);
    load8_f32(x, row * P + p, in_bf16 != 0, xv);
    load8_f32(y1, rrow * P + p, y_bf16 != 0, a1);
    load8_f32(y0, row * P + p, y_bf16 != 0, a0);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = fmaf(dtv, a1[e], dh * dyv[e]);
      sv = fmaf(dyv[e], a0[e], sv);
      su = fmaf(dyv[e], xv[e], su);
      sb = fmaf(a1[e], xv[e], sb);
    }
    *reinterpret_cast<float4*>(dx + row * P + p) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dx + row * P + p + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
#pragma unroll
  for (int off = 4; off > 0; off >>= 1) {
    sv += __shfl_xor(sv, off, 8);
    su += __shfl_xor(su, off, 8);
    sb += __shfl_xor(sb, off, 8);
  }
  if (l8 == 0) {
    v[row] = sv;
    u[row] = su;
    beta[row] = sb;
  }
}

// Per (b, h, chunk k): q over the chunk's tokens t0 .. te from its anchor,
//   q_{t0} = r_{t0} anc_k + dt_{t0} beta_{t0},  q_t = q_{t-1} - v_{t-1} + dt_t beta_t,
// as a prefix sum.  q at the last token is also known exactly from the next
// anchor, q_te = v_te + r_{te+1} anc_{k+1} (no decay after the sequence's last
// token, where anc_nc pairs dL/dfinal with the final state); the mismatch of
// the prefix sum there is the rounding it piled up, spread back linearly over
// the chunk (each token then leans on the nearer exact end).  Then ddt and the
// chunk's shares of dA and dD.
// One block per (b, k, tile of kCgHeads heads): thread (hh, sg) takes head
// h0 + hh and the PER = Q / kCgSegs consecutive tokens of segment sg, so the
// [B,L,H] rows of dt, beta, v, u and ddt are read and written as 64-byte
// pieces of kCgHeads heads (one wave per (b, h) would touch a cache line per
// lane and token).  Each thread sums its segment, the segments' totals are
// combined in order through LDS, and the chunk sums are reduced there too.
constexpr int kCgHeads = 16, kCgSegs = 16;
template <int PER>
__global__ __launch_bounds__(256) void chunk_grad_kernel(const float* __restrict__ dt, const float* __restrict__ A,
                                                         const float* __restrict__ beta, const float* __restrict__ v,
                                                         const float* __restrict__ u, const float* __restrict__ anc,
                                                         float* __restrict__ ddt, float* __restrict__ dA_part,
                                                         float* __restrict__ dD_part, int L, int H, int nc, int nht) {
  static_assert(kCgHeads * kCgSegs == 256, "one thread per (head, segment)");
  constexpr int Q = PER * kCgSegs;
  __shared__ float seg_tot[kCgSegs][kCgHeads];
  __shared__ float red_a[kCgSegs][kCgHeads], red_d[kCgSegs][kCgHeads];
  const int tid = threadIdx.x, hh = tid % kCgHeads, sg = tid / kCgHeads;
  const int ht = blockIdx.x % nht;
  const int k = (blockIdx.x / nht) % nc;
  const int64_t b = blockIdx.x / nht / nc;
  const int h = ht * kCgHeads + hh;
  const bool hv = h < H;
  const int hc = hv ? h : H - 1;  // a valid head for the address math of the idle threads
  const float a = A[hc];
  const int t0 = k * Q, t1 = min(L, t0 + Q), te = t1 - 1;
  auto at = [&](int t) -> int64_t { return (b * L + t) * H + hc; };
  const int64_t bh = b * H + hc;
  const float* ak = anc + bh * (nc + 1) + k;
  // every load of the thread first
  float dtv[PER], be[PER], vp[PER], uu[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int t = t0 + sg * PER + j;
    const bool ok = hv && t < t1;
    dtv[j] = ok ? dt[at(t)] : 0.f;
    be[j] = ok ? beta[at(t)] : 0.f;
    vp[j] = ok && t > t0 ? v[at(t - 1)] : 0.f;
    uu[j] = ok ? u[at(t)] : 0.f;
  }
  const float anc0 = ak[0], anc1 = ak[1];
  const float dt_next = k + 1 < nc ? dt[at(t1)] : 0.f;
  const float v_end = v[at(te)];
  float z[PER];
  float run = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int t = t0 + sg * PER + j;
    float zj = 0.f;
    if (t < t1) zj = t == t0 ? fmaf(expf(dtv[j] * a), anc0, dtv[j] * be[j]) : dtv[j] * be[j] - vp[j];
    run += zj;
    z[j] = run;  // inclusive prefix within the segment
  }
  seg_tot[sg][hh] = run;
  __syncthreads();
  float excl = 0.f, total = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < kCgSegs; ++s2) {
    const float st = seg_tot[s2][hh];
    if (s2 < sg) excl += st;
    total += st;  // the prefix sum's q at te
  }
  const float r_next = k + 1 < nc ? expf(dt_next * a) : 1.f;
  const float q_end = fmaf(r_next, anc1, v_end);
  const float corr = q_end - total;
  const float inv_span = te > t0 ? 1.f / (float)(te - t0) : 0.f;
  float sa = 0.f, sd = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int t = t0 + sg * PER + j;
    if (hv && t < t1) {
      const float q = fmaf((float)(t - t0) * inv_span, corr, excl + z[j]);
      const float dla = q - dtv[j] * be[j];
      ddt[at(t)] = fmaf(a, dla, be[j]);
      sa = fmaf(dtv[j], dla, sa);
      sd += uu[j];
    }
  }
  red_a[sg][hh] = sa;
  red_d[sg][hh] = sd;
  __syncthreads();
  if (sg == 0 && hv) {
    float ta = 0.f, td = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < kCgSegs; ++s2) {
      ta += red_a[s2][hh];
      td += red_d[s2][hh];
    }
    const int64_t w = (b * H + h) * nc + k;
    dA_part[w] = ta;
    dD_part[w] = td;
  }
}

// dh0[b, h] = exp(dt[b, 0, h] A[h]) g_0[b, h]
__global__ __launch_bounds__(256) void dh0_kernel(const float* __restrict__ dt, const float* __restrict__ A,
                                                  const float* __restrict__ g0, float* __restrict__ dh0, int L, int H,
                                                  int64_t NP, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t bh = i / NP;
  const int h = (int)(bh % H);
  const int64_t b = bh / H;
  dh0[i] = expf(dt[b * L * H + h] * A[h]) * g0[i];
}

// dA[h] = sum_{b,k} dA_part[b, h, k];  dD[h] likewise
__global__ __launch_bounds__(256) void combine_heads_kernel(const float* __restrict__ dA_part,
                                                            const float* __restrict__ dD_part, float* __restrict__ dA,
                                                            float* __restrict__ dD, int B, int H, int nc) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float sa = 0.f, sd = 0.f;
  for (int b = 0; b < B; ++b)
    for (int k = 0; k < nc; ++k) {
      sa += dA_part[((int64_t)b * H + h) * nc + k];
      sd += dD_part[((int64_t)b * H + h) * nc + k];
    }
  dA[h] = sa;
  dD[h] = sd;
}

// ------------------------------------------------------------------ host side
namespace {
unsigned nblocks(int64_t n, int per = 256) { return (unsigned)((n + per - 1) / per); }
size_t ru(size_t v) { return (v + 255) / 256 * 256; }

// Workspace pieces, in order; operand copies are sized for fp32 (bf16 copies
// use the first half).  Forward time: L tokens; reversed: Lp = nc*Q steps.
enum BwdBuf {
  kDyRev, kBRev, kCRev, kDtRev, kOnes, kZeroD,  // reversed operands
  kY0, kDA0, kDt0, kSt0, kFin0,                 // (0)
  kDA1, kDt1, kSt1, kY1, kFin1,                 // (1)
  kU,                                           // (2)
  kAnc, kBeta, kV, kUdot, kDAp, kDDp, kNumBwd
};

struct BwdLayout {
  size_t off[kNumBwd];
  size_t total;
};

BwdLayout bwd_layout(const Dims& d) {
  const size_t f = sizeof(float), B = d.B, L = d.L, Lp = d.nc * d.Q, H = d.H, P = d.P, N = d.N, G = d.G;
  const size_t chunk_q = f * B * H * d.nc * d.Q, states = f * B * d.nc * H * N * P, bhnp = f * B * H * N * P;
  size_t sz[kNumBwd] = {};
  sz[kDyRev] = f * B * Lp * H * P;
  sz[kBRev] = sz[kCRev] = f * B * Lp * G * N;
  sz[kDtRev] = f * B * Lp * H;
  sz[kOnes] = sz[kDA0] = sz[kDt0] = sz[kDA1] = sz[kDt1] = chunk_q;
  sz[kZeroD] = f * H;
  sz[kFin0] = sz[kFin1] = bhnp;
  sz[kSt0] = sz[kSt1] = states;
  sz[kY0] = f * B * L * H * P;
  sz[kY1] = f * B * Lp * H * P;
  sz[kU] = bwd_dbc_ws_bytes(d);
  sz[kBeta] = sz[kV] = sz[kUdot] = f * B * L * H;
  sz[kDAp] = sz[kDDp] = f * B * H * d.nc;
  sz[kAnc] = f * B * H * (d.nc + 1);
  BwdLayout w;
  size_t o = 0;
  for (int i = 0; i < kNumBwd; ++i) {
    w.off[i] = o;
    o = ru(o + sz[i]);
  }
  w.total = o;
  return w;
}
}  // namespace

size_t backward_workspace_bytes(const Dims& d) { return bwd_layout(d).total; }

#define BWD_TRY(expr)                \
  do {                               \
    const hipError_t e_ = (expr);    \
    if (e_ != hipSuccess) return e_; \
  } while (0)

hipError_t launch_backward(const Dims& d, const void* x, const float* dt, const float* A, const void* Bm,
                           const void* Cm, const float* D, bool in_bf16, const float* initial_states,
                           const void* dy, bool dy_bf16, const float* dfinal, float* dx, float* ddt, float* dA,
                           float* dB, float* dC, float* dD, float* dinit, bool f32_mma, void* workspace,
                           hipStream_t s) {
  const BwdLayout w = bwd_layout(d);
  char* base = static_cast<char*>(workspace);
  auto F = [&](int k) { return reinterpret_cast<float*>(base + w.off[k]); };
  auto V = [&](int k) { return static_cast<void*>(base + w.off[k]); };
  const int L = (int)d.L, Lp = (int)(d.nc * d.Q), H = (int)d.H, P = (int)d.P, N = (int)d.N, G = (int)d.G;
  if (!bwd_dbc_supported(d)) return hipErrorInvalidValue;
  // the reversed pass: Lp steps (whole chunks)
  Dims dR = d;
  dR.L = Lp;

  // ---- operands of the reversed pass (reversed copies of dy, C and B): bf16
  // with bf16 matrix operands (rounded there anyway), and with fp32 operands
  // when x, B, C and dy all arrive as bf16 (the copies are then exact, and the
  // chunk kernels take their fp32-operand head-group instances); fp32
  // otherwise.  The forward pass reads the caller's arrays as they are.
  const bool op_bf16 = !f32_mma || (in_bf16 && dy_bf16);
  auto gather = [&](const void* src, int src_bf16, int k, int Lout, int KO, int KI, int E, int reverse) {
    if (op_bf16)
      hipLaunchKernelGGL(gather_rows_kernel<true>, dim3((unsigned)(d.B * Lout)), dim3(256), 0, s, src, src_bf16, V(k),
                         L, Lout, KO, KI, E, reverse);
    else
      hipLaunchKernelGGL(gather_rows_kernel<false>, dim3((unsigned)(d.B * Lout)), dim3(256), 0, s, src, src_bf16,
                         V(k), L, Lout, KO, KI, E, reverse);
    return static_cast<const void*>(V(k));
  };
  const int ib = in_bf16 ? 1 : 0, db = dy_bf16 ? 1 : 0;
  // With bf16 x, B, C and dy on the head-group kernels' shapes, the reversed
  // pass reads dy, C and B where they are (reversed row addressing) instead
  // of reversed copies.
  const bool rev = in_bf16 && dy_bf16 && chunk_state_hg_supported(dR, true, f32_mma) &&
                   chunk_scan_hg_supported(dR, true, f32_mma);
  const void* DyRev = rev ? dy : gather(dy, db, kDyRev, Lp, H, H, P, 1);
  const void* BRev = rev ? Bm : gather(Bm, ib, kBRev, Lp, G, G, N, 1);
  const void* CRev = rev ? Cm : gather(Cm, ib, kCRev, Lp, G, G, N, 1);
  const int64_t nblh = d.B * d.L * d.H, rblh = d.B * Lp * d.H;
  hipLaunchKernelGGL(shift_reverse_dt_kernel, dim3(nblocks(rblh)), dim3(256), 0, s, dt, F(kDtRev), L, Lp, H, rblh);
  const int64_t nq = d.B * d.H * d.nc * d.Q;
  hipLaunchKernelGGL(step_mask_kernel, dim3(nblocks(nq)), dim3(256), 0, s, F(kOnes), L, Lp, nq);
  hipLaunchKernelGGL(fill_kernel, dim3(nblocks(d.H)), dim3(256), 0, s, F(kZeroD), 0.f, (int64_t)d.H);
  BWD_TRY(hipGetLastError());

  // Intermediates (chunk and carried states, y0, y1) are fp32, and bf16
  // (rounded to nearest even) with bf16 matrix operands, which round them as
  // operands anyway; final states and the anchors' sums stay fp32.
  const bool bfi = !f32_mma;

  // ---- (0) forward: y0 = C^T h (no skip term), carried states h
  if (chunk_state_hg_supported(d, in_bf16, f32_mma)) {
    BWD_TRY(launch_chunk_state_cumsum_hg(d, x, Bm, dt, A, F(kDA0), F(kDt0), V(kSt0), bfi, f32_mma, s));
  } else {
    BWD_TRY(launch_chunk_cumsum(d, dt, A, F(kDA0), F(kDt0), s));
    BWD_TRY(launch_chunk_state_any(d, x, Bm, in_bf16, F(kDt0), F(kDA0), V(kSt0), bfi, f32_mma, s));
  }
  BWD_TRY(launch_state_passing_any(d, V(kSt0), bfi, V(kSt0), bfi, F(kDA0), initial_states, F(kFin0), s));
  BWD_TRY(launch_chunk_scan(d, x, Bm, Cm, in_bf16, F(kDt0), F(kDA0), V(kSt0), bfi, F(kZeroD), V(kY0), bfi, f32_mma,
                            s));

  // ---- (1) adjoint in reversed time: decay from the shifted dt, input scale 1
  BWD_TRY(launch_chunk_cumsum(dR, F(kDtRev), A, F(kDA1), F(kDt1), s));
  if (rev)
    BWD_TRY(launch_chunk_state_hg_rev(dR, DyRev, CRev, F(kOnes), F(kDA1), V(kSt1), bfi, f32_mma, d.L, s));
  else
    BWD_TRY(launch_chunk_state_any(dR, DyRev, CRev, op_bf16, F(kOnes), F(kDA1), V(kSt1), bfi, f32_mma, s));
  BWD_TRY(launch_state_passing_any(dR, V(kSt1), bfi, V(kSt1), bfi, F(kDA1), dfinal, F(kFin1), s));
  if (rev)
    BWD_TRY(launch_chunk_scan_hg_rev(dR, DyRev, CRev, BRev, F(kOnes), F(kDA1), V(kSt1), bfi, F(kZeroD), V(kY1), f32_mma,
                                     d.L, s));
  else
    BWD_TRY(launch_chunk_scan(dR, DyRev, CRev, BRev, op_bf16, F(kOnes), F(kDA1), V(kSt1), bfi, F(kZeroD), V(kY1),
                              bfi, f32_mma, s));

  // ---- (2) dB and dC per (chunk, group)
  BWD_TRY(launch_bwd_dbc(d, x, in_bf16, dy, dy_bf16, Bm, Cm, in_bf16, F(kDA0), F(kDt0), V(kSt0), V(kSt1), bfi, A,
                         F(kU), dB, dC, f32_mma, s));

  // ---- combine
  hipLaunchKernelGGL(anchor_dot_kernel, dim3((unsigned)(d.B * (d.nc + 1) * d.H)), dim3(256), 0, s, V(kSt0), F(kFin0),
                     V(kSt1), F(kFin1), initial_states, dfinal, F(kAnc), H, (int)d.nc, d.N * d.P, bfi ? 1 : 0);
  hipLaunchKernelGGL(combine_token_kernel, dim3(nblocks(nblh, 32)), dim3(256), 0, s, dy, db, x, ib, dt, D, V(kY0),
                     V(kY1), bfi ? 1 : 0, dx, F(kBeta), F(kV), F(kUdot), L, Lp, H, P, nblh);
  {
    const int nht = (int)((H + kCgHeads - 1) / kCgHeads);
    auto cg = d.Q == 256 ? chunk_grad_kernel<16> : d.Q == 128 ? chunk_grad_kernel<8>
              : d.Q == 64 ? chunk_grad_kernel<4> : chunk_grad_kernel<2>;
    hipLaunchKernelGGL(cg, dim3((unsigned)(d.B * d.nc * nht)), dim3(256), 0, s, dt, A, F(kBeta), F(kV), F(kUdot),
                       F(kAnc), ddt, F(kDAp), F(kDDp), L, H, (int)d.nc, nht);
  }
  const int64_t nnp = d.B * d.H * d.N * d.P;
  if (dinit)
    hipLaunchKernelGGL(dh0_kernel, dim3(nblocks(nnp)), dim3(256), 0, s, dt, A, F(kFin1), dinit, L, H, d.N * d.P,
                       nnp);
  hipLaunchKernelGGL(combine_heads_kernel, dim3(nblocks(d.H)), dim3(256), 0, s, F(kDAp), F(kDDp), dA, dD, (int)d.B,
                     H, (int)d.nc);
  return hipGetLastError();
}

}  // namespace ssd
