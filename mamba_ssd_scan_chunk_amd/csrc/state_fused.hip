// state_fused.hip -- chunk states and the inter-chunk state advance in one
// pass (the fused state path): the chunk states never reach memory.
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), paragraph on the three kernels
// (the state pass walks the chunks in order, one matrix product per chunk,
// the running state kept on chip) and the jump-formula paragraph (each
// chunk's state is one product of the stacked, exponentially pre-multiplied
// b and x rows).  Per (b, h), with G = dA_cumsum[b,h,c,:], dt = dt_bhl[b,h,c,:]:
//     H_0 = initial state (or 0)
//     for c = 0..nc-1:
//         carried[b,c,h] = H_c
//         S_c     = sum_j exp(G_{Q-1} - G_j) dt_j B_j x_j^T          (N x P)
//         H_{c+1} = exp(G_{Q-1}) H_c + S_c
//     final[b,h] = H_nc
//
// Block = (b, HF heads of one group, NB state rows n, 64 columns p).  NB =
// 128 where N allows it and the chunk has at most 128 tokens (each chunk's x
// rows are then staged by half as many blocks), else 64; with NB = 128 and an
// even number of heads per group, HF = 2 heads share each chunk's staged B
// rows (16 waves), else HF = 1 (8 waves).  The waves form a WN x 2 grid
// (WN = waves / 2): wave w owns the RT = NB / 16 / WN row tiles
// 16 RT (w % WN) .. +16 RT - 1 of the block's n range and the columns
// 32 (w / WN) .. +31, for each of the HF heads; the running state of those
// elements lives in registers in the MFMA accumulator layout (lane: row l16,
// columns 16ct + 4lg .. +3).  Per
// chunk the x rows (scaled by w_j = exp(G_{Q-1} - G_j) dt_j, rounded to bf16)
// and the raw B rows are staged in LDS in their natural token-major layouts,
// and the MFMA fragments (token = contraction index) come from the transposing
// LDS read, as in the head-group chunk-state kernel.  The state recurrence
// makes the chunks of one block strictly sequential, so the block hides the
// memory latency itself: the x rows of the next two chunks (and the B rows of
// the next one) are in flight in registers while the current chunk is staged
// and multiplied, and two blocks share a compute unit.  S_c is accumulated from the same operands in the same
// order as the head-group chunk-state kernel, and the update is the same fused
// multiply-add as the state-passing kernel, so carried and final states are
// bit-identical to the two-call path.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

template <int Q, int WAVES, int NB_ = 64, int HF_ = 1>
struct SfCfg {
  static constexpr int HF = HF_;  // heads of one group per block (sharing the B rows)
  static constexpr int T = 64 * WAVES;
  static constexpr int NB = NB_, PT = 64;  // state rows (64 or 128) and columns of a block
  static constexpr int NBP = NB / 64;      // 16-byte B pieces per row and loader thread
  // wave grid: WN waves along n (RT 16-row tiles each) x 2 along p (two
  // 16-column tiles each)
  static constexpr int WN = WAVES / 2, RT = NB / 16 / WN;
  // row pitches (elements) of Xn and Bn: odd multiples of 8 dwords modulo 64,
  // so the transposing reads (8 consecutive rows x 32 bytes per half wave)
  // fall in distinct banks
  static constexpr int XP = PT + 16, BP = NB + 16;
  // 8 threads cover a row's 128-byte slice; LT threads load, RPT rows each
  static constexpr int LT = Q * 8 < T ? Q * 8 : T;
  static constexpr int RPT = Q * 8 / LT;
  static constexpr size_t lds_total = (size_t)HF * Q * XP * 2 + (size_t)Q * BP * 2;
};

template <int Q, int WAVES, bool CBF16, int NB_, int HF>
__global__ __launch_bounds__(64 * WAVES, WAVES >= 8 ? 4 : WAVES / 2) void state_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const float* __restrict__ dt_bhl,
    const float* __restrict__ dA_cumsum, const float* __restrict__ init, void* __restrict__ carried,
    float* __restrict__ fin, int L, int H, int P, int N, int G, int nc, int nnb, int npt, int remap) {
  using Cfg = SfCfg<Q, WAVES, NB_, HF>;
  using Op = OpBF16;
  using Frag = Op::Frag;
  constexpr int XP = Cfg::XP, BP = Cfg::BP, RPT = Cfg::RPT, LT = Cfg::LT, NB = Cfg::NB, PT = Cfg::PT;
  constexpr int WN = Cfg::WN, RT = Cfg::RT, NBP = Cfg::NBP;
  static_assert(Q % 32 == 0 && RPT >= 1, "chunk must be a multiple of 32");

  extern __shared__ __align__(16) unsigned char sf_smem[];
  uint16_t* Xn = reinterpret_cast<uint16_t*>(sf_smem);  // [HF][Q][XP]  w-scaled x rows of the chunk
  uint16_t* Bn = Xn + HF * Q * XP;                       // [Q][BP]  B rows of the chunk (the block's n)

  // block -> (b, h, p slice, n block); with remap the n blocks of one (b, h)
  // (same x rows) land on one XCD and share its L2
  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  if (remap) bid = (bid & 7u) * (nblk >> 3) + (bid >> 3);
  const int nb = bid % nnb;
  unsigned rest = bid / nnb;
  const int pt = rest % npt;
  rest /= npt;
  const int h = (rest % (H / HF)) * HF;  // the block's first head
  const int b = rest / (H / HF);
  const int g = h / (H / G);
  const int n0 = nb * NB, p0 = pt * PT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wn = wave % WN, wp = wave / WN;
  const int l16 = lane & 15, lg = lane >> 4;
  const int HP = H * P, GN = G * N;
  const int64_t bh = (int64_t)b * H + h;
  const int64_t NP = (int64_t)N * P;

  // ---- running state H[n = n0 + 16 (RT wn + rt) + l16][p = p0 + 32 wp + 16 ct + 4 lg .. +3]
  const int64_t soff = (int64_t)(n0 + 16 * RT * wn + l16) * P + p0 + 32 * wp + 4 * lg;  // within one state
  float4 hs[HF][RT][2];
#pragma unroll
  for (int hf = 0; hf < HF; ++hf)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        hs[hf][rt][ct] = init ? *reinterpret_cast<const float4*>(init + (bh + hf) * NP + soff + 16 * (rt * P + ct))
                              : make_float4(0.f, 0.f, 0.f, 0.f);

  // ---- per-chunk register prefetch.  Loader thread t takes the 16-byte column
  // piece t % 8 of rows RPT (t / 8) .. + RPT - 1 of x (64 columns of head h)
  // and of B (64 state indices of group g), plus those rows' G and dt; threads
  // past LT (short chunks only) load nothing.  x runs two chunks ahead in two
  // register sets used alternately; B (shared by all heads of the group,
  // mostly L2 hits) runs one chunk ahead and is issued first, so each wait on
  // the in-order load counter covers exactly what the next staging needs.  G
  // and dt travel with x where the register budget allows (4 waves), else
  // with B.
  constexpr bool GD2 = WAVES == 4;
  const bool loader = LT == Cfg::T || tid < LT;
  const int rbase = RPT * ((loader ? tid : 0) >> 3), cbp = tid & 7;
  struct GSet {
    float gv[RPT], dv[RPT], glast;
  };
  struct XSet {
    uint4 xv[HF][RPT];
    GSet g[HF];  // used when GD2
  };
  XSet sa, sb;
  GSet g1[HF];  // used when !GD2
  uint4 bv[RPT][NBP];
  auto load_g = [&](GSet& gs, int c, int hf) __attribute__((always_inline)) {
    const float* gsrc = dA_cumsum + ((bh + hf) * nc + c) * Q;
    const float* dsrc = dt_bhl + ((bh + hf) * nc + c) * Q;
    gs.glast = gsrc[Q - 1];
    if (!loader) return;
    if constexpr (RPT % 4 == 0) {
#pragma unroll
      for (int u = 0; u < RPT; u += 4) {
        const float4 g4 = *reinterpret_cast<const float4*>(gsrc + rbase + u);
        const float4 d4 = *reinterpret_cast<const float4*>(dsrc + rbase + u);
        gs.gv[u] = g4.x; gs.gv[u + 1] = g4.y; gs.gv[u + 2] = g4.z; gs.gv[u + 3] = g4.w;
        gs.dv[u] = d4.x; gs.dv[u + 1] = d4.y; gs.dv[u + 2] = d4.z; gs.dv[u + 3] = d4.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < RPT; ++u) {
        gs.gv[u] = gsrc[rbase + u];
        gs.dv[u] = dsrc[rbase + u];
      }
    }
  };
  auto issue_x = [&](XSet& st, int c) __attribute__((always_inline)) {
    if (loader) {
      const int64_t tok0 = (int64_t)b * L + (int64_t)c * Q;
      const int rmax = min(Q, L - c * Q) - 1;  // rows past the sequence end re-read the last (dt = 0 there)
#pragma unroll
      for (int hf = 0; hf < HF; ++hf) {
        const uint16_t* xs = x + (tok0 * H + h + hf) * (int64_t)P + p0 + 8 * cbp;
#pragma unroll
        for (int u = 0; u < RPT; ++u)
          st.xv[hf][u] = *reinterpret_cast<const uint4*>(xs + min(rbase + u, rmax) * HP);
      }
    }
    if constexpr (GD2)
#pragma unroll
      for (int hf = 0; hf < HF; ++hf) load_g(st.g[hf], c, hf);
  };
  auto issue_b = [&](int c) __attribute__((always_inline)) {
    if (loader) {
      const int64_t tok0 = (int64_t)b * L + (int64_t)c * Q;
      const int rmax = min(Q, L - c * Q) - 1;
      const uint16_t* bs = Bm + (tok0 * G + g) * (int64_t)N + n0 + 8 * cbp;
#pragma unroll
      for (int u = 0; u < RPT; ++u)
#pragma unroll
        for (int q = 0; q < NBP; ++q)
          bv[u][q] = *reinterpret_cast<const uint4*>(bs + 64 * q + min(rbase + u, rmax) * GN);
    }
    if constexpr (!GD2)
#pragma unroll
      for (int hf = 0; hf < HF; ++hf) load_g(g1[hf], c, hf);
  };
  // stage a prefetched chunk: x rows scaled by w_j in fp32 and rounded to
  // bf16 (the same arithmetic as the head-group chunk-state kernel), B raw
  auto commit = [&](const XSet& st) __attribute__((always_inline)) {
    if (!loader) return;
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const int row = rbase + u;
#pragma unroll
      for (int hf = 0; hf < HF; ++hf) {
        const GSet& gs = GD2 ? st.g[hf] : g1[hf];
        const float w = fast_exp(gs.glast - gs.gv[u]) * gs.dv[u];
        const uint4 q = st.xv[hf][u];
        uint4 o;
        o.x = pack_bf16x2(bf16_bits_to_f32(q.x & 0xffffu) * w, bf16_bits_to_f32(q.x >> 16) * w);
        o.y = pack_bf16x2(bf16_bits_to_f32(q.y & 0xffffu) * w, bf16_bits_to_f32(q.y >> 16) * w);
        o.z = pack_bf16x2(bf16_bits_to_f32(q.z & 0xffffu) * w, bf16_bits_to_f32(q.z >> 16) * w);
        o.w = pack_bf16x2(bf16_bits_to_f32(q.w & 0xffffu) * w, bf16_bits_to_f32(q.w >> 16) * w);
        *reinterpret_cast<uint4*>(Xn + (hf * Q + row) * XP + 8 * cbp) = o;
      }
#pragma unroll
      for (int q = 0; q < NBP; ++q) {
        const uint4 bq = bv[u][q];
        *reinterpret_cast<uint4*>(Bn + row * BP + 64 * q + 8 * cbp) = make_uint4(bq.x, bq.y, bq.z, bq.w);
      }
    }
  };
  // carried[b, c, h] = H_c (the running state), rounded to bf16 or fp32.  In
  // bf16 the lane-row pairs (lg, lg ^ 1) first trade halves (pair_tiles_16b),
  // so that one 16-byte store per lane writes the wave's 16 rows x 64 bytes.
  // Ordinary stores: the chunk scan reads these rows next, and part of them
  // is still cached then (non-temporal stores made the grouped forward ~4%
  // slower).
  auto store_carried = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int hf = 0; hf < HF; ++hf) {
      const int64_t coff = ((int64_t)b * nc + c) * H + h + hf;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const float4* hr = hs[hf][rt];
        if constexpr (CBF16) {
          const uint2 t0 = make_uint2(pack_bf16x2(hr[0].x, hr[0].y), pack_bf16x2(hr[0].z, hr[0].w));
          const uint2 t1 = make_uint2(pack_bf16x2(hr[1].x, hr[1].y), pack_bf16x2(hr[1].z, hr[1].w));
          // soff holds column 4 lg; the paired row starts at 4 lg + 12 (lg & 1)
          const int64_t o = coff * NP + soff + 16 * rt * P + 12 * (lg & 1);
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(carried) + o) = pair_tiles_16b(t0, t1);
        } else {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
            *reinterpret_cast<float4*>(static_cast<float*>(carried) + coff * NP + soff + 16 * (rt * P + ct)) = hr[ct];
        }
      }
    }
  };
  // one chunk: stage it, refill B with chunk c + 1 and `st` with chunk
  // c + 2 (past the end, the last chunk again, unused: no data-dependent
  // branch around the loads keeps the memory waits exact), store carried =
  // H_c, accumulate S_c, advance H.  The memory counter retires in order, so
  // the carried stores are issued after the loads (pinned there by a
  // scheduling barrier): the next staging then waits for its own rows only,
  // not for the stores to be acknowledged.
  auto chunk = [&](XSet& st, int c) __attribute__((always_inline)) {
    __syncthreads();  // the previous chunk's fragment reads are done
    commit(st);
    float gl[HF];  // G_{Q-1} of chunk c
#pragma unroll
    for (int hf = 0; hf < HF; ++hf) gl[hf] = GD2 ? st.g[hf].glast : g1[hf].glast;
    __syncthreads();
    int ln = lane;
    asm volatile("" : "+v"(ln));
    f32x4_t acc[HF][RT][2];
#pragma unroll
    for (int hf = 0; hf < HF; ++hf)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[hf][rt][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // The refills (B of chunk c + 1 with its G and dt, x of chunk c + 2) and
    // the carried stores of chunk c are spread over the contraction steps
    // instead of queued by every wave at once after the barrier (their
    // vector-memory issue stalled the waves for about as long as the
    // matrix work).  Loads go first, so each wait on the in-order memory
    // counter at the next staging covers its own rows, not the stores.
    constexpr int KS = Q / 32;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk == 0) issue_b(c + 1 < nc ? c + 1 : nc - 1);
      if (kk == (KS > 1 ? 1 : 0)) issue_x(st, c + 2 < nc ? c + 2 : nc - 1);
      if (kk == KS - 1) {
        __builtin_amdgcn_sched_barrier(0);
        store_carried(c);
      }
      Frag bf[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) bf[rt] = lds_frag_tr(Bn + 32 * kk * BP + 16 * (RT * wn + rt), BP, ln);
#pragma unroll
      for (int hf = 0; hf < HF; ++hf) {
        Frag xf[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          xf[ct] = lds_frag_tr(Xn + (hf * Q + 32 * kk) * XP + 32 * wp + 16 * ct, XP, ln);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) acc[hf][rt][ct] = Op::mma(xf[ct], bf[rt], acc[hf][rt][ct]);
      }
    }
    // H_{c+1} = exp(G_{Q-1}) H_c + S_c
#pragma unroll
    for (int hf = 0; hf < HF; ++hf) {
      const float dec = expf(gl[hf]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          float4& hv = hs[hf][rt][ct];
          hv.x = fmaf(dec, hv.x, acc[hf][rt][ct][0]);
          hv.y = fmaf(dec, hv.y, acc[hf][rt][ct][1]);
          hv.z = fmaf(dec, hv.z, acc[hf][rt][ct][2]);
          hv.w = fmaf(dec, hv.w, acc[hf][rt][ct][3]);
        }
    }
  };

  // prologue: the same issue sequence as a chunk body (x, B, x, stores),
  // so the first staging's wait matches the steady state; chunk 0 stores H_0
  // again (the same values)
  issue_x(sa, 0);
  issue_b(0);
  issue_x(sb, nc > 1 ? 1 : 0);
  __builtin_amdgcn_sched_barrier(0);
  store_carried(0);
  int c = 0;
  for (; c + 1 < nc; c += 2) {
    chunk(sa, c);
    chunk(sb, c + 1);
  }
  if (c < nc) chunk(sa, c);
  if (fin) {
#pragma unroll
    for (int hf = 0; hf < HF; ++hf)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          *reinterpret_cast<float4*>(fin + (bh + hf) * NP + soff + 16 * (rt * P + ct)) = hs[hf][rt][ct];
  }
}

// ------------------------------------------------------------------ host side
bool state_fused_supported(const Dims& d, bool in_bf16, bool f32_mma) {
  return in_bf16 && !f32_mma && d.N % 64 == 0 && d.P % 64 == 0 &&
         (d.Q == 32 || d.Q == 64 || d.Q == 128 || d.Q == 256);
}

// State rows per block: 128 where N allows it and the chunk is at most 128
// tokens (each chunk's x rows are then staged by half as many blocks; at 256
// tokens the larger tiles would not fit the register budget), else 64.
int state_fused_rows(const Dims& d) { return (d.N % 128 == 0 && d.Q <= 128) ? 128 : 64; }

// Heads per block: with 128 state rows, two heads of a group (16 waves, each
// with one row tile per head) share the staged B rows of every chunk, which
// halves the block's B staging per head.
int state_fused_heads(const Dims& d) { return (state_fused_rows(d) == 128 && (d.H / d.G) % 2 == 0) ? 2 : 1; }

// Independent walks (head, row block, column slice): a two-head block runs two
// of them with twice the waves, so this is the parallelism the dispatch rule
// weighs whatever the heads per block.
int64_t state_fused_blocks(const Dims& d) { return d.B * d.H * (d.N / state_fused_rows(d)) * (d.P / 64); }

template <int Q, bool CBF16, int NB, int WAVES = 8, int HF = 1>
static hipError_t launch_sf_inst(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                                 const float* dA_cumsum, const float* init, void* carried, float* fin,
                                 hipStream_t stream) {
  using Cfg = SfCfg<Q, WAVES, NB, HF>;
  auto kern = state_fused_kernel<Q, WAVES, CBF16, NB, HF>;
  const size_t lds = Cfg::lds_total;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int nnb = (int)(d.N / Cfg::NB), npt = (int)(d.P / Cfg::PT);
  const int64_t nblk = d.B * (d.H / HF) * npt * nnb;
  const int remap = (nblk % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(Cfg::T), lds, stream, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(Bm), dt_bhl, dA_cumsum, init, carried, fin, (int)d.L, (int)d.H,
                     (int)d.P, (int)d.N, (int)d.G, (int)d.nc, nnb, npt, remap);
  return hipGetLastError();
}

template <bool CBF16>
static hipError_t launch_sf_q(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                              const float* dA_cumsum, const float* init, void* carried, float* fin,
                              hipStream_t stream) {
  if (state_fused_heads(d) == 2) {
    switch (d.Q) {
      case 32: return launch_sf_inst<32, CBF16, 128, 16, 2>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
      case 64: return launch_sf_inst<64, CBF16, 128, 16, 2>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
      case 128: return launch_sf_inst<128, CBF16, 128, 16, 2>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (state_fused_rows(d) == 128) {
    switch (d.Q) {
      case 32: return launch_sf_inst<32, CBF16, 128>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
      case 64: return launch_sf_inst<64, CBF16, 128>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
      case 128: return launch_sf_inst<128, CBF16, 128>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (d.Q) {
    case 32: return launch_sf_inst<32, CBF16, 64>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
    case 64: return launch_sf_inst<64, CBF16, 64>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
    case 128: return launch_sf_inst<128, CBF16, 64>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
    case 256: return launch_sf_inst<256, CBF16, 64>(d, x, Bm, dt_bhl, dA_cumsum, init, carried, fin, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_state_fused(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                              const float* dA_cumsum, const float* initial_states, void* carried, bool carried_bf16,
                              float* final_states, hipStream_t stream) {
  if (carried_bf16)
    return launch_sf_q<true>(d, x, Bm, dt_bhl, dA_cumsum, initial_states, carried, final_states, stream);
  return launch_sf_q<false>(d, x, Bm, dt_bhl, dA_cumsum, initial_states, carried, final_states, stream);
}

}  // namespace ssd
