// chunk_state_hg.hip -- per-chunk states, head-group variant (bf16 operands).
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), jump-formula paragraph: the
// state advance over a chunk is one matrix product of the stacked b and x
// rows, and pre-multiplying rows by exponentials of the log-space sums keeps
// it one.  For chunk c of (b, h):
//     S[n][p] = sum_j B[j][n] * w_j * x[j][p],   w_j = exp(G_{Q-1} - G_j) dt_j
// The weight is folded into the x rows, so the B tile is the raw input shared
// by every head of a group.
//
// One block owns a (b, c, group, 64-column slice of P) and a run of HG heads of
// that group.  Both operands stay in LDS in their natural row-major layout,
// Bn[j][n] and Xn[j][p] (token-major), and the MFMA fragments, which need the
// token as the contraction index, are read with the transposing LDS read.
// The chunk's B rows are staged ONCE (plain 16-byte copies) for all heads.
// Per head, each thread prefetches 16-byte pieces of x rows (8 consecutive
// threads cover one 128-byte row slice, so every load is fully coalesced) and
// the G and dt of those rows into registers while the previous head
// computes; at commit the pieces are scaled by w_j in fp32, rounded to bf16
// and written back as 16-byte rows.  The output is accumulated transposed,
// D[p][n] = sum_j x[j][p] B[j][n] (A operand: x, B operand: B), so that each
// lane holds four consecutive p of one state row n and writes them as one
// 16-byte store.
// F32M (fp32 matrix operands, bf16 inputs): x stays in LDS as its exact
// bf16 values and the weight w_j goes to a per-head table; each transposed x
// fragment is widened to fp32 and multiplied by the weights of its 8 tokens
// in fp32, the B fragments (exact bf16) are widened, and eight fp32 16x16x4
// products consume each 32-token step.  No operand is rounded below fp32.
// 8 waves (two per SIMD) in a 4 x 2 grid: wave w owns the state rows of
// tiles NTW (w % 4) .. +NTW-1 (NTW = N / 64) and the column tiles 2 (w / 4),
// +1 of the slice; the B fragments of its rows stay in registers for all the
// block's heads, so per head a wave reads only its half of the x tile.
#include <type_traits>

#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kShgThreads = 512;

template <int Q, int N>
struct ShgCfg {
  static constexpr int T = kShgThreads;
  static constexpr int PT = 64;
  // Row pitches (elements) of Bn and Xn: an odd multiple of 8 dwords modulo
  // 64, so the transposing reads (per half wave: 8 consecutive rows x 32
  // bytes) fall in distinct banks.
  static constexpr int BP = N + 16;
  static constexpr int XP = PT + 16;
  // wave grid: 4 waves along n (NTW 16-row tiles each) x 2 along p (two
  // 16-column tiles each)
  static constexpr int NTW = N / 16 / 4;
  static constexpr int KS = Q / 32;  // 32-token contraction steps
  static constexpr size_t lds_b = (size_t)Q * BP * 2;
  static constexpr size_t lds_x = (size_t)Q * XP * 2;
  static constexpr size_t lds_total = lds_b + lds_x;
};

// FUSE: the block also computes the log-space sums of its heads and chunk
// from dt and A (the cumulative-sum step, same arithmetic as that kernel),
// keeps them in LDS, and writes dA_cumsum / dt_bhl for the later steps;
// otherwise it reads them.
// SBF16: the states are stored rounded to bf16 (nearest even, 8-byte stores
// of four consecutive p) instead of fp32.
// bf16 fragment (8 slots) widened to fp32, slot order kept
__device__ __forceinline__ OpF32::Frag widen_frag(const OpBF16::Frag& f) {
  OpF32::Frag r;
  r.lo = make_float4(bf16_bits_to_f32(f.v.x & 0xffffu), bf16_bits_to_f32(f.v.x >> 16),
                     bf16_bits_to_f32(f.v.y & 0xffffu), bf16_bits_to_f32(f.v.y >> 16));
  r.hi = make_float4(bf16_bits_to_f32(f.v.z & 0xffffu), bf16_bits_to_f32(f.v.z >> 16),
                     bf16_bits_to_f32(f.v.w & 0xffffu), bf16_bits_to_f32(f.v.w >> 16));
  return r;
}

template <int Q, int N, bool FUSE, bool SBF16, bool F32M, bool REV = false, bool VL = false>
__global__ __launch_bounds__(kShgThreads) void chunk_state_hg_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const float* __restrict__ dt_bhl,
    const float* __restrict__ dA_cumsum, const float* __restrict__ dt_raw, const float* __restrict__ Avec,
    float* __restrict__ dA_out, float* __restrict__ dt_out, void* __restrict__ states, int L, int H, int P, int G,
    int nc, int HG, int nhg, int npt, int remap, int lin, const int* __restrict__ seq_idx,
    int* __restrict__ seq_start_out, float* __restrict__ dA_pass) {
  static_assert(!(REV && FUSE), "the reversed reading serves the non-fused instance");
  static_assert(!VL || (FUSE && !F32M), "the packed-sequence steps ride on the fused cumulative sum");
  using Cfg = ShgCfg<Q, N>;
  using Op = OpBF16;
  using Frag = Op::Frag;
  constexpr int T = Cfg::T, PT = Cfg::PT, BP = Cfg::BP, XP = Cfg::XP, NTW = Cfg::NTW, KS = Cfg::KS;
  constexpr int NXB = Q * (PT / 8);  // 16-byte pieces of a head's x slice
  constexpr int XPT = NXB / T;
  static_assert(NXB % T == 0 && PT == 64, "x pieces must divide evenly over the block");
  static_assert(BP >= XP, "the second x buffer lives in the Bn area");

  extern __shared__ __align__(16) unsigned char shg_smem[];
  uint16_t* Bn = reinterpret_cast<uint16_t*>(shg_smem);  // [Q][BP]
  uint16_t* Xn = Bn + Q * BP;                             // [Q][XP]
  float* Gsa = reinterpret_cast<float*>(Xn + Q * XP);     // [HG][Q] log-space sums (FUSE)
  float* Dsa = Gsa + HG * Q;                               // [HG][Q] dt (FUSE)
  float* Wt = Gsa + (FUSE ? 2 * HG * Q : 0);               // [2][Q] weights of the two x buffers (F32M)
  int* Sts = reinterpret_cast<int*>(Wt);                   // [Q] sequence start of each row (VL)

  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  if (remap) bid = (bid & 7u) * (nblk >> 3) + (bid >> 3);
  const int pt = bid % npt;
  unsigned rest = bid / npt;
  const int hgi = rest % nhg;
  rest /= nhg;
  const int g = rest % G;
  rest /= G;
  const int c = rest % nc;
  const int b = rest / nc;
  const int hbase = g * (H / G) + hgi * HG;
  const int p0 = pt * PT;
  const int64_t tok0 = (int64_t)b * L + (int64_t)c * Q;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int HP = H * P;
  // last token row of the chunk inside the sequence: rows past it (ragged last
  // chunk) re-read this one, and their dt = 0 zeroes their contribution
  const int rmax = min(Q, L - c * Q) - 1;
  // REV (the backward's adjoint, run over reversed time): the inputs are the
  // forward arrays of lin tokens; row r of chunk c (step cQ + r of the L = nc Q
  // steps) reads forward token L-1-(cQ+r), clamped to lin-1 (the steps past
  // the forward sequence have input scale 0).  Input rows are addressed from
  // the chunk's first token tokb by the row offset ro(r).
  const int64_t tokb = REV ? (int64_t)b * lin + (L - (c + 1) * Q) : tok0;
  const int rmaxr = REV ? lin - 1 - (L - (c + 1) * Q) : rmax;
  auto ro = [&](int r) { return REV ? min(Q - 1 - r, rmaxr) : min(r, rmax); };

  // ---- per-head register prefetch of x pieces and their G, dt
  // Piece blk -> (row, 8-column block cb): 8 consecutive threads take the 8
  // pieces of one row; within a wave the 8 rows are ordered 0,4,1,5,2,6,3,7 so
  // that the two rows written by a 16-lane group fall in different banks.
  auto xmap = [&](int blk, int& row, int& cb) {
    const int lr = (blk >> 3) & 7;
    row = 8 * (blk >> 6) + (lr >> 1) + 4 * (lr & 1);
    cb = blk & 7;
  };
  // Two prefetch sets: while head hh computes, one set holds head hh + 1 and
  // the other takes head hh + 2.  ROT (bf16 operands without FUSE: the G and
  // dt rows are loaded per head too): the head loop is unrolled by two and the
  // sets swap roles, so head hh + 2's loads stay in flight across two heads'
  // compute.  Otherwise the second set is copied into the first after each
  // head, and the copy waits for the loads just issued, leaving them one
  // head's compute to arrive; with FUSE (x only) that measured slightly
  // faster, and with fp32 operands the unrolled loop spills.
  constexpr bool ROT = !FUSE && !F32M;
  struct XSet {
    uint4 xv[XPT];
    float gv[XPT], dv[XPT];
    float glast;
    int hcur;  // FUSE: head (within the group) of the pieces
  };
  auto issue = [&](XSet& st, int h) __attribute__((always_inline)) {
    const uint16_t* xs = x + (tokb * H + h) * (int64_t)P + p0;
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      int row, cb;
      xmap(tid + u * T, row, cb);
      st.xv[u] = *reinterpret_cast<const uint4*>(xs + ro(row) * HP + 8 * cb);
    }
    if constexpr (FUSE) {
      st.hcur = h - hbase;
    } else {
      const int64_t bhc = ((int64_t)b * H + h) * nc + c;
      const float* gsrc = dA_cumsum + bhc * Q;
      const float* dsrc = dt_bhl + bhc * Q;
#pragma unroll
      for (int u = 0; u < XPT; ++u) {
        int row, cb;
        xmap(tid + u * T, row, cb);
        st.gv[u] = gsrc[row];
        st.dv[u] = dsrc[row];
      }
      st.glast = gsrc[Q - 1];
    }
  };
  auto copy_set = [&](XSet& dst, const XSet& src) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      const uint4 q = src.xv[u];
      dst.xv[u] = make_uint4(q.x, q.y, q.z, q.w);
      if constexpr (!FUSE) {
        dst.gv[u] = src.gv[u];
        dst.dv[u] = src.dv[u];
      }
    }
    if constexpr (FUSE) dst.hcur = src.hcur;
    else dst.glast = src.glast;
  };
  // VL: in-chunk start of the sequence holding the chunk's last token (-1:
  // it runs in from an earlier chunk); rows before it do not reach the state
  // the chunk hands on
  int st_last = -1;
  auto commit = [&](XSet& st, uint16_t* dst, float* wdst) __attribute__((always_inline)) {
    float glast;
    if constexpr (FUSE) glast = Gsa[st.hcur * Q + Q - 1];
    else glast = st.glast;
#pragma unroll
    for (int u = 0; u < XPT; ++u) {
      int row, cb;
      xmap(tid + u * T, row, cb);
      float gu, du;
      if constexpr (FUSE) {
        gu = Gsa[st.hcur * Q + row];
        du = Dsa[st.hcur * Q + row];
        if constexpr (VL) du = row >= st_last ? du : 0.f;
      } else {
        gu = st.gv[u];
        du = st.dv[u];
      }
      const float w = fast_exp(glast - gu) * du;
      const uint4 q = st.xv[u];
      if constexpr (F32M) {
        // raw x (exact bf16) and the row's weight, applied in fp32 at use
        *reinterpret_cast<uint4*>(dst + row * XP + 8 * cb) = make_uint4(q.x, q.y, q.z, q.w);
        if (cb == 0) wdst[row] = w;
        continue;
      }
      uint4 o;
      o.x = pack_bf16x2(bf16_bits_to_f32(q.x & 0xffffu) * w, bf16_bits_to_f32(q.x >> 16) * w);
      o.y = pack_bf16x2(bf16_bits_to_f32(q.y & 0xffffu) * w, bf16_bits_to_f32(q.y >> 16) * w);
      o.z = pack_bf16x2(bf16_bits_to_f32(q.z & 0xffffu) * w, bf16_bits_to_f32(q.z >> 16) * w);
      o.w = pack_bf16x2(bf16_bits_to_f32(q.w & 0xffffu) * w, bf16_bits_to_f32(q.w >> 16) * w);
      *reinterpret_cast<uint4*>(dst + row * XP + 8 * cb) = o;
    }
  };

  // ---- B chunk -> Bn[j][n] (16-byte copies; a row's pieces go to
  // consecutive threads) and, with FUSE, the dt rows of the block's heads:
  // every load of the thread is issued before the first store (a store waits
  // for its load, and loads complete in order, so interleaving them would
  // serialize their latencies), then the first two heads' x pieces, which stay
  // in flight across the staging and the cumulative sums
  constexpr int NBQ = (Q * (N / 8) + T - 1) / T;
  uint4 bq[NBQ];
  const uint16_t* bsrc = Bm + (tokb * G + g) * N;
#pragma unroll
  for (int u = 0; u < NBQ; ++u) {
    const int blk = tid + u * T;
    if (blk < Q * (N / 8)) {
      const int j = blk / (N / 8), cb = blk % (N / 8);
      bq[u] = *reinterpret_cast<const uint4*>(bsrc + ro(j) * (G * N) + 8 * cb);
    }
  }
  // FUSE: 16-byte dt loads (4 heads of one token) where the head range allows
  // them; at most Q * MAXHQ / T per thread, MAXHQ bounding HG / 4 by the LDS
  constexpr int MAXHQ = (int)((160 * 1024 - Cfg::lds_total) / (8 * Q) / 4) + 1;
  constexpr int NDQ = FUSE ? (Q * MAXHQ + T - 1) / T : 1;
  float4 dq[NDQ];
  const bool dt16 = FUSE && (HG & 3) == 0 && (H & 3) == 0 && (hbase & 3) == 0;
  const int hq = HG / 4;
  if constexpr (FUSE) {
    if (dt16) {
#pragma unroll
      for (int u = 0; u < NDQ; ++u) {
        const int idx = tid + u * T;
        if (idx < Q * hq) {
          const int i = idx / hq, q4 = idx - i * hq;
          dq[u] = i <= rmax ? *reinterpret_cast<const float4*>(dt_raw + (tok0 + i) * H + hbase + 4 * q4)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
  }
  XSet sa, sb;
  issue(sa, hbase);
  issue(sb, HG > 1 ? hbase + 1 : hbase);
#pragma unroll
  for (int u = 0; u < NBQ; ++u) {
    const int blk = tid + u * T;
    if (blk < Q * (N / 8)) {
      const int j = blk / (N / 8), cb = blk % (N / 8);
      const uint4 q = bq[u];
      *reinterpret_cast<uint4*>(Bn + j * BP + 8 * cb) = make_uint4(q.x, q.y, q.z, q.w);
    }
  }

  if constexpr (FUSE) {
    // ---- cumulative-sum step for the block's heads: dt rows -> LDS, one wave
    // per head scans the chunk (chunk_cumsum_lane), pt == 0 blocks write the
    // sums and dt rows for the state passing and the chunk scan
    if (dt16) {
#pragma unroll
      for (int u = 0; u < NDQ; ++u) {
        const int idx = tid + u * T;
        if (idx < Q * hq) {
          const int i = idx / hq, q4 = idx - i * hq;
          const float4 v = dq[u];
          Dsa[(4 * q4 + 0) * Q + i] = v.x;
          Dsa[(4 * q4 + 1) * Q + i] = v.y;
          Dsa[(4 * q4 + 2) * Q + i] = v.z;
          Dsa[(4 * q4 + 3) * Q + i] = v.w;
        }
      }
    } else {
      for (int idx = tid; idx < Q * HG; idx += T) {
        const int i = idx / HG, hh = idx - i * HG;
        Dsa[hh * Q + i] = i <= rmax ? dt_raw[(tok0 + i) * H + hbase + hh] : 0.f;
      }
    }
    if constexpr (VL) {
      // packed sequences: wave 0 finds, for every row i, the in-chunk start of
      // its sequence (the last position <= i where seq_idx changes from the
      // token before, -1 if none): a per-lane run over E rows, then a
      // log-depth max-scan across the lanes; rows past the sequence end repeat
      // the last valid row's value
      if (wave == 0) {
        constexpr int E = Q / 64;
        const int lane = tid & 63;
        const int* sq = seq_idx + tok0;
        int run = -1, loc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = lane * E + e;
          if (i <= rmax && c * Q + i > 0 && sq[i] != sq[i - 1]) run = i;
          loc[e] = run;
        }
        int tot = run;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(tot, off, 64);
          if (lane >= off) tot = max(tot, o);
        }
        int excl = __shfl_up(tot, 1, 64);
        if (lane == 0) excl = -1;
#pragma unroll
        for (int e = 0; e < E; ++e) Sts[lane * E + e] = max(excl, loc[e]);
      }
    }
    __syncthreads();
    constexpr int E = Q / 64;
    const int lane = tid & 63;
    for (int hh = wave; hh < HG; hh += T / 64) {
      float d4[4], g4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) d4[e] = e < E ? Dsa[hh * Q + E * lane + e] : 0.f;
      chunk_cumsum_lane(d4, E, Avec[hbase + hh], lane, g4);
#pragma unroll
      for (int e = 0; e < E; ++e) Gsa[hh * Q + E * lane + e] = g4[e];
    }
    __syncthreads();
    if (pt == 0) {
      // rows of Q floats per head, written as 16-byte pieces
      for (int idx = tid; idx < HG * (Q / 4); idx += T) {
        const int hh = idx / (Q / 4), i4 = idx - hh * (Q / 4);
        const int64_t o = (((int64_t)b * H + hbase + hh) * nc + c) * Q + 4 * i4;
        *reinterpret_cast<float4*>(dA_out + o) = *reinterpret_cast<const float4*>(Gsa + hh * Q + 4 * i4);
        *reinterpret_cast<float4*>(dt_out + o) = *reinterpret_cast<const float4*>(Dsa + hh * Q + 4 * i4);
      }
    }
    if constexpr (VL) {
      st_last = __builtin_amdgcn_readfirstlane(Sts[Q - 1]);
      if (pt == 0) {
        // the state passing reads one decay per chunk, at position Q-1: -inf
        // where the chunk's last sequence starts inside it (the incoming state
        // then decays to exactly 0); no other entry of dA_pass is written
        for (int hh = tid; hh < HG; hh += T) {
          const int64_t o = (((int64_t)b * H + hbase + hh) * nc + c) * Q + Q - 1;
          dA_pass[o] = st_last >= 0 ? -INFINITY : Gsa[hh * Q + Q - 1];
        }
        // one block per (b, c) hands the row starts on to the chunk scan
        if (hgi == 0 && g == 0)
          for (int i = tid; i < Q; i += T) seq_start_out[((int64_t)b * nc + c) * Q + i] = Sts[i];
      }
    }
  }

  __syncthreads();  // Bn complete
  // The B rows are the same for every head of the block: each wave keeps the
  // fragments of its state rows in registers for the whole head loop, so per
  // head only the x tile is read from LDS (a quarter of it per wave pair of
  // columns instead of all of it per wave).
  const int wn = wave & 3, wp = wave >> 2;
  Frag bfr[NTW][KS];
#pragma unroll
  for (int i = 0; i < NTW; ++i)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) bfr[i][kk] = lds_frag_tr(Bn + 32 * kk * BP + 16 * (NTW * wn + i), BP, tid & 63);
  commit(sa, Xn, Wt);
  if constexpr (!ROT) copy_set(sa, sb);
  __syncthreads();  // every wave holds its B fragments: the Bn area is free from here on

  // x tiles double-buffered: head hh computes from one buffer while head
  // hh + 1 is committed to the other (the first lies in the Bn area), so a
  // head needs one barrier
  auto step = [&](const int hh, XSet& sfree, XSet& snext, auto copy_back) __attribute__((always_inline)) {
    const int h = hbase + hh;
    uint16_t* const xcur = (hh & 1) ? Bn : Xn;
    uint16_t* const xnext = (hh & 1) ? Xn : Bn;
    const float* const wcur = Wt + (hh & 1) * Q;
    float* const wnext = Wt + ((hh + 1) & 1) * Q;
    // The prefetch and the commit run on every iteration (the last one loads
    // its own head again, unused): with no conditional around them the
    // compiler's memory-counter waits stay exact, so the loads of the next
    // head remain in flight across the whole compute of this one.
    issue(sfree, hh + 2 < HG ? h + 2 : hbase + HG - 1);
    {
      // lane index laundered per head: lane-dependent addresses are recomputed
      // here rather than hoisted out of the head loop
      int ln = tid & 63;
      asm volatile("" : "+v"(ln));
      const int l16 = ln & 15, lg = ln >> 4;
      f32x4_t acc[NTW][2];
#pragma unroll
      for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[i][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        Frag xf[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) xf[ct] = lds_frag_tr(xcur + 32 * kk * XP + 16 * (2 * wp + ct), XP, ln);
        if constexpr (F32M) {
          // weights of the lane's tokens j = 32kk + 16t + 4lg + r (slot 4t + r)
          const float4 w0 = *reinterpret_cast<const float4*>(wcur + 32 * kk + 4 * lg);
          const float4 w1 = *reinterpret_cast<const float4*>(wcur + 32 * kk + 16 + 4 * lg);
          OpF32::Frag xw[2];
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            xw[ct] = widen_frag(xf[ct]);
            xw[ct].lo.x *= w0.x; xw[ct].lo.y *= w0.y; xw[ct].lo.z *= w0.z; xw[ct].lo.w *= w0.w;
            xw[ct].hi.x *= w1.x; xw[ct].hi.y *= w1.y; xw[ct].hi.z *= w1.z; xw[ct].hi.w *= w1.w;
          }
#pragma unroll
          for (int i = 0; i < NTW; ++i) {
            const OpF32::Frag bw = widen_frag(bfr[i][kk]);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc[i][ct] = OpF32::mma(xw[ct], bw, acc[i][ct]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < NTW; ++i)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) acc[i][ct] = Op::mma(xf[ct], bfr[i][kk], acc[i][ct]);
        }
      }
      // lane holds S[n = 16*(NTW*wn + i) + l16][p = p0 + 16(2wp + ct) + 4lg .. +3]
      const int64_t so = (((int64_t)b * nc + c) * H + h) * (int64_t)(N * P) + p0;
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int n = 16 * (NTW * wn + i) + l16;
        if constexpr (SBF16) {
          // the wave's two column tiles paired across lane rows: 8
          // consecutive columns (one 16-byte store) per lane
          const uint2 t0 = make_uint2(pack_bf16x2(acc[i][0][0], acc[i][0][1]), pack_bf16x2(acc[i][0][2], acc[i][0][3]));
          const uint2 t1 = make_uint2(pack_bf16x2(acc[i][1][0], acc[i][1][1]), pack_bf16x2(acc[i][1][2], acc[i][1][3]));
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(states) + so + n * P + 32 * wp + pair_tiles_col(lg)) =
              pair_tiles_16b(t0, t1);
        } else {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const int pc = 16 * (2 * wp + ct) + 4 * lg;
            *reinterpret_cast<float4*>(static_cast<float*>(states) + so + n * P + pc) =
                make_float4(acc[i][ct][0], acc[i][ct][1], acc[i][ct][2], acc[i][ct][3]);
          }
        }
      }
    }
    // the other buffer was last read by the previous head, which every wave
    // finished before the previous barrier
    commit(snext, xnext, wnext);
    if constexpr (decltype(copy_back)::value) copy_set(snext, sfree);  // the set just issued becomes the next one
    __syncthreads();
  };
  if constexpr (!ROT) {
    for (int hh = 0; hh < HG; ++hh) step(hh, sb, sa, std::true_type{});
  } else {
    int hh = 0;
    for (; hh + 1 < HG; hh += 2) {
      step(hh, sa, sb, std::false_type{});
      step(hh + 1, sb, sa, std::false_type{});
    }
    if (hh < HG) step(hh, sa, sb, std::false_type{});
  }
}

// ------------------------------------------------------------------ host side

// (chunk, N) pairs with an instance: N >= 128 (a 16-row state tile per wave
// and per 128 rows of N) and the B and x tiles within the LDS
#define SHG_SHAPES(X) X(64, 128) X(128, 128) X(256, 128) X(64, 256) X(128, 256)

bool chunk_state_hg_supported(const Dims& d, bool in_bf16, bool f32_mma) {
  // bf16 inputs only (the fp32-operand instance widens exact bf16 values);
  // room for one head's sums and dt rows, and (fp32 operands) the two
  // weight tables
  if (!in_bf16 || d.P % 64 != 0) return false;
  const size_t extra = 8 * (size_t)d.Q * (f32_mma ? 2 : 1);
#define SHG_MATCH(QQ, NN) if (d.Q == QQ && d.N == NN) return ShgCfg<QQ, NN>::lds_total + extra <= 160 * 1024;
  SHG_SHAPES(SHG_MATCH)
#undef SHG_MATCH
  return false;
}

bool chunk_state_hg_varlen_supported(const Dims& d) {
  // the fused instance plus one row of Q sequence starts
  if (d.P % 64 != 0) return false;
#define SHG_MATCH(QQ, NN) \
  if (d.Q == QQ && d.N == NN) return ShgCfg<QQ, NN>::lds_total + 12 * (size_t)d.Q <= 160 * 1024;
  SHG_SHAPES(SHG_MATCH)
#undef SHG_MATCH
  return false;
}

template <int Q, int N, bool FUSE, bool SBF16, bool F32M, bool REV = false, bool VL = false>
static hipError_t launch_shg_inst(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                                  const float* dA_cumsum, const float* dt_raw, const float* A, float* dA_out,
                                  float* dt_out, void* states, hipStream_t stream, int lin = 0,
                                  const int* seq_idx = nullptr, int* seq_start = nullptr,
                                  float* dA_pass = nullptr) {
  using Cfg = ShgCfg<Q, N>;
  auto kern = chunk_state_hg_kernel<Q, N, FUSE, SBF16, F32M, REV, VL>;
  // with FUSE the block also holds the sums and dt rows of its heads in LDS;
  // with F32M the two weight tables, with VL the row of sequence starts
  const size_t wts = F32M ? (size_t)8 * Q : (VL ? (size_t)4 * Q : 0);
  const int64_t cap = FUSE ? (int64_t)((160 * 1024 - Cfg::lds_total - wts) / (8 * Q)) : (int64_t)1 << 30;
  const int npt = (int)(d.P / Cfg::PT);
  const int64_t hpg = d.H / d.G;
  const int64_t base = d.B * d.nc * d.G * npt;
  int HG = 1;
  for (int64_t k = 1; k <= hpg; ++k) {
    if (hpg % k || hpg / k > cap) continue;
    HG = (int)(hpg / k);
    if (base * k >= device_cu_count()) break;
  }
  const int tuned = tuning_for(d, F32M).state_hg;
  if (tuned > 0 && hpg % tuned == 0 && tuned <= cap) HG = tuned;
  // the kernel's prologue preloads the dt rows of at most 4 (MAXHQ - 1) heads
  // (HG <= cap keeps within that)
  if (FUSE && HG / 4 >= (int)((160 * 1024 - Cfg::lds_total) / (8 * Q) / 4) + 1) return hipErrorInvalidValue;
  const size_t lds = Cfg::lds_total + (FUSE ? (size_t)8 * Q * HG : 0) + wts;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int nhg = (int)(hpg / HG);
  const int64_t nblk = base * nhg;
  const int remap = (nblk % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(Cfg::T), lds, stream, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(Bm), dt_bhl, dA_cumsum, dt_raw, A, dA_out, dt_out, states,
                     (int)d.L, (int)d.H, (int)d.P, (int)d.G, (int)d.nc, HG, nhg, npt, remap, lin, seq_idx,
                     seq_start, dA_pass);
  return hipGetLastError();
}

template <int Q, int N, bool FUSE>
static hipError_t launch_shg_any(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                                 const float* dA_cumsum, const float* dt_raw, const float* A, float* dA_out,
                                 float* dt_out, void* states, bool states_bf16, bool f32_mma, hipStream_t stream) {
  if (f32_mma)
    return states_bf16 ? launch_shg_inst<Q, N, FUSE, true, true>(d, x, Bm, dt_bhl, dA_cumsum, dt_raw, A, dA_out,
                                                                  dt_out, states, stream)
                       : launch_shg_inst<Q, N, FUSE, false, true>(d, x, Bm, dt_bhl, dA_cumsum, dt_raw, A, dA_out,
                                                                   dt_out, states, stream);
  return states_bf16 ? launch_shg_inst<Q, N, FUSE, true, false>(d, x, Bm, dt_bhl, dA_cumsum, dt_raw, A, dA_out,
                                                                 dt_out, states, stream)
                     : launch_shg_inst<Q, N, FUSE, false, false>(d, x, Bm, dt_bhl, dA_cumsum, dt_raw, A, dA_out,
                                                                  dt_out, states, stream);
}

hipError_t launch_chunk_state_hg(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                                 const float* dA_cumsum, void* states, bool states_bf16, bool f32_mma,
                                 hipStream_t stream) {
#define SHG_LAUNCH(QQ, NN)                                                                                  \
  if (d.Q == QQ && d.N == NN)                                                                               \
    return launch_shg_any<QQ, NN, false>(d, x, Bm, dt_bhl, dA_cumsum, nullptr, nullptr, nullptr, nullptr,     \
                                         states, states_bf16, f32_mma, stream);
  SHG_SHAPES(SHG_LAUNCH)
#undef SHG_LAUNCH
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_state_cumsum_hg(const Dims& d, const void* x, const void* Bm, const float* dt,
                                        const float* A, float* dA_cumsum, float* dt_bhl, void* states,
                                        bool states_bf16, bool f32_mma, hipStream_t stream) {
#define SHG_LAUNCH(QQ, NN)                                                                            \
  if (d.Q == QQ && d.N == NN)                                                                         \
    return launch_shg_any<QQ, NN, true>(d, x, Bm, nullptr, nullptr, dt, A, dA_cumsum, dt_bhl, states, \
                                        states_bf16, f32_mma, stream);
  SHG_SHAPES(SHG_LAUNCH)
#undef SHG_LAUNCH
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_state_cumsum_hg_varlen(const Dims& d, const void* x, const void* Bm, const float* dt,
                                               const float* A, const int* seq_idx, float* dA_cumsum, float* dt_bhl,
                                               int* seq_start, float* dA_pass, void* states, hipStream_t stream) {
#define SHG_LAUNCH(QQ, NN)                                                                                  \
  if (d.Q == QQ && d.N == NN)                                                                               \
    return launch_shg_inst<QQ, NN, true, true, false, false, true>(d, x, Bm, nullptr, nullptr, dt, A, dA_cumsum, \
                                                                   dt_bhl, states, stream, 0, seq_idx,       \
                                                                   seq_start, dA_pass);
  SHG_SHAPES(SHG_LAUNCH)
#undef SHG_LAUNCH
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_state_hg_rev(const Dims& d, const void* x, const void* Bm, const float* dt_bhl,
                                     const float* dA_cumsum, void* states, bool states_bf16, bool f32_mma,
                                     int64_t lin, hipStream_t stream) {
  // the backward's two precision modes: bf16 states with bf16 operands, fp32
  // with fp32
  if (states_bf16 == f32_mma || lin <= d.L - d.Q || lin > d.L) return hipErrorInvalidValue;
#define SHG_LAUNCH(QQ, NN)                                                                                    \
  if (d.Q == QQ && d.N == NN)                                                                                 \
    return f32_mma ? launch_shg_inst<QQ, NN, false, false, true, true>(d, x, Bm, dt_bhl, dA_cumsum, nullptr,  \
                                                                       nullptr, nullptr, nullptr, states,     \
                                                                       stream, (int)lin)                      \
                   : launch_shg_inst<QQ, NN, false, true, false, true>(d, x, Bm, dt_bhl, dA_cumsum, nullptr,  \
                                                                       nullptr, nullptr, nullptr, states,     \
                                                                       stream, (int)lin);
  SHG_SHAPES(SHG_LAUNCH)
#undef SHG_LAUNCH
  return hipErrorInvalidValue;
}

}  // namespace ssd
