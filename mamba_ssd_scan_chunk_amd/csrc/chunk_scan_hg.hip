// chunk_scan_hg.hip -- fused chunk output, head-group variant (bf16 operands).
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), compute_out paragraph: the
// interaction tile C.B^T is built on the matrix units (phase 1), decayed and
// causally masked in registers (phase 2), and fused with the carried-state
// term and the skip connection; the full interaction matrix never reaches
// memory.  For token i of chunk c:
//     y_i = exp(G_i) C_i^T H_in  +  sum_{j<=i} (C_i . B_j) exp(G_i - G_j) dt_j x_j  +  D x_i
//
// C.B^T depends only on (batch, chunk, B/C group), not on the head.  One block
// owns a (b, c, group) and a run of HG heads of that group: it computes the
// causal C.B^T tiles of the whole chunk ONCE, keeps them in fp32 registers,
// and reuses them for all HG heads, so the per-head work is the decay, the
// M.X product and the C.H_in product.
//
// Waves and tiles (Q = chunk in {128, 256}, QT = Q/16 row tiles of 16 rows):
//  * QT/2 waves; wave w owns the row tiles w and QT-1-w, which together hold
//    QT+1 causal 16x16 sub-tiles whatever w is (balanced work).  All waves
//    run one code path: the tile indices are wave-uniform run-time values
//    (scalar branches), while the register slot of every sub-tile is a
//    compile-time constant, so the CB^T sub-tiles stay in registers for the
//    block's life.
//  * the CB^T sub-tiles are computed with operand roles swapped (B as the A
//    operand, C as the B operand), so each lane holds four consecutive j for
//    one row i; after decay and mask those are directly the A fragment of
//    M.X (slot e = 4t + r <-> token 32k + 16t + 4lg + r), which is exactly
//    the slot map of the transposing LDS read of the x tile.
//  * decay: for the sub-tile pairs below the diagonal pair of row tile t,
//    exp(G_i - G_j) = exp(G_i - G_R) * exp(G_R - G_j) with the reference row
//    R = 32 * (t / 2) between j and i, so both factors are <= 1 (no overflow;
//    an underflowing factor means a negligible product).  The column factor
//    times dt_j comes from a per-head LDS table, the row factor scales the
//    accumulator once; only the diagonal pair takes exact per-element
//    exponentials, behind the causal select.
//  * the B and C chunks are staged once in LDS ([token][n] rows, n permuted
//    inside each 32-block as npos() states, so that the C fragment of C.H_in
//    takes the slot map of the transposing read of H_in); C rows are the B
//    operand of both CB^T and C.H_in.
// Per head: x (Xn[j][p]) and H_in (Hn[n][p], rounded to bf16) are staged in
// their natural row-major layouts, plus the G and dt rows; the A-operand
// fragments (the contraction index down the rows) come from the transposing
// LDS read.  The next head's rows are loaded into registers (fully coalesced:
// consecutive threads take consecutive 16-byte pieces of a row) while the
// current head computes (software pipeline), then written to LDS after a
// barrier; the first head's rows are issued right behind the B and C loads of
// the block's prologue, so they arrive while the C.B^T tiles are built.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

#include <type_traits>

namespace ssd {

template <int Q, int NK, int CT, bool F32M = false>
struct HgCfg {
  static constexpr int QT = Q / 16;
  static constexpr int NPAIR = QT / 2;  // row-tile pairs: pair w holds row tiles w and QT-1-w
  // SPLIT: waves per row-tile pair.  At Q = 128 with N >= 128 one block per
  // compute unit is all the LDS allows, so the pair's column tiles are split
  // over two waves (each builds the pair's decayed interaction fragments):
  // eight waves per block instead of four, two per SIMD.
  static constexpr int SPLIT = (Q == 128 && NK >= 4) ? 2 : 1;
  static constexpr int NCW = NPAIR * SPLIT;  // compute waves
  static constexpr int T = 64 * NCW;
  static constexpr int CW = CT / SPLIT;      // column tiles per wave
  static constexpr int PT = CT * 16;
  static constexpr int N = NK * 32;   // this variant needs N == NK*32
  // Row pitches are 16 elements (8 dwords) past a multiple of 64 dwords: the
  // 16-byte fragment reads of 16 rows by 4 lane groups then fall in distinct
  // banks (a 4-dword pad halves the read rate on this LDS).
  static constexpr int NPI = N + 16;  // pitch (elements) of n-indexed LDS rows
  // pitch of the p-indexed rows Xn, Hn: an odd multiple of 8 dwords modulo
  // 64, so a transposing read (per half wave: 8 consecutive rows x 32 bytes)
  // is free of bank conflicts
  static constexpr int XNP = PT + 16;
  static constexpr size_t lds_bs = (size_t)Q * NPI * 2;
  // F32M (fp32 matrix operands): H_in is staged in fp32, transposed ([p][n])
  // with its 16-byte groups of n XOR-swizzled by the row p (see ht_pos)
  static constexpr size_t lds_h = F32M ? sizeof(float) * (size_t)PT * N : (size_t)N * XNP * 2;
  static constexpr size_t lds_xh = (size_t)Q * XNP * 2 + lds_h;
  static constexpr size_t lds_a = lds_bs > lds_xh ? lds_bs : lds_xh;  // Bs, later Xn + Hn
  static constexpr size_t lds_c = (size_t)Q * NPI * 2;                // Cs
  static constexpr size_t lds_w = sizeof(float) * (size_t)(QT / 2) * Q;  // Ws
  // DB (N = 64, 128): the per-head tiles are double-buffered -- two buffers
  // of Xn, Hn, Ws, Gs, dts, both aliasing the phase-0/1 Bs + Cs area, with
  // the C fragments of C.H_in kept in registers -- so a head needs one
  // barrier instead of two.  N = 256 keeps the single-buffer layout (its C
  // fragments would not fit in registers).
  static constexpr bool DB = (NK == 2 || NK == 4) && !F32M;
  static constexpr size_t lds_buf = lds_xh + lds_w + 2 * sizeof(float) * Q;  // one buffer
  static constexpr size_t lds_db = 2 * lds_bs > 2 * lds_buf ? 2 * lds_bs : 2 * lds_buf;
  static constexpr size_t lds_total = DB ? lds_db : lds_a + lds_c + lds_w + 2 * sizeof(float) * Q;
  static constexpr size_t lds_varlen = lds_total + sizeof(int) * Q;  // + the seq-start row (packed sequences)
};

// LDS tiles of one head: x, H_in, the column-factor table, G and dt
struct HgBuf {
  uint16_t* Xn;  // [Q][XNP]
  uint16_t* Hn;  // [N][XNP] (bf16 operands)
  float* Ht;     // [PT][N] swizzled (fp32 operands)
  float* Ws;     // [QT/2][Q]
  float* Gs;     // [Q]
  float* dts;    // [Q]
};

struct HgArgs {
  const void* x;
  const void* Bm;
  const void* Cm;
  const float* dt_bhl;
  const float* dA_cumsum;
  const void* carried;  // fp32, or bf16 bits when H_BF16
  const float* D;
  const int* seq_start;  // packed sequences (VARLEN): [B,nc,Q]
  void* y;
  int L, H, P, G, nc, HG;
  int lin;  // REV: tokens of the forward input arrays
  int b, c, g, hlast, p0;  // hlast: the block's last head (walked first)
  int64_t tok0;
};

// Position of state index n inside a Bs / Cs row.  The transposing read of
// H_in gives lane (l16, lg) at step s the indices n = 32s + 16t + 4lg + r as
// slots 4t + r (t = 0, 1; r = 0..3); storing n at 32s + 8lg + 4t + r makes the
// matching C fragment one 16-byte read.  CB^T reads B and C rows at the same
// positions, so its contraction is unaffected.
__device__ __forceinline__ int npos(int n) {
  return (n & ~31) | ((n & 12) << 1) | ((n & 16) >> 2) | (n & 3);
}

// Element offset of H_in[n][p] in the fp32 transposed tile Ht[p][n] (row
// pitch N): the 16-byte group n / 4 is XOR-ed with ((p / 4) + 4 (p mod 4))
// mod 16, so that both the transposing writes (16 rows p = 4c + q, one n)
// and the fragment reads (16 rows p, one group of n each) fall in distinct
// banks of the 64-bank LDS.
template <int N>
__device__ __forceinline__ int ht_pos(int n, int p) {
  const int sw = ((p >> 2) + 4 * (p & 3)) & 15;
  return p * N + ((((n >> 2) ^ sw)) << 2) + (n & 3);
}

// bf16 fragment (8 slots) widened to fp32, slot order kept
__device__ __forceinline__ OpF32::Frag widen_frag8(const OpBF16::Frag& f) {
  OpF32::Frag r;
  r.lo = make_float4(bf16_bits_to_f32(f.v.x & 0xffffu), bf16_bits_to_f32(f.v.x >> 16),
                     bf16_bits_to_f32(f.v.y & 0xffffu), bf16_bits_to_f32(f.v.y >> 16));
  r.hi = make_float4(bf16_bits_to_f32(f.v.z & 0xffffu), bf16_bits_to_f32(f.v.z >> 16),
                     bf16_bits_to_f32(f.v.w & 0xffffu), bf16_bits_to_f32(f.v.w >> 16));
  return r;
}

template <int Q, int NK, int CT, bool H_BF16, bool Y_BF16, bool RAGGED, bool VARLEN, bool F32M, bool REV>
__device__ __forceinline__ void hg_body(const HgArgs& a, unsigned char* smem, const int tid) {
  using Cfg = HgCfg<Q, NK, CT, F32M>;
  using Op = OpBF16;  // C.B^T (exact: B and C are bf16 inputs)
  using Frag = Op::Frag;
  // M.X and C.H_in: bf16 operands, or (F32M) fp32 operands -- the decayed
  // interaction tile and H_in in fp32, x widened exactly from bf16
  using OpM = std::conditional_t<F32M, OpF32, OpBF16>;
  using FragM = typename OpM::Frag;
  auto to_m = [](const Frag& f) -> FragM {
    if constexpr (F32M) return widen_frag8(f);
    else return f;
  };
  constexpr int QT = Cfg::QT, PT = Cfg::PT, N = Cfg::N, NPI = Cfg::NPI, XNP = Cfg::XNP, T = Cfg::T;
  constexpr int CW = Cfg::CW, NPAIR = Cfg::NPAIR;
  static_assert(PT == 64, "the prefetch maps assume a 64-column slice");
  constexpr int NXB = Q * (PT / 8);          // x prefetch pieces (16 bytes: 8 columns of one token)
  // H prefetch pieces (16 bytes: 4 fp32 or 8 bf16 columns of one n)
  constexpr int HCOL = H_BF16 ? 8 : 4;
  constexpr int NHB = N * (PT / HCOL);
  constexpr int XPT = NXB / T;               // pieces per thread
  constexpr int HPT = NHB / T;
  static_assert(NXB % T == 0 && NHB % T == 0, "prefetch pieces must divide evenly over the block");
  constexpr int NSL = QT + 1;                // CB^T sub-tiles held per wave
  static_assert(T % Q == 0 && (Q & (Q - 1)) == 0, "the G/dt staging assumes T is a multiple of Q");

  constexpr bool DB = Cfg::DB;
  uint16_t* Bs = reinterpret_cast<uint16_t*>(smem);                                  // [Q][NPI]  (phase 0-1 only)
  uint16_t* Cs = reinterpret_cast<uint16_t*>(smem + (DB ? Cfg::lds_bs : Cfg::lds_a));  // [Q][NPI]
  // buffer k of the per-head tiles (single buffer: Xn, Hn alias Bs; Ws, Gs,
  // dts follow Cs)
  auto hbuf = [&](int k) -> HgBuf {
    HgBuf r;
    if constexpr (DB) {
      unsigned char* base = smem + (size_t)k * Cfg::lds_buf;
      r.Xn = reinterpret_cast<uint16_t*>(base);
      r.Hn = r.Xn + Q * XNP;
      r.Ws = reinterpret_cast<float*>(base + Cfg::lds_xh);
    } else {
      r.Xn = reinterpret_cast<uint16_t*>(smem);
      r.Hn = r.Xn + Q * XNP;
      r.Ws = reinterpret_cast<float*>(smem + Cfg::lds_a + Cfg::lds_c);
    }
    r.Ht = reinterpret_cast<float*>(r.Xn + Q * XNP);
    r.Gs = r.Ws + (QT / 2) * Q;
    r.dts = r.Gs + Q;
    return r;
  };
  HgBuf cur = hbuf(0);  // the tiles of the head being computed
  // VARLEN: per row of the chunk, the first token of its sequence inside the
  // chunk (-1: the sequence runs in from before the chunk); a row sees column
  // j only if j >= that, and sees the carried state only if it is -1
  int* Sts = reinterpret_cast<int*>(smem + Cfg::lds_total);

  const int lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int H = a.H, P = a.P, G = a.G, nc = a.nc;
  const int64_t tok0 = a.tok0;
  const int HP = H * P;
  // RAGGED (L % Q != 0): rows past the end of the sequence re-read its last
  // row (their dt = 0 zeroes them as interaction columns) and their outputs
  // are not stored
  const int rmax = RAGGED ? min(Q, a.L - a.c * Q) - 1 : Q - 1;
  auto rowc = [&](int r) { return RAGGED ? min(r, rmax) : r; };
  // REV (the backward's adjoint, run over reversed time; never ragged): x, B
  // and C are the forward arrays of a.lin tokens; row r of chunk c (step
  // cQ + r of the L = nc Q steps) reads forward token L-1-(cQ+r), clamped to
  // lin-1 (the steps past the forward sequence have input scale 0).  Input
  // rows are addressed from the chunk's first token tokb by the row offset
  // ro(r); y stays in the kernel's own (reversed) token order.
  static_assert(!(REV && (RAGGED || VARLEN)), "the reversed reading covers whole chunks");
  const int64_t tokb = REV ? (int64_t)a.b * a.lin + (a.L - (a.c + 1) * Q) : tok0;
  const int rmaxr = REV ? a.lin - 1 - (a.L - (a.c + 1) * Q) : 0;
  auto ro = [&](int r) { return REV ? min(Q - 1 - r, rmaxr) : rowc(r); };

  // ---- per-head register prefetch: issued before a head's compute,
  // committed to LDS after it.
  uint4 xv[XPT];   // 16-byte pieces of x rows (8 columns, bf16)
  uint4 hv[HPT];   // 16-byte pieces of H_in rows (4 fp32 or 8 bf16 columns)
  float pg = 0.f, pd = 0.f;
  // x piece blk -> (row, 8-column block cb): 8 consecutive threads take the 8
  // pieces of one row; within a wave the 8 rows are ordered 0,4,1,5,2,6,3,7 so
  // that the two rows written by a 16-lane group fall in different banks.
  auto xmap = [&](int blk, int& row, int& cb) {
    const int lr = (blk >> 3) & 7;
    row = 8 * (blk >> 6) + (lr >> 1) + 4 * (lr & 1);
    cb = blk & 7;
  };
  // Column-factor table rows handled by this thread: entry tid + T*m of Ws is
  // (u, j) = (tid / Q + (T / Q) * m, tid % Q); the reference G_{32u} is the
  // same for the whole wave (Q >= 64), so it is a scalar load.
  constexpr int NWM = (QT / 2) * Q / T;
  static_assert(((QT / 2) * Q) % T == 0, "column-factor entries must divide evenly over the block");
  float gref[NWM];
  // x pieces and the token's G, dt (issued at the top of a head) ...
  // VARLEN: the thread index is laundered through an empty asm at every
  // issue, so the lane-dependent row offsets are recomputed there instead of
  // being hoisted out of the head loop and held (64-bit) in registers for the
  // block's life; the packed-sequence instance would otherwise spill one of
  // them and reload it, with a wait for every load in flight, inside the
  // steps.  (The other instances keep them: recomputing costs them more.)
  auto tid_v = [&]() __attribute__((always_inline)) -> int {
    if constexpr (VARLEN) {
      int lt = tid;
      asm volatile("" : "+v"(lt));
      return lt;
    } else {
      return tid;
    }
  };
  auto issue_xpiece = [&](int h, int uu) __attribute__((always_inline)) {
    const uint16_t* xh = static_cast<const uint16_t*>(a.x) + (tokb * H + h) * (int64_t)P + a.p0;
    const int blk = tid_v() + uu * T;
    if (blk < NXB) {  // always true; the block boundary keeps the scheduler from hoisting across it
      int row, cb;
      xmap(blk, row, cb);
      xv[uu] = *reinterpret_cast<const uint4*>(xh + ro(row) * HP + 8 * cb);
    }
  };
  auto issue_xmeta = [&](int h) __attribute__((always_inline)) {
    // every thread loads (and later stores) the values of token tid mod Q:
    // T is a multiple of Q, and branch-free code keeps the memory waits exact
    const int64_t bhc = ((int64_t)a.b * H + h) * nc + a.c;
    pg = a.dA_cumsum[bhc * Q + (tid_v() & (Q - 1))];
    pd = a.dt_bhl[bhc * Q + (tid_v() & (Q - 1))];
    const int uq = __builtin_amdgcn_readfirstlane(tid / Q);
#pragma unroll
    for (int m = 0; m < NWM; ++m) gref[m] = a.dA_cumsum[bhc * Q + 32 * (uq + (T / Q) * m)];
  };
  auto issue_x = [&](int h) __attribute__((always_inline)) {
#pragma unroll
    for (int uu = 0; uu < XPT; ++uu) issue_xpiece(h, uu);
    issue_xmeta(h);
  };
  // ... and H_in pieces (issued after the C.H_in product, spreading the
  // vector-memory issue over the head)
  auto issue_h = [&](int h) __attribute__((always_inline)) {
    // H_in piece blk -> (n = blk / (PT / HCOL), columns HCOL * (blk % (PT / HCOL)) ..):
    // consecutive threads read one row
    const int64_t hoff = (((int64_t)a.b * nc + a.c) * H + h) * (int64_t)(N * P) + a.p0;
#pragma unroll
    for (int uu = 0; uu < HPT; ++uu) {
      const int blk = tid_v() + uu * T;
      const int n = blk / (PT / HCOL), col = HCOL * (blk % (PT / HCOL));
      if constexpr (H_BF16) {
        if (blk < NHB) hv[uu] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.carried) + hoff + n * P + col);
      } else {
        if (blk < NHB) hv[uu] = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.carried) + hoff + n * P + col);
      }
    }
  };
  // ---- phase 0: B and C chunks -> Bs, Cs ([token][npos(n)], bf16).  A
  // 16-byte piece holds n = 8nb .. 8nb+7, whose two 4-element halves land at
  // npos(8nb) and npos(8nb + 4).
  {
    const int64_t bc0 = (tokb * G + a.g) * N;  // element offset of (token 0 of the chunk, group g)
    const int GN = G * N;
    // all of the thread's B and C pieces are loaded first, then the first
    // head's x and H_in pieces are issued, so that those stay in flight
    // across the C.B^T products below
    constexpr int NBC = (Q * (N / 8) + T - 1) / T;
    uint4 bq[NBC], cq[NBC];
#pragma unroll
    for (int u = 0; u < NBC; ++u) {
      const int idx = tid + u * T;
      if (idx < Q * (N / 8)) {
        const int j = idx / (N / 8), nb = idx - (idx / (N / 8)) * (N / 8);
        const int off = ro(j) * GN + 8 * nb;
        bq[u] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.Bm) + bc0 + off);
        cq[u] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.Cm) + bc0 + off);
      }
    }
    // VARLEN: the row of sequence starts (one entry per thread, T >= Q)
    const int st_row = VARLEN && tid < Q ? a.seq_start[((int64_t)a.b * a.nc + a.c) * Q + tid] : 0;
    issue_x(a.hlast);
    issue_h(a.hlast);
    if constexpr (VARLEN)
      if (tid < Q) Sts[tid] = st_row;
#pragma unroll
    for (int u = 0; u < NBC; ++u) {
      const int idx = tid + u * T;
      if (idx < Q * (N / 8)) {
        const int j = idx / (N / 8), nb = idx - (idx / (N / 8)) * (N / 8);
        const int q0 = j * NPI + npos(8 * nb), q1 = j * NPI + npos(8 * nb + 4);
        const uint4 bv = bq[u], cv = cq[u];
        *reinterpret_cast<uint2*>(Bs + q0) = make_uint2(bv.x, bv.y);
        *reinterpret_cast<uint2*>(Bs + q1) = make_uint2(bv.z, bv.w);
        *reinterpret_cast<uint2*>(Cs + q0) = make_uint2(cv.x, cv.y);
        *reinterpret_cast<uint2*>(Cs + q1) = make_uint2(cv.z, cv.w);
      }
    }
  }
  __syncthreads();

  // ---- phase 1: causal CB^T sub-tiles of the wave's two row tiles (fp32,
  // registers).  Tile ra = w keeps its sub-tile js at slot js, tile
  // rb = QT-1-w at slot QT - js; the slots of a sub-tile pair (2k, 2k+1) are
  // therefore compile-time constants whatever the wave.
  const int wave = tid >> 6;
  const int pair = Cfg::SPLIT == 1 ? wave : wave % NPAIR;  // the wave's row-tile pair
  const int ra = pair, rb = QT - 1 - pair;
  f32x4_t cb[NSL];
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    const bool first = sl <= ra;
    const int js = first ? sl : QT - sl;
    const int tile = first ? ra : rb;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const Frag bf = Lds<Op>::load8(Bs + (16 * js + l16) * NPI + 32 * s + 8 * lg);
      const Frag cf = Lds<Op>::load8(Cs + (16 * tile + l16) * NPI + 32 * s + 8 * lg);
      acc = Op::mma(bf, cf, acc);
    }
    cb[sl] = acc;
  }
  // VARLEN: the latest sequence start over the rows of each of the wave's
  // two row tiles (wave-uniform; -1: no row starts a sequence in the chunk)
  int msta = -1, mstb = -1;
  if constexpr (VARLEN) {
    int va = Sts[16 * ra + l16], vb = Sts[16 * rb + l16];
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      va = max(va, __shfl_xor(va, off, 16));
      vb = max(vb, __shfl_xor(vb, off, 16));
    }
    msta = __builtin_amdgcn_readfirstlane(va);
    mstb = __builtin_amdgcn_readfirstlane(vb);
  }
  // DB: the C fragments of the wave's two row tiles for C.H_in, in registers
  Frag cfa[DB ? NK : 1], cfb[DB ? NK : 1];
  if constexpr (DB) {
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      cfa[s] = Lds<Op>::load8(Cs + (16 * ra + l16) * NPI + 32 * s + 8 * lg);
      cfb[s] = Lds<Op>::load8(Cs + (16 * rb + l16) * NPI + 32 * s + 8 * lg);
    }
  }

  auto commit = [&](const HgBuf& t) __attribute__((always_inline)) {
#pragma unroll
    for (int uu = 0; uu < XPT; ++uu) {
      const int blk = tid + uu * T;
      if (blk >= NXB) continue;
      int row, cb;
      xmap(blk, row, cb);
      const uint4 q = xv[uu];  // rebuilt from its components: a whole-struct copy kept xv in scratch
      *reinterpret_cast<uint4*>(t.Xn + row * XNP + 8 * cb) = make_uint4(q.x, q.y, q.z, q.w);
    }
#pragma unroll
    for (int uu = 0; uu < HPT; ++uu) {
      const int blk = tid + uu * T;
      if (blk >= NHB) continue;
      const int n = blk / (PT / HCOL), col = HCOL * (blk % (PT / HCOL));
      const uint4 q = hv[uu];
      if constexpr (F32M) {
        // fp32 values (bf16 carried states widened exactly), transposed
        float hvl[HCOL];
        if constexpr (H_BF16) {
          const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hvl[2 * e] = bf16_bits_to_f32(w4[e] & 0xffffu);
            hvl[2 * e + 1] = bf16_bits_to_f32(w4[e] >> 16);
          }
        } else {
          hvl[0] = __uint_as_float(q.x); hvl[1] = __uint_as_float(q.y);
          hvl[2] = __uint_as_float(q.z); hvl[3] = __uint_as_float(q.w);
        }
#pragma unroll
        for (int e = 0; e < HCOL; ++e) t.Ht[ht_pos<N>(n, col + e)] = hvl[e];
      } else if constexpr (H_BF16) {
        *reinterpret_cast<uint4*>(t.Hn + n * XNP + col) = make_uint4(q.x, q.y, q.z, q.w);
      } else {
        *reinterpret_cast<uint2*>(t.Hn + n * XNP + col) =
            make_uint2(pack_bf16x2(__uint_as_float(q.x), __uint_as_float(q.y)),
                       pack_bf16x2(__uint_as_float(q.z), __uint_as_float(q.w)));
      }
    }
    // G is kept in base-2 units (G log2 e) on chip: every use is an exponential
    const float pg2 = pg * kLog2e;
    t.Gs[tid & (Q - 1)] = pg2;  // threads tid and tid + Q write the same value
    t.dts[tid & (Q - 1)] = pd;
    // Column factors of the off-diagonal sub-tiles: for the reference row
    // R = 32u, Ws[u][j] = exp(G_R - G_j) dt_j, read only for j < R (so
    // G_R <= G_j and the factor is <= 1); entries with j >= R are unused.
#pragma unroll
    for (int m = 0; m < NWM; ++m) t.Ws[tid + T * m] = fast_exp2(gref[m] * kLog2e - pg2) * pd;
  };


  // Sub-tile pair steps of one head for both row tiles of the wave.  TSEL (0:
  // tile ra, 1: tile rb) fixes the register-slot map of a tile; the tile
  // indices are run-time, wave-uniform values, so all waves share this code.
  // The helpers only build the M fragment of a pair; each tile has a single
  // MFMA site per step, so its accumulators are updated in place (alternative
  // MFMA sites per branch made the compiler copy accumulators at every merge,
  // each copy waiting for the MFMA results).
  // Off-diagonal pair k of a tile whose diagonal pair is U: M' = CB * Ws[U][j].
  auto offdiag_frag = [&](auto tsel_c, const int k, const int U, int lg, int sti, int ms) -> FragM {
    constexpr int TSEL = decltype(tsel_c)::value;
    const float4 w0 = *reinterpret_cast<const float4*>(cur.Ws + U * Q + 32 * k + 4 * lg);
    const float4 w1 = *reinterpret_cast<const float4*>(cur.Ws + U * Q + 32 * k + 16 + 4 * lg);
    const f32x4_t c0 = cb[TSEL ? (QT - 2 * k) : 2 * k];
    const f32x4_t c1 = cb[TSEL ? (QT - 2 * k - 1) : 2 * k + 1];
    float m[8] = {c0[0] * w0.x, c0[1] * w0.y, c0[2] * w0.z, c0[3] * w0.w,
                  c1[0] * w1.x, c1[1] * w1.y, c1[2] * w1.z, c1[3] * w1.w};
    if constexpr (VARLEN) {
      // only pairs left of the tile's latest sequence start hold masked
      // entries (ms is wave-uniform: a scalar branch)
      if (ms > 32 * k) {
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8)
          if (32 * k + 16 * (e8 >> 2) + 4 * lg + (e8 & 3) < sti) m[e8] = 0.f;
      }
    }
    return OpM::from_f32(m);
  };
  // Diagonal pair k = tile / 2: the row factor exp(G_i - G_R) first scales
  // everything accumulated so far (in place), then the pair takes exact
  // decays, with the causal select made before the exponential: a masked
  // entry gets exp(-inf) = 0, which zeroes its finite C.B^T value.  (The
  // upper sub-tile of an even tile, whose slot holds the other tile's values,
  // is zeroed outright; that select also keeps the register allocator from
  // copying the accumulators.)
  auto diag_frag = [&](auto tsel_c, const int k, const int tile, f32x4_t (&acc)[CW], int l16, int lg, int sti,
                       int ms) -> FragM {
    constexpr int TSEL = decltype(tsel_c)::value;
    const int i = 16 * tile + l16;  // the token this lane's interaction values and outputs belong to
    // G and dt of the lane's 8 tokens j = 32k + 16t + 4lg + r, read as vectors
    const float4 g0 = *reinterpret_cast<const float4*>(cur.Gs + 32 * k + 4 * lg);
    const float4 g1 = *reinterpret_cast<const float4*>(cur.Gs + 32 * k + 16 + 4 * lg);
    const float4 d0 = *reinterpret_cast<const float4*>(cur.dts + 32 * k + 4 * lg);
    const float4 d1 = *reinterpret_cast<const float4*>(cur.dts + 32 * k + 16 + 4 * lg);
    const float gi = cur.Gs[i];  // base-2 units
    const float gR = cur.Gs[32 * k];
    {
      const float e = fast_exp2(gi - gR);
#pragma unroll
      for (int c2 = 0; c2 < CW; ++c2) acc[c2] *= e;
    }
    const float gj[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float dj[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    const f32x4_t c0 = cb[TSEL ? (QT - 2 * k) : 2 * k];
    const f32x4_t c1 = (2 * k + 1 <= tile) ? cb[TSEL ? (QT - 2 * k - 1) : 2 * k + 1] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    const float cvv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    float m[8];
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
      const int j = 32 * k + 16 * (e8 >> 2) + 4 * lg + (e8 & 3);
      const bool keep = VARLEN ? (j <= i && (ms <= 32 * k || j >= sti)) : j <= i;
      const float dec = fast_exp2(keep ? gi - gj[e8] : -INFINITY);
      m[e8] = cvv[e8] * dj[e8] * dec;
    }
    return OpM::from_f32(m);
  };
  // One pass over the pair index k serves both tiles (ta = w < tb = QT-1-w, so
  // the diagonal pair of ta comes first): the x fragments of a step are read
  // once for both, and those of step k+1 are read while step k computes.
  // `ln` is the lane index laundered through an empty asm at the top of each
  // head iteration: lane-dependent addresses are recomputed per head instead
  // of being hoisted out of the head loop, where they would stay live.
  auto steps = [&](const int ta, const int tb, f32x4_t (&acc0)[CW], f32x4_t (&acc1)[CW], int ln, int hn, int ctb) {
    const int l16 = ln & 15, lg = ln >> 4;
    const int Ua = ta >> 1, Ub = tb >> 1;
    const int sta = VARLEN ? Sts[16 * ta + l16] : -1, stb = VARLEN ? Sts[16 * tb + l16] : -1;
    Frag xn[CW];
#pragma unroll
    for (int c2 = 0; c2 < CW; ++c2) xn[c2] = lds_frag_tr(cur.Xn + 16 * (ctb + c2), XNP, ln);
#pragma unroll
    for (int k = 0; k < QT / 2; ++k) {
      if (k <= Ub) {
        // one 16-byte piece of the next head's x rows per step: the
        // vector-memory issue is spread over the head instead of queued at
        // its start by all waves at once
        if (k < XPT) issue_xpiece(hn, k);
        Frag xf[CW];
#pragma unroll
        for (int c2 = 0; c2 < CW; ++c2) xf[c2] = xn[c2];
        if (k + 1 < QT / 2) {
#pragma unroll
          for (int c2 = 0; c2 < CW; ++c2) xn[c2] = lds_frag_tr(cur.Xn + 32 * (k + 1) * XNP + 16 * (ctb + c2), XNP, ln);
        }
        if (k <= Ua) {
          FragM mfa;
          if (k < Ua) mfa = offdiag_frag(std::integral_constant<int, 0>{}, k, Ua, lg, sta, msta);
          else mfa = diag_frag(std::integral_constant<int, 0>{}, k, ta, acc0, l16, lg, sta, msta);
#pragma unroll
          for (int c2 = 0; c2 < CW; ++c2) acc0[c2] = OpM::mma(to_m(xf[c2]), mfa, acc0[c2]);
        }
        FragM mfb;
        if (k < Ub) mfb = offdiag_frag(std::integral_constant<int, 1>{}, k, Ub, lg, stb, mstb);
        else mfb = diag_frag(std::integral_constant<int, 1>{}, k, tb, acc1, l16, lg, stb, mstb);
#pragma unroll
        for (int c2 = 0; c2 < CW; ++c2) acc1[c2] = OpM::mma(to_m(xf[c2]), mfb, acc1[c2]);
      }
    }
  };
  // skip connection and store of one row tile: y[i][16ct + 4lg .. +3]
  auto store_tile = [&](const int tile, const f32x4_t (&acc)[CW], int h, float dsk, int ln, int ctb) {
    const int l16 = ln & 15, lg = ln >> 4;
    const int i = 16 * tile + l16;
    if (RAGGED && i > rmax) return;
    const int64_t ybase = (tok0 * H + h) * (int64_t)P + a.p0;
    uint2 w[CW];
#pragma unroll
    for (int c2 = 0; c2 < CW; ++c2) {
      const int ct = ctb + c2;
      const int pc = 16 * ct + 4 * lg;
      const int off = i * HP + pc;
      float v[4];
      const uint2 xq = *reinterpret_cast<const uint2*>(cur.Xn + i * XNP + pc);  // x[i][pc .. pc+3]
      const float xr[4] = {bf16_bits_to_f32(xq.x & 0xffffu), bf16_bits_to_f32(xq.x >> 16),
                           bf16_bits_to_f32(xq.y & 0xffffu), bf16_bits_to_f32(xq.y >> 16)};
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[c2][r] + dsk * xr[r];
      if constexpr (Y_BF16) {
        w[c2].x = pack_bf16x2(v[0], v[1]);
        w[c2].y = pack_bf16x2(v[2], v[3]);
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + ybase + off) = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    if constexpr (Y_BF16) {
      // column tiles paired (0,1), (2,3): one 16-byte store per pair and lane
#pragma unroll
      for (int cp = 0; cp < CW / 2; ++cp)
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.y) + ybase + i * HP + 16 * ctb + 32 * cp +
                                  pair_tiles_col(lg)) = pair_tiles_16b(w[2 * cp], w[2 * cp + 1]);
    }
  };

  __syncthreads();  // every wave is done reading Bs (and Cs, with DB) before the tiles overwrite them
  commit(hbuf(0));
  __syncthreads();

  for (int hh = 0; hh < a.HG; ++hh) {
    const int h = a.hlast - hh;
    cur = hbuf(DB ? (hh & 1) : 0);
    // The prefetch and commit run on every iteration (the last one loads its
    // own head again, unused): with no conditional around them the compiler's
    // memory-counter waits stay exact, so the loads of the next head remain in
    // flight across the whole compute of this one.
    const int hn = hh + 1 < a.HG ? h - 1 : h;
    issue_xmeta(hn);
    const float dsk = a.D[h];
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // wave index laundered as well, then made wave-uniform (an SGPR), so the
    // branches on the tile index are scalar branches
    int wv = wave;
    asm volatile("" : "+v"(wv));
    wv = __builtin_amdgcn_readfirstlane(wv);
    const int wpair = Cfg::SPLIT == 1 ? wv : wv % NPAIR;
    const int ta = wpair, tb = QT - 1 - wpair;
    const int ctb = Cfg::SPLIT == 1 ? 0 : CW * (wv / NPAIR);  // the wave's first column tile
    {
      const int l16 = ln & 15, lg = ln >> 4;
      // The output tiles are accumulated TRANSPOSED, Y^T = H^T C^T + X^T M^T
      // (operand order swapped, same fragments): lane (l16, lg) holds
      // y[i = 16*tile + l16][p = 16ct + 4lg + r], r = 0..3, written with one
      // 8-byte store.  Carried-state term first, for both tiles at once (each
      // H fragment read once per wave), scaled by exp(G_R) now and by
      // exp(G_i - G_R) at the tile's diagonal step.
      f32x4_t acc0[CW], acc1[CW];
#pragma unroll
      for (int c2 = 0; c2 < CW; ++c2) {
        acc0[c2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1[c2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        const FragM ca0 = to_m(DB ? cfa[DB ? s : 0] : Lds<Op>::load8(Cs + (16 * ta + l16) * NPI + 32 * s + 8 * lg));
        const FragM ca1 = to_m(DB ? cfb[DB ? s : 0] : Lds<Op>::load8(Cs + (16 * tb + l16) * NPI + 32 * s + 8 * lg));
        if constexpr (F32M) {
          // one fp32 H fragment at a time (slots 4t + r <-> n = 32s + 16t +
          // 4lg + r, as the C fragment)
#pragma unroll
          for (int c2 = 0; c2 < CW; ++c2) {
            const int p = 16 * (ctb + c2) + l16;
            FragM hf;
            hf.lo = *reinterpret_cast<const float4*>(cur.Ht + ht_pos<N>(32 * s + 4 * lg, p));
            hf.hi = *reinterpret_cast<const float4*>(cur.Ht + ht_pos<N>(32 * s + 16 + 4 * lg, p));
            acc0[c2] = OpM::mma(hf, ca0, acc0[c2]);
            acc1[c2] = OpM::mma(hf, ca1, acc1[c2]);
          }
        } else {
          Frag hf[CW];
#pragma unroll
          for (int c2 = 0; c2 < CW; ++c2) hf[c2] = lds_frag_tr(cur.Hn + 32 * s * XNP + 16 * (ctb + c2), XNP, ln);
#pragma unroll
          for (int c2 = 0; c2 < CW; ++c2) {
            acc0[c2] = OpM::mma(hf[c2], ca0, acc0[c2]);
            acc1[c2] = OpM::mma(hf[c2], ca1, acc1[c2]);
          }
        }
      }
      issue_h(hn);
      float e0 = fast_exp2(cur.Gs[32 * (ta >> 1)]), e1 = fast_exp2(cur.Gs[32 * (tb >> 1)]);
      if constexpr (VARLEN) {
        // rows that start their sequence inside the chunk do not see the carried state
        const int l16c = ln & 15;
        if (Sts[16 * ta + l16c] >= 0) e0 = 0.f;
        if (Sts[16 * tb + l16c] >= 0) e1 = 0.f;
      }
#pragma unroll
      for (int c2 = 0; c2 < CW; ++c2) {
        acc0[c2] *= e0;
        acc1[c2] *= e1;
      }
      // the waves whose steps carry both tiles most often take priority
      // over their SIMD neighbours (same MFMA count, denser chains)
      if (wpair >= QT / 4) __builtin_amdgcn_s_setprio(2);
      steps(ta, tb, acc0, acc1, ln, hn, ctb);
      __builtin_amdgcn_s_setprio(0);
      // pieces a short step loop did not issue
#pragma unroll
      for (int k = 0; k < XPT; ++k)
        if (k > (tb >> 1)) issue_xpiece(hn, k);
      store_tile(ta, acc0, h, dsk, ln, ctb);
      store_tile(tb, acc1, h, dsk, ln, ctb);
    }
    if constexpr (DB) {
      // the other buffer was last read by the previous head, which every wave
      // finished before the previous barrier
      commit(hbuf((hh + 1) & 1));
      __syncthreads();
    } else {
      __syncthreads();  // all reads of this head's tiles are done
      commit(cur);
      __syncthreads();
    }
  }
}

// Y_BF16 is a template parameter rather than a run-time flag: a branch around
// the output stores would make the compiler's memory-counter waits for the
// prefetched loads conservative (they would also wait for the stores).
template <int Q, int NK, int CT, bool H_BF16, bool Y_BF16, bool RAGGED, bool VARLEN, bool F32M, bool REV = false>
__global__ __launch_bounds__((HgCfg<Q, NK, CT, F32M>::T)) void chunk_scan_hg_kernel(
    const void* __restrict__ x, const void* __restrict__ Bm, const void* __restrict__ Cm,
    const float* __restrict__ dt_bhl, const float* __restrict__ dA_cumsum, const void* __restrict__ carried,
    const float* __restrict__ D, void* __restrict__ y, int L, int H, int P, int G, int nc, int HG,
    int nhg, int npt, int remap, const int* __restrict__ seq_start, int lin) {
  extern __shared__ __align__(16) unsigned char hg_smem[];
  // block -> (b, c, g, head group, p slice).  With remap != 0 the mapping is
  // XCD-aware: consecutive logical blocks (same chunk, neighbouring head
  // groups) land on the same XCD and share its L2 for the B/C chunk.
  const unsigned nblk = gridDim.x;
  unsigned bid = blockIdx.x;
  if (remap) bid = (bid & 7u) * (nblk >> 3) + (bid >> 3);
  HgArgs a;
  a.x = x; a.Bm = Bm; a.Cm = Cm; a.dt_bhl = dt_bhl; a.dA_cumsum = dA_cumsum; a.carried = carried; a.D = D; a.y = y;
  a.seq_start = seq_start;
  a.L = L; a.H = H; a.P = P; a.G = G; a.nc = nc; a.HG = HG;
  a.lin = lin;
  const int pt = bid % npt;
  unsigned rest = bid / npt;
  const int hgi = rest % nhg;
  rest /= nhg;
  a.g = rest % G;
  rest /= G;
  // chunks in reverse order: the state step before this kernel (state
  // passing, or the fused walk) writes the carried states of the last chunks
  // last, so those are the likeliest to be still cached when read first
  a.c = nc - 1 - (int)(rest % nc);
  a.b = rest / nc;
  // The block walks its heads from the last to the first: in the forward the
  // chunk-state kernel, launched just before, walks the same head groups
  // first to last, so the x rows it read last are the likeliest to be still
  // in the last-level cache.
  a.hlast = a.g * (H / G) + hgi * HG + HG - 1;
  a.p0 = pt * HgCfg<Q, NK, CT, F32M>::PT;
  a.tok0 = (int64_t)a.b * L + (int64_t)a.c * Q;
  hg_body<Q, NK, CT, H_BF16, Y_BF16, RAGGED, VARLEN, F32M, REV>(a, hg_smem, threadIdx.x);
}

// ------------------------------------------------------------------ host side

// Heads per block: the largest divisor HG of the group's head count such that
// the grid still gives every CU at least one block.
static int pick_heads_per_block(const Dims& d, int npt) {
  const int64_t hpg = d.H / d.G;
  const int64_t base = d.B * d.nc * d.G * npt;
  const int cus = device_cu_count();
  int best = 1;
  for (int64_t k = 1; k <= hpg; ++k) {
    if (hpg % k) continue;
    best = (int)(hpg / k);
    if (base * k >= cus) break;
  }
  return best;
}

template <int Q, int NK, bool H_BF16, bool Y_BF16, bool F32M>
static auto pick_hg_kernel(bool ragged, bool varlen) {
  // packed sequences: the guarded-store instance only where the last chunk
  // is ragged as well
  if (varlen)
    return ragged ? chunk_scan_hg_kernel<Q, NK, 4, H_BF16, Y_BF16, true, true, F32M>
                  : chunk_scan_hg_kernel<Q, NK, 4, H_BF16, Y_BF16, false, true, F32M>;
  return ragged ? chunk_scan_hg_kernel<Q, NK, 4, H_BF16, Y_BF16, true, false, F32M>
                : chunk_scan_hg_kernel<Q, NK, 4, H_BF16, Y_BF16, false, false, F32M>;
}

template <int Q, int NK, bool H_BF16, bool F32M>
static hipError_t launch_hg_inst(const Dims& d, const void* x, const void* Bm, const void* Cm, const float* dt_bhl,
                                 const float* dA_cumsum, const void* carried, const float* D, void* y,
                                 bool y_bf16, hipStream_t stream, const int* seq_start, int lin = 0) {
  constexpr int CT = 4;
  using Cfg = HgCfg<Q, NK, CT, F32M>;
  const bool ragged = d.L % Q != 0, varlen = seq_start != nullptr;
  auto kern = y_bf16 ? pick_hg_kernel<Q, NK, H_BF16, true, F32M>(ragged, varlen)
                     : pick_hg_kernel<Q, NK, H_BF16, false, F32M>(ragged, varlen);
  if (lin > 0) {
    // reversed reading: the backward's precision modes only (bf16 carried
    // states and y with bf16 operands, fp32 with fp32), whole chunks
    if constexpr (H_BF16 != F32M) {
      if (ragged || varlen || y_bf16 != H_BF16) return hipErrorInvalidValue;
      kern = chunk_scan_hg_kernel<Q, NK, CT, H_BF16, H_BF16, false, false, F32M, true>;
    } else {
      return hipErrorInvalidValue;
    }
  }
  const size_t lds = varlen ? Cfg::lds_varlen : Cfg::lds_total;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int threads = Cfg::T;
  const int npt = (int)(d.P / Cfg::PT);
  int HG = pick_heads_per_block(d, npt);
  const int tuned = tuning_for(d, F32M).scan_hg;
  if (tuned > 0 && (d.H / d.G) % tuned == 0) HG = tuned;
  const int nhg = (int)(d.H / d.G) / HG;
  const int64_t nblk = d.B * d.nc * d.G * nhg * npt;
  const int remap = (nblk % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(threads), lds, stream, x, Bm, Cm, dt_bhl, dA_cumsum, carried,
                     D, y, (int)d.L, (int)d.H, (int)d.P, (int)d.G, (int)d.nc, HG, nhg, npt, remap, seq_start, lin);
  return hipGetLastError();
}

template <int Q, int NK, bool F32M>
static bool hg_fits() {
  using Cfg = HgCfg<Q, NK, 4, F32M>;
  return Cfg::lds_varlen <= 160 * 1024 && Q <= Cfg::T && 64 * Cfg::NCW <= Cfg::T && (Q == 128 || Q == 256);
}

bool chunk_scan_hg_supported(const Dims& d, bool in_bf16, bool f32_mma) {
  // bf16 inputs only: C.B^T runs on bf16 matrix instructions (exact for bf16
  // values), and the fp32-operand instance widens x exactly
  if (!in_bf16) return false;
  if (d.P % 64 != 0) return false;
  if (d.nc * d.B * d.G * (d.H / d.G) * (d.P / 64) > 0x7fffffff) return false;
  const int64_t key = d.Q * 1000 + d.N;
#define HG_FITS(QQ, KK) (f32_mma ? hg_fits<QQ, KK, true>() : hg_fits<QQ, KK, false>())
  switch (key) {
    case 128 * 1000 + 64: return HG_FITS(128, 2);
    case 128 * 1000 + 128: return HG_FITS(128, 4);
    case 128 * 1000 + 256: return HG_FITS(128, 8);
    case 256 * 1000 + 64: return HG_FITS(256, 2);
    case 256 * 1000 + 128: return HG_FITS(256, 4);
    default: return false;
  }
#undef HG_FITS
}

template <bool H_BF16, bool F32M>
static hipError_t launch_hg_dtype(const Dims& d, const void* x, const void* Bm, const void* Cm, const float* dt_bhl,
                                  const float* dA_cumsum, const void* carried, const float* D, void* y, bool y_bf16,
                                  hipStream_t stream, const int* seq_start) {
  const int64_t key = d.Q * 1000 + d.N;
#define HG_CASE(QQ, NN, KK)                                                                                      \
  case QQ * 1000 + NN:                                                                                           \
    return launch_hg_inst<QQ, KK, H_BF16, F32M>(d, x, Bm, Cm, dt_bhl, dA_cumsum, carried, D, y, y_bf16, stream, \
                                                seq_start);
  switch (key) {
    HG_CASE(128, 64, 2)
    HG_CASE(128, 128, 4)
    HG_CASE(128, 256, 8)
    HG_CASE(256, 64, 2)
    HG_CASE(256, 128, 4)
    default: return hipErrorInvalidValue;
  }
#undef HG_CASE
}

hipError_t launch_chunk_scan_hg(const Dims& d, const void* x, const void* Bm, const void* Cm, bool in_bf16,
                                const float* dt_bhl, const float* dA_cumsum, const void* carried, bool carried_bf16,
                                const float* D, void* y, bool y_bf16, bool f32_mma, hipStream_t stream,
                                const int* seq_start) {
  if (!in_bf16) return hipErrorInvalidValue;
  if (f32_mma) {
    if (carried_bf16)
      return launch_hg_dtype<true, true>(d, x, Bm, Cm, dt_bhl, dA_cumsum, carried, D, y, y_bf16, stream, seq_start);
    return launch_hg_dtype<false, true>(d, x, Bm, Cm, dt_bhl, dA_cumsum, carried, D, y, y_bf16, stream, seq_start);
  }
  if (carried_bf16)
    return launch_hg_dtype<true, false>(d, x, Bm, Cm, dt_bhl, dA_cumsum, carried, D, y, y_bf16, stream, seq_start);
  return launch_hg_dtype<false, false>(d, x, Bm, Cm, dt_bhl, dA_cumsum, carried, D, y, y_bf16, stream, seq_start);
}

hipError_t launch_chunk_scan_hg_rev(const Dims& d, const void* x, const void* Bm, const void* Cm, const float* dt_bhl,
                                    const float* dA_cumsum, const void* carried, bool carried_bf16, const float* D,
                                    void* y, bool f32_mma, int64_t lin, hipStream_t stream) {
  if (lin <= d.L - d.Q || lin > d.L) return hipErrorInvalidValue;
  const int64_t key = d.Q * 1000 + d.N;
#define HG_REV(QQ, NN, KK)                                                                                     \
  case QQ * 1000 + NN:                                                                                         \
    return f32_mma ? launch_hg_inst<QQ, KK, false, true>(d, x, Bm, Cm, dt_bhl, dA_cumsum, carried, D, y,        \
                                                         carried_bf16, stream, nullptr, (int)lin)               \
                   : launch_hg_inst<QQ, KK, true, false>(d, x, Bm, Cm, dt_bhl, dA_cumsum, carried, D, y,        \
                                                         carried_bf16, stream, nullptr, (int)lin);
  if (carried_bf16 == f32_mma) return hipErrorInvalidValue;
  switch (key) {
    HG_REV(128, 64, 2)
    HG_REV(128, 128, 4)
    HG_REV(128, 256, 8)
    HG_REV(256, 64, 2)
    HG_REV(256, 128, 4)
    default: return hipErrorInvalidValue;
  }
#undef HG_REV
}

}  // namespace ssd
