// chunk_scan.hip -- fused chunk output on MFMA: carried-state term, decayed and
// causally masked C.B^T interaction applied to x, and the D skip.
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), compute_out paragraph: the
// three terms are fused in one tiled kernel; the interaction tile C.B^T is
// accumulated on the matrix units (phase 1), then decayed by exp(G_i - G_j)
// and causally masked (phase 2) with a register-level select built from index
// comparisons, so no mask tensor and no [B, nc, Q, Q] matrix ever reaches
// memory; entries with i < j (positive exponents) are discarded by the
// select.  For token i of chunk c:
//     y_i = exp(G_i) C_i^T H_in  +  sum_{j<=i} (C_i . B_j) exp(G_i - G_j) dt_j x_j  +  D x_i
//
// Work split: one 256-thread block per (b, c, HPB heads of one group, column
// slice of P, group of 64 output rows); wave w owns the 16-row tile
// rt = 4*group + w of every head of the block.  The C.B^T sub-tiles depend on
// the group only, so each is computed once and serves all HPB heads (each
// with its own decays, x and accumulators).  Blocks of the heaviest row group
// (the chunk's last rows see the most columns) are dispatched first.
//
// Register/LDS data flow, per wave (l16 = lane % 16, lg = lane / 16):
//  * C rows of the wave's tile are loaded once from HBM as fragments
//    (row l16, contraction slots n = 32s + 8lg + e); they are the A operand
//    of C.H_in and the B operand of the interaction product.
//  * H_in (fp32 [N][P] in HBM) is staged head by head into LDS transposed,
//    Ht[p][n], as the B operand of C.H_in.  The result is scaled per row by
//    exp(G_i) and stays in that head's output accumulators.
//  * For every 32-token column step j0 up to the diagonal, the block stages
//    B rows (natural layout Bs[j][n]) and each head's x transposed
//    (Xt[head][p][j]).  The wave
//    computes the TRANSPOSED interaction tile CB^T[j][i] = B_j . C_i (operand
//    roles swapped, since (C B^T)^T = B C^T), so that each lane ends up with
//    four consecutive j for one row i.  After decay and mask in registers,
//    those values are directly the A fragment of M.X: slot e = 4t + r of lane
//    (row l16, lg) stands for token j = j0 + 16t + 4lg + r, and the x fragment
//    is read from Xt with the same slot map.  M never leaves registers.
//  * Epilogue: y = acc + D x, written in the output dtype.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

#include <type_traits>

namespace ssd {

constexpr int kScanThreads = 256;
constexpr int kScanKS = 32;  // tokens per column step
constexpr int kScanRows = 64;  // output rows per block (4 waves x 16)

template <class Op>
struct ScanCfg {
  static constexpr int PAD = Op::kBytes == 2 ? 8 : 4;
  static constexpr int XP = kScanKS + PAD;  // pitch of Xt rows (elements)
};

template <class Op, int NK, int CT, int HPB>
__global__ __launch_bounds__(kScanThreads) void chunk_scan_kernel(
    const void* __restrict__ x, const void* __restrict__ Bm, const void* __restrict__ Cm, int in_bf16,
    const float* __restrict__ dt_bhl, const float* __restrict__ dA_cumsum, const void* __restrict__ carried,
    int h_bf16, const float* __restrict__ D, void* __restrict__ y, int y_bf16, int L, int H, int P, int N, int G,
    int Q, int nc, const int* __restrict__ seq_start) {
  using E = typename OpElem<Op>::type;
  using Frag = typename Op::Frag;
  constexpr int PT = CT * 16;
  constexpr int NPI = NK * 32 + ScanCfg<Op>::PAD;  // pitch of n-indexed rows (elements)
  constexpr int XP = ScanCfg<Op>::XP;
  extern __shared__ __align__(16) unsigned char sc_smem[];
  E* Ht = reinterpret_cast<E*>(sc_smem);  // [PT][NPI]  carried state of one head, transposed
  E* Bs = Ht + PT * NPI;                  // [KS][NPI]  B rows of the column step
  E* Xt = Bs + kScanKS * NPI;             // [HPB][PT][XP]  x of the column step, transposed
  float* Gs = reinterpret_cast<float*>(Xt + HPB * PT * XP);  // [HPB][Q]
  float* dts = Gs + HPB * Q;                                  // [HPB][Q]
  // packed sequences (seq_start != NULL): per row, the first token of its
  // sequence inside the chunk, or -1 when it continues from before the chunk
  int* Sts = reinterpret_cast<int*>(dts + HPB * Q);  // [Q]

  const int npt = P / PT;
  const int nrg = Q > kScanRows ? Q / kScanRows : 1;
  const int h0 = (blockIdx.x / npt) * HPB, pt = blockIdx.x - (blockIdx.x / npt) * npt;
  const int rg = (nrg - 1) - (int)(blockIdx.y / nc);
  const int c = blockIdx.y - (blockIdx.y / nc) * nc;
  const int b = blockIdx.z;
  const int g = h0 / (H / G);  // the block's heads share the group (HPB divides H / G)
  const int p0 = pt * PT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lg = lane >> 4;
  const bool bf = in_bf16 != 0;

  const int i0 = (rg * 4 + wave) * 16;  // first row of this wave's tile
  const bool active = i0 < Q;
  const int row_end = min(Q, (rg + 1) * kScanRows);

  const int64_t tok0 = (int64_t)b * L + (int64_t)c * Q;
  // Rows past the end of the sequence (ragged last chunk) re-read the last
  // row: their dt = 0 zeroes them as interaction columns, and their outputs
  // are not stored.
  const int rmax = min(Q, L - c * Q) - 1;

  for (int j = tid; j < row_end; j += kScanThreads) {
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      const int64_t bhc = ((int64_t)b * H + h0 + hh) * nc + c;
      Gs[hh * Q + j] = dA_cumsum[bhc * Q + j];
      dts[hh * Q + j] = dt_bhl[bhc * Q + j];
    }
    Sts[j] = seq_start ? seq_start[((int64_t)b * nc + c) * Q + j] : -1;
  }

  // H_in of head h -> Ht[p][n] (zero for padded n >= N), by 8x8 register transposes.
  auto stage_h = [&](int h) {
    const int64_t hoff = (((int64_t)b * nc + c) * H + h) * (int64_t)N * P + p0;
    const int nbn = NK * 4;  // 8-row blocks along n (padded)
    for (int blk = tid; blk < nbn * (PT / 8); blk += kScanThreads) {
      const int bn = blk % nbn, bp = blk / nbn;
      float v[8][8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int n = 8 * bn + r;
        if (n < N) {
          // fp32 or bf16 carried states (bf16 widens exactly)
          load8_as_f32(carried, hoff + (int64_t)n * P + 8 * bp, h_bf16 != 0, v[r]);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[r][q] = 0.f;
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float col[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) col[r] = v[r][q];
        Lds<Op>::store8(Ht + (8 * bp + q) * NPI + 8 * bn, col);
      }
    }
  };

  // C fragments of this wave's rows: row i0 + l16, slots n = 32s + 8lg + e.
  Frag cf[NK];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    const int n = 32 * s + 8 * lg;
    if (active && n < N) {
      float t[8];
      load8_as_f32(Cm, ((tok0 + min(i0 + l16, rmax)) * G + g) * N + n, bf, t);
      cf[s] = Op::from_f32(t);
    } else {
      cf[s] = Op::zero();
    }
  }

  f32x4_t acc[HPB][CT];
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[hh][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  float gi[HPB];  // G of row i0 + l16 (interaction-tile column index), per head
  int sti = -1;   // first token of that row's sequence in the chunk (-1: before it)
#pragma unroll
  for (int hh = 0; hh < HPB; ++hh) {
    if (hh > 0) __syncthreads();  // the previous head's Ht reads are done
    stage_h(h0 + hh);
    __syncthreads();
    gi[hh] = 0.f;
    if (active) {
      // carried-state term: acc = C_rows . H_in, rows then scaled by exp(G_i)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s = 0; s < NK; ++s)
          acc[hh][ct] = Op::mma(cf[s], Lds<Op>::load8(Ht + (16 * ct + l16) * NPI + 32 * s + 8 * lg), acc[hh][ct]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // a row that starts its sequence inside the chunk does not see the carried state
        const float e = Sts[i0 + 4 * lg + r] < 0 ? fast_exp(Gs[hh * Q + i0 + 4 * lg + r]) : 0.f;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[hh][ct][r] *= e;
      }
      gi[hh] = Gs[hh * Q + i0 + l16];
      sti = Sts[i0 + l16];
    }
  }

  for (int j0 = 0; j0 < row_end; j0 += kScanKS) {
    __syncthreads();  // previous step's fragment reads are done
    // B rows, natural layout, zero-padded to NK*32 columns
    for (int idx = tid; idx < kScanKS * NK * 4; idx += kScanThreads) {
      const int j = idx / (NK * 4), nb = idx - (idx / (NK * 4)) * (NK * 4);
      const int n = 8 * nb;
      float t[8];
      if (n < N) {
        load8_as_f32(Bm, ((tok0 + min(j0 + j, rmax)) * G + g) * N + n, bf, t);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) t[q] = 0.f;
      }
      Lds<Op>::store8(Bs + j * NPI + n, t);
    }
    // x of each head transposed, 8x8 register transposes
    for (int blk = tid; blk < HPB * (kScanKS / 8) * (PT / 8); blk += kScanThreads) {
      const int hh = blk / ((kScanKS / 8) * (PT / 8)), rb = blk - hh * ((kScanKS / 8) * (PT / 8));
      const int jb = rb & 3, pb = rb >> 2;
      float v[8][8];
#pragma unroll
      for (int r = 0; r < 8; ++r)
        load8_as_f32(x, ((tok0 + min(j0 + 8 * jb + r, rmax)) * H + h0 + hh) * P + p0 + 8 * pb, bf, v[r]);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float col[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) col[r] = v[r][q];
        Lds<Op>::store8(Xt + (hh * PT + 8 * pb + q) * XP + 8 * jb, col);
      }
    }
    __syncthreads();

    if (active && j0 <= i0 + 15) {
      const int i = i0 + l16;
      // the two C.B^T sub-tiles of the step, shared by the block's heads:
      // lane holds CB^T[j = j0 + 16t + 4lg + r][i]
      f32x4_t cb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        cb[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (j0 + 16 * t <= i0 + 15) {
#pragma unroll
          for (int s = 0; s < NK; ++s)
            cb[t] = Op::mma(Lds<Op>::load8(Bs + (16 * t + l16) * NPI + 32 * s + 8 * lg), cf[s], cb[t]);
        }
      }
#pragma unroll
      for (int hh = 0; hh < HPB; ++hh) {
        // The causal select comes first: a masked entry never reaches exp,
        // and its G/dt reads are redirected to row i (always staged).
        float m[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = j0 + 16 * t + 4 * lg + r;
            const bool keep = j <= i && j >= sti;  // causal, and inside row i's sequence
            const int jc = keep ? j : i;
            const float dec = fast_exp(keep ? gi[hh] - Gs[hh * Q + jc] : -INFINITY) * dts[hh * Q + jc];
            m[4 * t + r] = keep ? cb[t][r] * dec : 0.f;
          }
        const Frag mf = Op::from_f32(m);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const E* xr = Xt + (hh * PT + 16 * ct + l16) * XP + 4 * lg;
          acc[hh][ct] = Op::mma(mf, Lds<Op>::load4x2(xr, xr + 16), acc[hh][ct]);
        }
      }
    }
  }

  if (active) {
#pragma unroll
    for (int hh = 0; hh < HPB; ++hh) {
      const int h = h0 + hh;
      const float dsk = D[h];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (i0 + 4 * lg + r > rmax) continue;
          const int64_t off = ((tok0 + i0 + 4 * lg + r) * H + h) * P + p0 + 16 * ct + l16;
          const float v = acc[hh][ct][r] + dsk * load1_as_f32(x, off, bf);
          if (y_bf16)
            reinterpret_cast<uint16_t*>(y)[off] = (uint16_t)f32_to_bf16_bits(v);
          else
            reinterpret_cast<float*>(y)[off] = v;
        }
    }
  }
}

static int scan_ct(int64_t P) { return (P % 64 == 0) ? 4 : (P % 32 == 0) ? 2 : 1; }
static int scan_nk(int64_t N) {
  const int64_t k = (N + 31) / 32;
  return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : 8;
}

static size_t scan_lds_hpb(const Dims& d, bool f32_mma, int hpb) {
  const size_t PT = 16 * scan_ct(d.P);
  const size_t eb = f32_mma ? 4 : 2;
  const size_t pad = f32_mma ? ScanCfg<OpF32>::PAD : ScanCfg<OpBF16>::PAD;
  const size_t npi = 32 * scan_nk(d.N) + pad;
  const size_t xp = kScanKS + pad;
  return eb * (PT * npi + kScanKS * npi + hpb * PT * xp) + (2 * hpb + 1) * sizeof(float) * (size_t)d.Q;
}

// one head per block: the support limit
size_t chunk_scan_lds_bytes(const Dims& d, bool f32_mma) { return scan_lds_hpb(d, f32_mma, 1); }

// Heads per block: the largest of 4, 2, 1 that divides the group's head count
// and keeps the block within 80 KB of LDS (two blocks per compute unit).
static int scan_hpb(const Dims& d, bool f32_mma) {
  const int64_t hpg = d.H / d.G;
  for (int k : {4, 2})
    if (hpg % k == 0 && scan_lds_hpb(d, f32_mma, k) <= 80 * 1024) return k;
  return 1;
}

template <class Op, int NK, int CT>
static hipError_t launch_scan_inst(const Dims& d, const void* x, const void* Bm, const void* Cm, bool in_bf16,
                                   const float* dt_bhl, const float* dA_cumsum, const void* carried,
                                   bool h_bf16, const float* D, void* y, bool y_bf16, const int* seq_start,
                                   hipStream_t stream, size_t) {
  const bool f32m = std::is_same<Op, OpF32>::value;
  const int hpb = scan_hpb(d, f32m);
  auto kern = hpb == 4 ? chunk_scan_kernel<Op, NK, CT, 4>
              : hpb == 2 ? chunk_scan_kernel<Op, NK, CT, 2>
                         : chunk_scan_kernel<Op, NK, CT, 1>;
  const size_t lds = scan_lds_hpb(d, f32m, hpb);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t nrg = d.Q > kScanRows ? d.Q / kScanRows : 1;
  const dim3 grid((unsigned)((d.H / hpb) * (d.P / (16 * CT))), (unsigned)(nrg * d.nc), (unsigned)d.B);
  hipLaunchKernelGGL(kern, grid, dim3(kScanThreads), lds, stream, x, Bm, Cm, (int)in_bf16, dt_bhl, dA_cumsum,
                     carried, (int)h_bf16, D, y, (int)y_bf16, (int)d.L, (int)d.H, (int)d.P, (int)d.N, (int)d.G, (int)d.Q,
                     (int)d.nc, seq_start);
  return hipGetLastError();
}

template <class Op, int NK>
static hipError_t launch_scan_ct(const Dims& d, const void* x, const void* Bm, const void* Cm, bool in_bf16,
                                 const float* dt_bhl, const float* dA_cumsum, const void* carried,
                                 bool h_bf16, const float* D, void* y, bool y_bf16, const int* seq_start,
                                 hipStream_t stream, size_t lds) {
  switch (scan_ct(d.P)) {
    case 4: return launch_scan_inst<Op, NK, 4>(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, seq_start, stream, lds);
    case 2: return launch_scan_inst<Op, NK, 2>(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, seq_start, stream, lds);
    default: return launch_scan_inst<Op, NK, 1>(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, seq_start, stream, lds);
  }
}

template <class Op>
static hipError_t launch_scan_op(const Dims& d, const void* x, const void* Bm, const void* Cm, bool in_bf16,
                                 const float* dt_bhl, const float* dA_cumsum, const void* carried,
                                 bool h_bf16, const float* D, void* y, bool y_bf16, const int* seq_start,
                                 hipStream_t stream, size_t lds) {
  switch (scan_nk(d.N)) {
    case 1: return launch_scan_ct<Op, 1>(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, seq_start, stream, lds);
    case 2: return launch_scan_ct<Op, 2>(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, seq_start, stream, lds);
    case 4: return launch_scan_ct<Op, 4>(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, seq_start, stream, lds);
    default: return launch_scan_ct<Op, 8>(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, seq_start, stream, lds);
  }
}

hipError_t launch_chunk_scan(const Dims& d, const void* x, const void* Bm, const void* Cm, bool in_bf16,
                             const float* dt_bhl, const float* dA_cumsum, const void* carried, bool h_bf16,
                             const float* D, void* y, bool y_bf16, bool f32_mma, hipStream_t stream,
                             const int* seq_start) {
  if (chunk_scan_hg_supported(d, in_bf16, f32_mma))
    return launch_chunk_scan_hg(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, f32_mma,
                                stream, seq_start);
  const size_t lds = chunk_scan_lds_bytes(d, f32_mma);
  if (f32_mma)
    return launch_scan_op<OpF32>(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, seq_start, stream, lds);
  return launch_scan_op<OpBF16>(d, x, Bm, Cm, in_bf16, dt_bhl, dA_cumsum, carried, h_bf16, D, y, y_bf16, seq_start, stream, lds);
}

}  // namespace ssd
