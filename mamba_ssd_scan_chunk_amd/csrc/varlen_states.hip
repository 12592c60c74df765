// varlen_states.hip -- states at chosen tokens of packed sequences.
//
// Page: "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
// Tensor Cores with cuTile" (disconfirmai.com), paragraph on the three kernels
// (the state after a chunk is the decayed incoming state plus the chunk's own
// pre-multiplied b x^T product) and jump-formula paragraph.  The same
// decomposition holds at any token t of chunk c, position i = t - cQ, of a
// sequence that runs through position st..i of the chunk:
//     h_t = [st = -1] exp(G_i) H_in[c] + sum_{j = max(st, 0)}^{i} exp(G_i - G_j) dt_j B_j x_j^T
// where H_in[c] is the carried state entering the chunk and st the start of
// t's sequence inside the chunk (-1: it runs in from before).  One 256-thread
// block per (requested token, head, 32 x 32 tile of the state): thread
// (n = tid / 8, p = 4 (tid % 8) .. +3) accumulates its four elements over the
// chunk's tokens, staged 64 at a time in LDS with their weights applied
// (one thread per token and 8-element group of each row: 16-byte loads for
// bf16 inputs).  H_in is fp32, or bf16 bits when carried_bf16.
#include "ssd_device.hpp"
#include "ssd_launch.hpp"

namespace ssd {

constexpr int kVsThreads = 256;
constexpr int kVsTok = 64;  // tokens staged per step

__global__ __launch_bounds__(kVsThreads) void varlen_states_kernel(
    const void* __restrict__ x, const void* __restrict__ Bm, int in_bf16, const float* __restrict__ dt_bhl,
    const float* __restrict__ dA_cumsum, const int* __restrict__ seq_start, const void* __restrict__ carried,
    int carried_bf16, const int64_t* __restrict__ last_token, float* __restrict__ out, int64_t ntok, int L, int H,
    int P, int N, int G, int Q, int nc, int tn, int tp) {
  __shared__ __align__(16) float Bsh[kVsTok][32];
  __shared__ __align__(16) float Xsh[kVsTok][32];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x % (tn * tp);
  const int h = (blockIdx.x / (tn * tp)) % H;
  const int64_t s = blockIdx.x / (tn * tp) / H;
  const int n0 = 32 * (tile / tp), p0 = 32 * (tile % tp);
  const int64_t bt = last_token[s];  // flattened token b * L + t
  if (bt < 0 || bt >= ntok) return;    // out of range: the output is left untouched
  const int64_t b = bt / L;
  const int t = (int)(bt - b * L);
  const int c = t / Q, ie = t - c * Q;
  const int g = h / (H / G);
  const int64_t bhc = ((int64_t)b * H + h) * nc + c;
  const int st = seq_start[((int64_t)b * nc + c) * Q + ie];
  const int j0 = st < 0 ? 0 : st;
  const float gi = dA_cumsum[bhc * Q + ie];
  const int nl = tid >> 3, pl = 4 * (tid & 7);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const int64_t tok0 = (int64_t)b * L + (int64_t)c * Q;
  for (int js = j0; js <= ie; js += kVsTok) {
    const int cnt = min(kVsTok, ie + 1 - js);
    __syncthreads();  // the previous step's reads are done
    {
      // thread -> (token jj = tid / 4, 8-element group k8 = tid % 4); N, P are
      // multiples of 16, so a group lies wholly inside or outside the range
      const int jj = tid >> 2, k8 = 8 * (tid & 3);
      float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (jj < cnt) {
        const int j = js + jj;
        const float w = fast_exp(gi - dA_cumsum[bhc * Q + j]) * dt_bhl[bhc * Q + j];
        if (n0 + k8 < N) {
          load8_as_f32(Bm, ((tok0 + j) * G + g) * N + n0 + k8, in_bf16 != 0, bv);
#pragma unroll
          for (int e = 0; e < 8; ++e) bv[e] *= w;
        }
        if (p0 + k8 < P) load8_as_f32(x, ((tok0 + j) * H + h) * P + p0 + k8, in_bf16 != 0, xv);
      }
      *reinterpret_cast<float4*>(&Bsh[jj][k8]) = make_float4(bv[0], bv[1], bv[2], bv[3]);
      *reinterpret_cast<float4*>(&Bsh[jj][k8 + 4]) = make_float4(bv[4], bv[5], bv[6], bv[7]);
      *reinterpret_cast<float4*>(&Xsh[jj][k8]) = make_float4(xv[0], xv[1], xv[2], xv[3]);
      *reinterpret_cast<float4*>(&Xsh[jj][k8 + 4]) = make_float4(xv[4], xv[5], xv[6], xv[7]);
    }
    __syncthreads();
    for (int jj = 0; jj < cnt; ++jj) {
      const float bv = Bsh[jj][nl];
      const float4 xv = *reinterpret_cast<const float4*>(&Xsh[jj][pl]);
      acc[0] = fmaf(bv, xv.x, acc[0]);
      acc[1] = fmaf(bv, xv.y, acc[1]);
      acc[2] = fmaf(bv, xv.z, acc[2]);
      acc[3] = fmaf(bv, xv.w, acc[3]);
    }
  }
  const int n = n0 + nl;
  if (n >= N) return;
  const int64_t NP = (int64_t)N * P;
  const int64_t hoff = (((int64_t)b * nc + c) * H + h) * NP + (int64_t)n * P;
  const float e = st < 0 ? fast_exp(gi) : 0.f;
  float* o = out + ((int64_t)s * H + h) * NP + (int64_t)n * P;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = p0 + pl + r;
    if (p < P) {
      const float hin = st < 0 ? load1_as_f32(carried, hoff + p, carried_bf16 != 0) : 0.f;
      o[p] = st < 0 ? fmaf(e, hin, acc[r]) : acc[r];
    }
  }
}

// The same states on the matrix cores (bf16 inputs, N and P multiples of 64):
// one 256-thread block per (requested token, head, 64 x 64 state tile).  The
// chunk's tokens from the 32-token block holding the sequence's first token
// j0 up to i are staged token-major in LDS, 64 at a time -- x rows scaled by
// w_j = exp(G_i - G_j) dt_j
// and rounded to bf16 (the chunk-state kernels' arithmetic), or raw with the
// weights applied in fp32 at use (F32M) -- and the contraction over tokens
// takes its fragments from the transposing LDS read, as in the chunk states:
// wave w accumulates S^T for n in 32 (w % 2) .. +31, p in 32 (w / 2) .. +31.
constexpr int kVmXP = 64 + 16;  // row pitch (elements): conflict-free transposing reads
constexpr int kVmWin = 64;      // tokens staged per step

template <bool F32M>
__global__ __launch_bounds__(kVsThreads) void varlen_states_mma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm, const float* __restrict__ dt_bhl,
    const float* __restrict__ dA_cumsum, const int* __restrict__ seq_start, const void* __restrict__ carried,
    int carried_bf16, const int64_t* __restrict__ last_token, float* __restrict__ out, int64_t ntok, int L, int H,
    int P, int N, int G, int Q, int nc, int tn, int tp) {
  __shared__ __align__(16) uint16_t Xs[kVmWin * kVmXP];  // x rows of the window (p0 .. p0+63)
  __shared__ __align__(16) uint16_t Bs[kVmWin * kVmXP];  // B rows of the window (n0 .. n0+63)
  __shared__ __align__(16) float Wj[kVmWin];              // their weights
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x % (tn * tp);
  const int h = (blockIdx.x / (tn * tp)) % H;
  const int64_t s = blockIdx.x / (tn * tp) / H;
  const int n0 = 64 * (tile / tp), p0 = 64 * (tile % tp);
  const int64_t bt = last_token[s];
  if (bt < 0 || bt >= ntok) return;  // out of range: the output is left untouched (whole block, no barrier yet)
  const int64_t b = bt / L;
  const int t = (int)(bt - b * L);
  const int c = t / Q, ie = t - c * Q;
  const int g = h / (H / G);
  const int64_t bhc = ((int64_t)b * H + h) * nc + c;
  const int st = seq_start[((int64_t)b * nc + c) * Q + ie];
  const int j0 = st < 0 ? 0 : st;
  const float gi = dA_cumsum[bhc * Q + ie];
  const int64_t tok0 = (int64_t)b * L + (int64_t)c * Q;
  const int nh = wave & 1, ph = wave >> 1, l16 = lane & 15, lg = lane >> 4;
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[i][ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // windows of kVmWin tokens from the 32-token block holding j0 to the one
  // holding ie; rows outside j0 .. ie weigh 0 (and re-read row ie)
  for (int r0 = 32 * (j0 / 32); r0 <= ie; r0 += kVmWin) {
    __syncthreads();  // the previous window's fragment reads are done
    if (tid < kVmWin) {
      const int j = r0 + tid;
      Wj[tid] = (j >= j0 && j <= ie) ? fast_exp(gi - dA_cumsum[bhc * Q + j]) * dt_bhl[bhc * Q + j] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kVmWin * 8 / kVsThreads; ++u) {
      const int e = tid + kVsThreads * u;
      const int jj = e >> 3, c8 = e & 7;
      const int j = min(r0 + jj, ie);
      const uint4 xq = *reinterpret_cast<const uint4*>(x + ((tok0 + j) * H + h) * (int64_t)P + p0 + 8 * c8);
      const uint4 bq = *reinterpret_cast<const uint4*>(Bm + ((tok0 + j) * G + g) * (int64_t)N + n0 + 8 * c8);
      uint4 xo = xq;
      if constexpr (!F32M) {
        const float w = Wj[jj];
        xo.x = pack_bf16x2(bf16_bits_to_f32(xq.x & 0xffffu) * w, bf16_bits_to_f32(xq.x >> 16) * w);
        xo.y = pack_bf16x2(bf16_bits_to_f32(xq.y & 0xffffu) * w, bf16_bits_to_f32(xq.y >> 16) * w);
        xo.z = pack_bf16x2(bf16_bits_to_f32(xq.z & 0xffffu) * w, bf16_bits_to_f32(xq.z >> 16) * w);
        xo.w = pack_bf16x2(bf16_bits_to_f32(xq.w & 0xffffu) * w, bf16_bits_to_f32(xq.w >> 16) * w);
      }
      *reinterpret_cast<uint4*>(Xs + jj * kVmXP + 8 * c8) = xo;
      *reinterpret_cast<uint4*>(Bs + jj * kVmXP + 8 * c8) = bq;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kVmWin / 32; ++kk) {
      OpBF16::Frag bf[2], xf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) bf[i] = lds_frag_tr(Bs + 32 * kk * kVmXP + 16 * (2 * nh + i), kVmXP, lane);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) xf[ct] = lds_frag_tr(Xs + 32 * kk * kVmXP + 16 * (2 * ph + ct), kVmXP, lane);
      if constexpr (F32M) {
        // weights of the lane's tokens 32kk + 16t + 4lg + r (slot 4t + r)
        const float4 w0 = *reinterpret_cast<const float4*>(Wj + 32 * kk + 4 * lg);
        const float4 w1 = *reinterpret_cast<const float4*>(Wj + 32 * kk + 16 + 4 * lg);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          OpF32::Frag xw;
          xw.lo = make_float4(bf16_bits_to_f32(xf[ct].v.x & 0xffffu) * w0.x, bf16_bits_to_f32(xf[ct].v.x >> 16) * w0.y,
                              bf16_bits_to_f32(xf[ct].v.y & 0xffffu) * w0.z, bf16_bits_to_f32(xf[ct].v.y >> 16) * w0.w);
          xw.hi = make_float4(bf16_bits_to_f32(xf[ct].v.z & 0xffffu) * w1.x, bf16_bits_to_f32(xf[ct].v.z >> 16) * w1.y,
                              bf16_bits_to_f32(xf[ct].v.w & 0xffffu) * w1.z, bf16_bits_to_f32(xf[ct].v.w >> 16) * w1.w);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            OpF32::Frag bw;
            bw.lo = make_float4(bf16_bits_to_f32(bf[i].v.x & 0xffffu), bf16_bits_to_f32(bf[i].v.x >> 16),
                                bf16_bits_to_f32(bf[i].v.y & 0xffffu), bf16_bits_to_f32(bf[i].v.y >> 16));
            bw.hi = make_float4(bf16_bits_to_f32(bf[i].v.z & 0xffffu), bf16_bits_to_f32(bf[i].v.z >> 16),
                                bf16_bits_to_f32(bf[i].v.w & 0xffffu), bf16_bits_to_f32(bf[i].v.w >> 16));
            acc[i][ct] = OpF32::mma(xw, bw, acc[i][ct]);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) acc[i][ct] = OpBF16::mma(xf[ct], bf[i], acc[i][ct]);
      }
    }
  }
  // lane holds S[n = n0 + 16 (2 nh + i) + l16][p = p0 + 16 (2 ph + ct) + 4 lg .. +3]
  const int64_t NP = (int64_t)N * P;
  const int64_t hbase = (((int64_t)b * nc + c) * H + h) * NP;
  const float e = st < 0 ? fast_exp(gi) : 0.f;
  float* o = out + ((int64_t)s * H + h) * NP;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int n = n0 + 16 * (2 * nh + i) + l16, p = p0 + 16 * (2 * ph + ct) + 4 * lg;
      float hin[4] = {0.f, 0.f, 0.f, 0.f};
      if (st < 0) {
        if (carried_bf16) {
          const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(carried) + hbase + n * P + p);
          hin[0] = bf16_bits_to_f32(q.x & 0xffffu); hin[1] = bf16_bits_to_f32(q.x >> 16);
          hin[2] = bf16_bits_to_f32(q.y & 0xffffu); hin[3] = bf16_bits_to_f32(q.y >> 16);
        } else {
          const float4 q = *reinterpret_cast<const float4*>(static_cast<const float*>(carried) + hbase + n * P + p);
          hin[0] = q.x; hin[1] = q.y; hin[2] = q.z; hin[3] = q.w;
        }
      }
      *reinterpret_cast<float4*>(o + n * P + p) =
          make_float4(fmaf(e, hin[0], acc[i][ct][0]), fmaf(e, hin[1], acc[i][ct][1]), fmaf(e, hin[2], acc[i][ct][2]),
                      fmaf(e, hin[3], acc[i][ct][3]));
    }
}

hipError_t launch_varlen_states(const Dims& d, const void* x, const void* Bm, bool in_bf16, const float* dt_bhl,
                                const float* dA_cumsum, const int* seq_start, const void* carried, bool carried_bf16,
                                int64_t nseq, const int64_t* last_token, float* out, bool f32_mma,
                                hipStream_t stream) {
  if (nseq <= 0) return hipSuccess;
  if (in_bf16 && d.N % 64 == 0 && d.P % 64 == 0) {
    const int tn = (int)(d.N / 64), tp = (int)(d.P / 64);
    const int64_t nblk = nseq * d.H * tn * tp;
    auto kern = f32_mma ? varlen_states_mma_kernel<true> : varlen_states_mma_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(kVsThreads), 0, stream, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(Bm), dt_bhl, dA_cumsum, seq_start, carried, (int)carried_bf16,
                       last_token, out, d.B * d.L, (int)d.L, (int)d.H, (int)d.P, (int)d.N, (int)d.G, (int)d.Q,
                       (int)d.nc, tn, tp);
    return hipGetLastError();
  }
  const int tn = (int)((d.N + 31) / 32), tp = (int)((d.P + 31) / 32);
  const int64_t nblk = nseq * d.H * tn * tp;
  hipLaunchKernelGGL(varlen_states_kernel, dim3((unsigned)nblk), dim3(kVsThreads), 0, stream, x, Bm, (int)in_bf16,
                     dt_bhl, dA_cumsum, seq_start, carried, (int)carried_bf16, last_token, out, d.B * d.L, (int)d.L,
                     (int)d.H, (int)d.P,
                     (int)d.N, (int)d.G, (int)d.Q, (int)d.nc, tn, tp);
  return hipGetLastError();
}

}  // namespace ssd
