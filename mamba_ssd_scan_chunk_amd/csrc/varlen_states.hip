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

hipError_t launch_varlen_states(const Dims& d, const void* x, const void* Bm, bool in_bf16, const float* dt_bhl,
                                const float* dA_cumsum, const int* seq_start, const void* carried, bool carried_bf16,
                                int64_t nseq, const int64_t* last_token, float* out, hipStream_t stream) {
  if (nseq <= 0) return hipSuccess;
  const int tn = (int)((d.N + 31) / 32), tp = (int)((d.P + 31) / 32);
  const int64_t nblk = nseq * d.H * tn * tp;
  hipLaunchKernelGGL(varlen_states_kernel, dim3((unsigned)nblk), dim3(kVsThreads), 0, stream, x, Bm, (int)in_bf16,
                     dt_bhl, dA_cumsum, seq_start, carried, (int)carried_bf16, last_token, out, d.B * d.L, (int)d.L,
                     (int)d.H, (int)d.P,
                     (int)d.N, (int)d.G, (int)d.Q, (int)d.nc, tn, tp);
  return hipGetLastError();
}

}  // namespace ssd
