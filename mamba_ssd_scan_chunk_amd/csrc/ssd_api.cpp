// ssd_api.cpp -- the C ABI declared in include/ssd.h: argument validation
// (host only, before any HIP call), workspace carving and kernel dispatch.
#include "ssd.h"

#include <hip/hip_runtime.h>

#include <atomic>

#include "ssd_forward.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// Compute units of the current device, queried once per device and kept in
// an atomic per device (the calls may come from several host threads); 256
// (an MI355X) when the query fails.
int device_cu_count() {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool cached = dev >= 0 && dev < kMaxDev;
  if (cached) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  if (cached) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace ssd

namespace {

using ssd::Dims;

constexpr size_t kLdsLimit = 160 * 1024;  // gfx950 LDS per workgroup
constexpr size_t kWsAlign = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Shape checks shared by every call.  Returns SSD_OK and fills `d`.
ssd_status check_shape(const ssd_shape* s, Dims* d) {
  if (!s) return SSD_ERR_NULL;
  if (s->batch <= 0 || s->seqlen <= 0 || s->nheads <= 0 || s->headdim <= 0 || s->dstate <= 0 ||
      s->ngroups <= 0 || s->chunk <= 0)
    return SSD_ERR_SHAPE;
  if (s->nheads % s->ngroups != 0) return SSD_ERR_SHAPE;
  if (s->headdim % 16 != 0 || s->dstate % 16 != 0 || s->headdim > 256 || s->dstate > 256)
    return SSD_ERR_UNSUPPORTED;
  if (s->chunk != 32 && s->chunk != 64 && s->chunk != 128 && s->chunk != 256) return SSD_ERR_UNSUPPORTED;
  // a ragged last chunk (seqlen % chunk != 0) is allowed: nc = ceil(seqlen / chunk)
  const int64_t nc = (s->seqlen - 1) / s->chunk + 1;  // no overflow for any positive seqlen
  // keep every element offset comfortably inside 32-bit grid dimensions
  if (nc > 65535 || s->batch > 65535 || s->nheads > 65535) return SSD_ERR_UNSUPPORTED;
  // The kernels address the rows of one chunk with 32-bit offsets from the
  // chunk's first token (row * H*P into x and y, row * G*N into B and C), and
  // number their blocks per (batch, chunk, head, 16-column tile of P) in 32
  // bits: refuse shapes where either could reach 2^31.
  const int64_t k31 = int64_t(1) << 31;
  if (s->chunk * s->nheads * s->headdim >= k31 || s->chunk * s->ngroups * s->dstate >= k31)
    return SSD_ERR_UNSUPPORTED;
  if (s->batch * nc * s->nheads * (s->headdim / 16) >= k31) return SSD_ERR_UNSUPPORTED;
  d->B = s->batch; d->L = s->seqlen; d->H = s->nheads; d->P = s->headdim;
  d->N = s->dstate; d->G = s->ngroups; d->Q = s->chunk; d->nc = nc;
  return SSD_OK;
}

ssd_status check_dtype(ssd_dtype t) { return (t == SSD_F32 || t == SSD_BF16) ? SSD_OK : SSD_ERR_DTYPE; }
ssd_status check_mma(ssd_mma m) { return (m == SSD_MMA_BF16 || m == SSD_MMA_F32) ? SSD_OK : SSD_ERR_DTYPE; }

ssd_status from_hip(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

#define SSD_TRY(expr)                  \
  do {                                 \
    const ssd_status st_ = (expr);     \
    if (st_ != SSD_OK) return st_;     \
  } while (0)

ssd_status validate_cumsum(const ssd_shape* shape, const float* dt, const float* A, float* dA_cumsum,
                           float* dt_bhl, Dims* d) {
  SSD_TRY(check_shape(shape, d));
  if (!dt || !A || !dA_cumsum) return SSD_ERR_NULL;
  if (!aligned16(dt) || !aligned16(A) || !aligned16(dA_cumsum) || (dt_bhl && !aligned16(dt_bhl)))
    return SSD_ERR_ALIGN;
  return SSD_OK;
}

ssd_status validate_state(const ssd_shape* shape, const void* x, const void* Bm, ssd_dtype in,
                          const float* dt_bhl, const float* dA_cumsum, void* states, ssd_dtype states_dtype,
                          ssd_mma mma, Dims* d) {
  SSD_TRY(check_shape(shape, d));
  SSD_TRY(check_dtype(in));
  SSD_TRY(check_dtype(states_dtype));
  SSD_TRY(check_mma(mma));
  if (!x || !Bm || !dt_bhl || !dA_cumsum || !states) return SSD_ERR_NULL;
  if (!aligned16(x) || !aligned16(Bm) || !aligned16(dt_bhl) || !aligned16(dA_cumsum) || !aligned16(states))
    return SSD_ERR_ALIGN;
  if (ssd::chunk_state_lds_bytes(*d, mma == SSD_MMA_F32) > kLdsLimit) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

ssd_status validate_passing(const ssd_shape* shape, const void* chunk_states, ssd_dtype states_dtype, void* carried,
                            ssd_dtype carried_dtype, const float* dA_cumsum, const float* initial_states,
                            float* final_states, Dims* d) {
  SSD_TRY(check_shape(shape, d));
  SSD_TRY(check_dtype(states_dtype));
  SSD_TRY(check_dtype(carried_dtype));
  if (!chunk_states || !carried || !dA_cumsum) return SSD_ERR_NULL;
  // in place only between equal element sizes
  if (carried_dtype != states_dtype && carried == chunk_states) return SSD_ERR_UNSUPPORTED;
  if (!aligned16(chunk_states) || !aligned16(carried) || !aligned16(dA_cumsum) ||
      (initial_states && !aligned16(initial_states)) || (final_states && !aligned16(final_states)))
    return SSD_ERR_ALIGN;
  return SSD_OK;
}

ssd_status validate_scan(const ssd_shape* shape, const void* x, const void* Bm, const void* Cm, ssd_dtype in,
                         const float* dt_bhl, const float* dA_cumsum, const void* carried, ssd_dtype carried_dtype,
                         const float* D, void* y, ssd_dtype y_dtype, ssd_mma mma, Dims* d) {
  SSD_TRY(check_shape(shape, d));
  SSD_TRY(check_dtype(in));
  SSD_TRY(check_dtype(carried_dtype));
  SSD_TRY(check_dtype(y_dtype));
  SSD_TRY(check_mma(mma));
  if (!x || !Bm || !Cm || !dt_bhl || !dA_cumsum || !carried || !D || !y) return SSD_ERR_NULL;
  if (!aligned16(x) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(dt_bhl) || !aligned16(dA_cumsum) ||
      !aligned16(carried) || !aligned16(D) || !aligned16(y))
    return SSD_ERR_ALIGN;
  if (ssd::chunk_scan_lds_bytes(*d, mma == SSD_MMA_F32) > kLdsLimit) return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

// ssd_forward_varlen's workspace: dA_cumsum, dt_bhl, fp32 carried states
// [B,nc,H,N,P], a bf16 chunk-state area, sequence starts (int32 [B,nc,Q]),
// dA_cumsum for the state passing and dt masked to each chunk's last sequence
// (fp32 [B,H,nc,Q]), each 256-byte aligned.
struct WsLayout {
  size_t dA_off, dt_off, st_off, hb_off, total;
  size_t ss_off, dAp_off, dtl_off, total_varlen;
};

WsLayout workspace_layout(const Dims& d) {
  WsLayout w;
  const size_t bhl = sizeof(float) * (size_t)(d.B * d.H * d.nc * d.Q);
  const size_t st = sizeof(float) * (size_t)(d.B * d.nc * d.H) * (size_t)(d.N * d.P);
  w.dA_off = 0;
  w.dt_off = round_up(w.dA_off + bhl, kWsAlign);
  w.st_off = round_up(w.dt_off + bhl, kWsAlign);
  w.hb_off = round_up(w.st_off + st, kWsAlign);  // bf16 carried states (half the bytes of st)
  w.total = round_up(w.hb_off + st / 2, kWsAlign);
  w.ss_off = w.total;
  w.dAp_off = round_up(w.ss_off + sizeof(int32_t) * (size_t)(d.B * d.nc * d.Q), kWsAlign);
  w.dtl_off = round_up(w.dAp_off + bhl, kWsAlign);
  w.total_varlen = round_up(w.dtl_off + bhl, kWsAlign);
  return w;
}

}  // namespace

extern "C" {

ssd_status ssd_chunk_cumsum(const ssd_shape* shape, const float* dt, const float* A, float* dA_cumsum,
                            float* dt_bhl, void* stream) {
  Dims d;
  SSD_TRY(validate_cumsum(shape, dt, A, dA_cumsum, dt_bhl, &d));
  return from_hip(ssd::launch_chunk_cumsum(d, dt, A, dA_cumsum, dt_bhl, (hipStream_t)stream));
}

ssd_status ssd_chunk_state(const ssd_shape* shape, const void* x, const void* Bm, ssd_dtype in,
                           const float* dt_bhl, const float* dA_cumsum, void* states, ssd_dtype states_dtype,
                           ssd_mma mma, void* stream) {
  Dims d;
  SSD_TRY(validate_state(shape, x, Bm, in, dt_bhl, dA_cumsum, states, states_dtype, mma, &d));
  return from_hip(ssd::launch_chunk_state_any(d, x, Bm, in == SSD_BF16, dt_bhl, dA_cumsum, states,
                                              states_dtype == SSD_BF16, mma == SSD_MMA_F32, (hipStream_t)stream));
}

ssd_status ssd_chunk_cumsum_state(const ssd_shape* shape, const void* x, const void* Bm, ssd_dtype in,
                                  const float* dt, const float* A, float* dA_cumsum, float* dt_bhl, void* states,
                                  ssd_dtype states_dtype, ssd_mma mma, void* stream) {
  Dims d;
  SSD_TRY(validate_state(shape, x, Bm, in, dt_bhl, dA_cumsum, states, states_dtype, mma, &d));
  if (!dt || !A) return SSD_ERR_NULL;
  if (!aligned16(dt) || !aligned16(A)) return SSD_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  const bool bf = in == SSD_BF16, f32m = mma == SSD_MMA_F32, sbf = states_dtype == SSD_BF16;
  // the head-group chunk-state kernel computes the cumulative sums itself
  if (ssd::chunk_state_hg_supported(d, bf, f32m))
    return from_hip(ssd::launch_chunk_state_cumsum_hg(d, x, Bm, dt, A, dA_cumsum, dt_bhl, states, sbf, f32m, s));
  SSD_TRY(from_hip(ssd::launch_chunk_cumsum(d, dt, A, dA_cumsum, dt_bhl, s)));
  return from_hip(ssd::launch_chunk_state_any(d, x, Bm, bf, dt_bhl, dA_cumsum, states, sbf, f32m, s));
}

ssd_status ssd_state_passing(const ssd_shape* shape, const void* chunk_states, ssd_dtype states_dtype,
                             void* carried, ssd_dtype carried_dtype, const float* dA_cumsum,
                             const float* initial_states, float* final_states, void* stream) {
  Dims d;
  SSD_TRY(validate_passing(shape, chunk_states, states_dtype, carried, carried_dtype, dA_cumsum, initial_states,
                           final_states, &d));
  return from_hip(ssd::launch_state_passing_any(d, chunk_states, states_dtype == SSD_BF16, carried,
                                                carried_dtype == SSD_BF16, dA_cumsum, initial_states, final_states,
                                                (hipStream_t)stream));
}

ssd_status ssd_chunk_state_passing(const ssd_shape* shape, const void* x, const void* Bm, ssd_dtype in,
                                   const float* dt_bhl, const float* dA_cumsum, const float* initial_states,
                                   void* carried, ssd_dtype carried_dtype, float* final_states, ssd_mma mma,
                                   void* stream) {
  Dims d;
  SSD_TRY(check_shape(shape, &d));
  SSD_TRY(check_dtype(in));
  SSD_TRY(check_dtype(carried_dtype));
  SSD_TRY(check_mma(mma));
  if (!x || !Bm || !dt_bhl || !dA_cumsum || !carried) return SSD_ERR_NULL;
  if (!aligned16(x) || !aligned16(Bm) || !aligned16(dt_bhl) || !aligned16(dA_cumsum) || !aligned16(carried) ||
      (initial_states && !aligned16(initial_states)) || (final_states && !aligned16(final_states)))
    return SSD_ERR_ALIGN;
  if (!ssd::state_fused_supported(d, in == SSD_BF16, mma == SSD_MMA_F32)) return SSD_ERR_UNSUPPORTED;
  return from_hip(ssd::launch_state_fused(d, x, Bm, dt_bhl, dA_cumsum, initial_states, carried,
                                          carried_dtype == SSD_BF16, final_states, (hipStream_t)stream));
}

ssd_status ssd_decode_step(const ssd_shape* shape, const void* x, const float* dt, const float* A, const void* Bm,
                           const void* Cm, const float* D, ssd_dtype in, float* state, void* y, ssd_dtype y_dtype,
                           void* stream) {
  if (!shape) return SSD_ERR_NULL;
  const ssd_shape* s = shape;
  if (s->batch <= 0 || s->nheads <= 0 || s->headdim <= 0 || s->dstate <= 0 || s->ngroups <= 0 || s->seqlen != 1)
    return SSD_ERR_SHAPE;
  if (s->nheads % s->ngroups != 0) return SSD_ERR_SHAPE;
  SSD_TRY(check_dtype(in));
  SSD_TRY(check_dtype(y_dtype));
  if (!ssd::decode_step_supported(s->headdim)) return SSD_ERR_UNSUPPORTED;
  if (s->batch > 0x7fffffff / s->nheads || s->dstate > 0x7fffffff / s->headdim) return SSD_ERR_UNSUPPORTED;
  if (!x || !dt || !A || !Bm || !Cm || !D || !state || !y) return SSD_ERR_NULL;
  if (!aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(D) ||
      !aligned16(state) || !aligned16(y))
    return SSD_ERR_ALIGN;
  return from_hip(ssd::launch_decode_step(s->batch, s->nheads, s->headdim, s->dstate, s->ngroups, x, dt, A, Bm, Cm,
                                          D, in == SSD_BF16, state, y, y_dtype == SSD_BF16, (hipStream_t)stream));
}

ssd_status ssd_chunk_scan(const ssd_shape* shape, const void* x, const void* Bm, const void* Cm, ssd_dtype in,
                          const float* dt_bhl, const float* dA_cumsum, const void* carried, ssd_dtype carried_dtype,
                          const float* D, void* y, ssd_dtype y_dtype, ssd_mma mma, void* stream) {
  Dims d;
  SSD_TRY(validate_scan(shape, x, Bm, Cm, in, dt_bhl, dA_cumsum, carried, carried_dtype, D, y, y_dtype, mma, &d));
  return from_hip(ssd::launch_chunk_scan(d, x, Bm, Cm, in == SSD_BF16, dt_bhl, dA_cumsum, carried,
                                         carried_dtype == SSD_BF16, D, y,
                                         y_dtype == SSD_BF16, mma == SSD_MMA_F32, (hipStream_t)stream));
}

size_t ssd_workspace_bytes(const ssd_shape* shape) {
  Dims d;
  if (check_shape(shape, &d) != SSD_OK) return 0;
  // enough for either precision path (the fp32 one needs more)
  return ssd::forward_workspace_bytes(d, true);
}

size_t ssd_workspace_bytes_varlen(const ssd_shape* shape) {
  Dims d;
  if (check_shape(shape, &d) != SSD_OK) return 0;
  return workspace_layout(d).total_varlen;
}

// ssd_forward's state step: the fused kernel (chunk states stay on chip) or
// the two-kernel path (fp32 chunk states through memory).  The fused kernel
// walks the chunks in sequence inside each block, so it only pays off with
// enough blocks to keep every compute unit busy: at least two per unit
// (measured: 2048 blocks on 256 units 24% faster per forward, 320 blocks 8%
// slower).
static bool prefer_fused_state(const Dims& d) {
  return ssd::state_fused_blocks(d) >= 2 * (int64_t)ssd::device_cu_count();
}

}  // extern "C"

namespace ssd {

ssd_status forward_validate(const ssd_shape* shape, const void* x, const float* dt, const float* A, const void* Bm,
                            const void* Cm, const float* D, ssd_dtype in, const float* initial_states, const void* y,
                            ssd_dtype y_dtype, const float* final_states, ssd_mma mma, Dims* d) {
  SSD_TRY(check_shape(shape, d));
  SSD_TRY(check_dtype(in));
  SSD_TRY(check_dtype(y_dtype));
  SSD_TRY(check_mma(mma));
  if (!x || !dt || !A || !Bm || !Cm || !D || !y) return SSD_ERR_NULL;
  if (!aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(D) ||
      !aligned16(y) || (initial_states && !aligned16(initial_states)) || (final_states && !aligned16(final_states)))
    return SSD_ERR_ALIGN;
  if (chunk_state_lds_bytes(*d, mma == SSD_MMA_F32) > kLdsLimit || chunk_scan_lds_bytes(*d, mma == SSD_MMA_F32) > kLdsLimit)
    return SSD_ERR_UNSUPPORTED;
  return SSD_OK;
}

// The forward's workspace: dA_cumsum and dt_bhl (fp32 [B,H,nc,Q] each), then
// one state area [B,nc,H,N,P] -- bf16 on the bf16-operand path (the chunk
// states, then the carried states written over them; or the fused state
// path's carried states), fp32 on the fp32 path -- each 256-byte aligned.
struct FwdLayout {
  size_t dA_off, dt_off, st_off, total;
};

static FwdLayout forward_layout(const Dims& d, bool f32_mma) {
  FwdLayout w;
  const size_t bhl = sizeof(float) * (size_t)(d.B * d.H * d.nc * d.Q);
  const size_t st = (f32_mma ? 4 : 2) * (size_t)(d.B * d.nc * d.H) * (size_t)(d.N * d.P);
  w.dA_off = 0;
  w.dt_off = round_up(w.dA_off + bhl, kWsAlign);
  w.st_off = round_up(w.dt_off + bhl, kWsAlign);
  w.total = round_up(w.st_off + st, kWsAlign);
  return w;
}

size_t forward_workspace_bytes(const Dims& d, bool f32_mma) { return forward_layout(d, f32_mma).total; }

ssd_status forward_run(const Dims& d, const void* x, const float* dt, const float* A, const void* Bm, const void* Cm,
                       const float* D, ssd_dtype in, const float* initial_states, void* y, ssd_dtype y_dtype,
                       float* final_states, void* workspace, ssd_mma mma, hipStream_t s) {
  const bool bf = in == SSD_BF16, f32m = mma == SSD_MMA_F32;
  const FwdLayout ws = forward_layout(d, f32m);
  char* base = static_cast<char*>(workspace);
  float* dA = reinterpret_cast<float*>(base + ws.dA_off);
  float* dtb = reinterpret_cast<float*>(base + ws.dt_off);
  void* st = base + ws.st_off;

  const int path = tuning_for(d, f32m).path;
  if (path == 3 && fwd_fused_supported(d, bf, f32m)) {
    // fused forward: neither chunk states nor carried states reach memory
    SSD_TRY(from_hip(launch_chunk_cumsum(d, dt, A, dA, dtb, s)));
    SSD_TRY(from_hip(launch_fwd_fused(d, x, Bm, Cm, dtb, dA, D, initial_states, y, y_dtype == SSD_BF16,
                                      final_states, s)));
    return SSD_OK;
  }
  if (state_fused_supported(d, bf, f32m) && (path == 1 || (path == 0 && prefer_fused_state(d)))) {
    // fused state path: the chunk states never reach memory; the carried
    // states go to the chunk scan as bf16 (its matrix-operand values)
    SSD_TRY(from_hip(launch_chunk_cumsum(d, dt, A, dA, dtb, s)));
    SSD_TRY(from_hip(launch_state_fused(d, x, Bm, dtb, dA, initial_states, st, true, final_states, s)));
    SSD_TRY(from_hip(launch_chunk_scan(d, x, Bm, Cm, bf, dtb, dA, st, true, D, y, y_dtype == SSD_BF16, f32m, s)));
    return SSD_OK;
  }
  // bf16 matrix operands: the chunk states pass through memory as bf16 and
  // the state passing (fp32 recurrence) writes the carried states in place
  // over them, rounded to bf16 -- the operand values the chunk scan would
  // round them to; fp32 matrix operands: fp32 throughout
  const bool sbf = !f32m;
  if (chunk_state_hg_supported(d, bf, f32m)) {
    // the head-group chunk-state kernel computes the cumulative sums itself
    SSD_TRY(from_hip(launch_chunk_state_cumsum_hg(d, x, Bm, dt, A, dA, dtb, st, sbf, f32m, s)));
  } else {
    SSD_TRY(from_hip(launch_chunk_cumsum(d, dt, A, dA, dtb, s)));
    SSD_TRY(from_hip(launch_chunk_state_any(d, x, Bm, bf, dtb, dA, st, sbf, f32m, s)));
  }
  SSD_TRY(from_hip(launch_state_passing_any(d, st, sbf, st, sbf, dA, initial_states, final_states, s)));
  SSD_TRY(from_hip(launch_chunk_scan(d, x, Bm, Cm, bf, dtb, dA, st, sbf, D, y, y_dtype == SSD_BF16, f32m, s)));
  return SSD_OK;
}

}  // namespace ssd

extern "C" {

ssd_status ssd_forward(const ssd_shape* shape, const void* x, const float* dt, const float* A, const void* Bm,
                       const void* Cm, const float* D, ssd_dtype in, const float* initial_states, void* y,
                       ssd_dtype y_dtype, float* final_states, void* workspace, size_t workspace_bytes,
                       ssd_mma mma, void* stream) {
  Dims d;
  SSD_TRY(ssd::forward_validate(shape, x, dt, A, Bm, Cm, D, in, initial_states, y, y_dtype, final_states, mma, &d));
  if (!workspace) return SSD_ERR_WORKSPACE;
  if (workspace_bytes < ssd::forward_workspace_bytes(d, mma == SSD_MMA_F32)) return SSD_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SSD_ERR_ALIGN;
  return ssd::forward_run(d, x, dt, A, Bm, Cm, D, in, initial_states, y, y_dtype, final_states, workspace, mma,
                          (hipStream_t)stream);
}

ssd_status ssd_forward_varlen(const ssd_shape* shape, const void* x, const float* dt, const float* A,
                              const void* Bm, const void* Cm, const float* D, ssd_dtype in, const int32_t* seq_idx,
                              const float* initial_states, void* y, ssd_dtype y_dtype, float* final_states,
                              int64_t nseq, const int64_t* seq_last, float* seq_states, void* workspace,
                              size_t workspace_bytes, ssd_mma mma, void* stream) {
  Dims d;
  SSD_TRY(check_shape(shape, &d));
  SSD_TRY(check_dtype(in));
  SSD_TRY(check_dtype(y_dtype));
  SSD_TRY(check_mma(mma));
  if (!x || !dt || !A || !Bm || !Cm || !D || !y || !seq_idx) return SSD_ERR_NULL;
  if (nseq < 0 || nseq > 0x7fffffff / (d.H * ((d.N + 31) / 32) * ((d.P + 31) / 32))) return SSD_ERR_SHAPE;
  if (nseq > 0 && (!seq_last || !seq_states)) return SSD_ERR_NULL;
  if (!workspace) return SSD_ERR_WORKSPACE;
  const WsLayout ws = workspace_layout(d);
  if (workspace_bytes < ws.total_varlen) return SSD_ERR_WORKSPACE;
  if (nseq > 0 && (!aligned16(seq_last) || !aligned16(seq_states))) return SSD_ERR_ALIGN;
  if (!aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(D) ||
      !aligned16(y) || !aligned16(seq_idx) || !aligned16(workspace) ||
      (initial_states && !aligned16(initial_states)) || (final_states && !aligned16(final_states)))
    return SSD_ERR_ALIGN;
  if (ssd::chunk_state_lds_bytes(d, mma == SSD_MMA_F32) > kLdsLimit ||
      ssd::chunk_scan_lds_bytes(d, mma == SSD_MMA_F32) > kLdsLimit)
    return SSD_ERR_UNSUPPORTED;

  char* base = static_cast<char*>(workspace);
  float* dA = reinterpret_cast<float*>(base + ws.dA_off);
  float* dtb = reinterpret_cast<float*>(base + ws.dt_off);
  float* st = reinterpret_cast<float*>(base + ws.st_off);
  int* sst = reinterpret_cast<int*>(base + ws.ss_off);
  float* dAp = reinterpret_cast<float*>(base + ws.dAp_off);
  float* dtl = reinterpret_cast<float*>(base + ws.dtl_off);
  const hipStream_t s = (hipStream_t)stream;
  const bool bf = in == SSD_BF16, f32m = mma == SSD_MMA_F32;

  // the two-kernel state path, fed with the packed-sequence masks: chunk
  // states of each chunk's last sequence only, and a state passing that
  // restarts where a sequence starts inside a chunk.  With bf16 inputs and
  // operands one chunk-state kernel also takes the cumulative sums, the
  // sequence starts and both masks; otherwise three small steps come first.
  const bool fused = bf && !f32m && ssd::chunk_state_hg_varlen_supported(d);
  if (!fused) {
    SSD_TRY(from_hip(ssd::launch_chunk_cumsum(d, dt, A, dA, dtb, s)));
    SSD_TRY(from_hip(ssd::launch_seq_start(d, seq_idx, sst, s)));
    SSD_TRY(from_hip(ssd::launch_varlen_prep(d, dA, dtb, sst, dAp, dtl, s)));
  }
  // As in ssd_forward: with bf16 matrix operands the chunk states pass
  // through memory as bf16 and the state passing writes the carried states in
  // place over them as bf16 (the values the chunk scan uses as operands, and
  // the incoming state of the per-sequence states); fp32 throughout with fp32
  // operands.  The recurrence and the final states stay fp32.
  if (!f32m) {
    uint16_t* sb = reinterpret_cast<uint16_t*>(base + ws.hb_off);
    if (fused)
      SSD_TRY(from_hip(ssd::launch_chunk_state_cumsum_hg_varlen(d, x, Bm, dt, A, seq_idx, dA, dtb, sst, dAp, sb, s)));
    else
      SSD_TRY(from_hip(ssd::launch_chunk_state_any(d, x, Bm, bf, dtl, dA, sb, true, f32m, s)));
    SSD_TRY(from_hip(ssd::launch_state_passing_any(d, sb, true, sb, true, dAp, initial_states, final_states, s)));
    SSD_TRY(from_hip(
        ssd::launch_varlen_states(d, x, Bm, bf, dtb, dA, sst, sb, true, nseq, seq_last, seq_states, f32m, s)));
  } else {
    SSD_TRY(from_hip(ssd::launch_chunk_state(d, x, Bm, bf, dtl, dA, st, f32m, s)));
    SSD_TRY(from_hip(ssd::launch_state_passing(d, st, st, dAp, initial_states, final_states, s)));
    SSD_TRY(from_hip(
        ssd::launch_varlen_states(d, x, Bm, bf, dtb, dA, sst, st, false, nseq, seq_last, seq_states, f32m, s)));
  }
  const void* car = f32m ? static_cast<const void*>(st) : static_cast<const void*>(base + ws.hb_off);
  SSD_TRY(from_hip(ssd::launch_chunk_scan(d, x, Bm, Cm, bf, dtb, dA, car, !f32m, D, y, y_dtype == SSD_BF16, f32m, s,
                                          sst)));
  return SSD_OK;
}

size_t ssd_backward_workspace_bytes(const ssd_shape* shape) {
  Dims d;
  if (check_shape(shape, &d) != SSD_OK) return 0;
  return ssd::backward_workspace_bytes(d);
}

ssd_status ssd_backward(const ssd_shape* shape, const void* x, const float* dt, const float* A, const void* Bm,
                        const void* Cm, const float* D, ssd_dtype in, const float* initial_states, const void* dy,
                        ssd_dtype dy_dtype, const float* dfinal, float* dx, float* ddt, float* dA, float* dB,
                        float* dC, float* dD, float* dinitial, void* workspace, size_t workspace_bytes,
                        ssd_mma mma, void* stream) {
  Dims d;
  SSD_TRY(check_shape(shape, &d));
  SSD_TRY(check_dtype(in));
  SSD_TRY(check_dtype(dy_dtype));
  SSD_TRY(check_mma(mma));
  if (!x || !dt || !A || !Bm || !Cm || !D || !dy || !dx || !ddt || !dA || !dB || !dC || !dD) return SSD_ERR_NULL;
  if (!workspace) return SSD_ERR_WORKSPACE;
  if (workspace_bytes < ssd::backward_workspace_bytes(d)) return SSD_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(dt) || !aligned16(A) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(D) ||
      !aligned16(dy) || !aligned16(dx) || !aligned16(ddt) || !aligned16(dA) || !aligned16(dB) || !aligned16(dC) ||
      !aligned16(dD) || !aligned16(workspace) || (initial_states && !aligned16(initial_states)) ||
      (dfinal && !aligned16(dfinal)) || (dinitial && !aligned16(dinitial)))
    return SSD_ERR_ALIGN;
  const bool f32m = mma == SSD_MMA_F32;
  if (ssd::chunk_state_lds_bytes(d, f32m) > kLdsLimit || ssd::chunk_scan_lds_bytes(d, f32m) > kLdsLimit ||
      !ssd::bwd_dbc_supported(d) || ssd::bwd_dbc_lds_bytes(d, f32m) > kLdsLimit)
    return SSD_ERR_UNSUPPORTED;
  // elementwise launches of 256 threads per block over B*L*H*max(P,N) elements
  const int64_t wide = d.P > d.N ? d.P : d.N;
  if (d.B * d.L * d.H > (int64_t(1) << 39) / wide) return SSD_ERR_UNSUPPORTED;
  return from_hip(ssd::launch_backward(d, x, dt, A, Bm, Cm, D, in == SSD_BF16, initial_states, dy,
                                       dy_dtype == SSD_BF16, dfinal, dx, ddt, dA, dB, dC, dD, dinitial, f32m,
                                       workspace, (hipStream_t)stream));
}

const char* ssd_status_string(ssd_status status) {
  switch (status) {
    case SSD_OK: return "SSD_OK: success";
    case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE: a size is not positive or nheads is not a multiple of ngroups";
    case SSD_ERR_DTYPE: return "SSD_ERR_DTYPE: unknown dtype or mma mode";
    case SSD_ERR_UNSUPPORTED:
      return "SSD_ERR_UNSUPPORTED: shape outside this version's limits (P, N multiples of 16 and <= 256; "
             "chunk in {32,64,128,256})";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or smaller than ssd_workspace_bytes";
    case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: a pointer is not 16-byte aligned";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: a HIP kernel launch failed";
    case SSD_ERR_SCRATCH:
      return "SSD_ERR_SCRATCH: the shape needs more workspace than ssd_forward_noalloc's static scratch array "
             "(SSD_NOALLOC_SCRATCH_BYTES) holds";
  }
  return "unknown ssd_status";
}

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

}  // extern "C"
