// abi_stubs.cpp -- stand-ins for the device-side launchers of the SSD library,
// for a host-only build of ssd_api.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure; never part of the library).
// The sanitizer driver only makes calls whose arguments fail validation, so no
// launcher may ever be reached: each one aborts.  The shape-policy queries
// return fixed values that let validation run to its end.
#include <cstdio>
#include <cstdlib>

#include "ssd_launch.hpp"

namespace ssd {

[[noreturn]] static void reached(const char* what) {
  std::fprintf(stderr, "launcher reached on arguments that should have been rejected: %s\n", what);
  std::abort();
}

size_t chunk_state_lds_bytes(const Dims&, bool) { return 0; }
size_t chunk_scan_lds_bytes(const Dims&, bool) { return 0; }
bool chunk_state_hg_supported(const Dims&, bool, bool) { return false; }
bool chunk_scan_hg_supported(const Dims&, bool, bool) { return false; }
bool state_fused_supported(const Dims&, bool, bool) { return false; }
bool fwd_fused_supported(const Dims&, bool, bool) { return false; }
int64_t state_fused_blocks(const Dims& d) { return d.B * d.H; }
bool decode_step_supported(int64_t P) { return P % 4 == 0 && P <= 1024; }
size_t backward_workspace_bytes(const Dims& d) { return (size_t)(d.B * d.H) * 4096; }
bool bwd_dbc_supported(const Dims& d) { return d.N % 16 == 0 && d.P % 16 == 0; }
size_t bwd_dbc_lds_bytes(const Dims&, bool) { return 0; }

hipError_t launch_chunk_cumsum(const Dims&, const float*, const float*, float*, float*, hipStream_t) {
  reached("chunk_cumsum");
}
hipError_t launch_seq_start(const Dims&, const int*, int*, hipStream_t) { reached("seq_start"); }
hipError_t launch_fwd_fused(const Dims&, const void*, const void*, const void*, const float*, const float*,
                            const float*, const float*, void*, bool, float*, hipStream_t) {
  reached("fwd_fused");
}
hipError_t launch_varlen_prep(const Dims&, const float*, const float*, const int*, float*, float*, hipStream_t) {
  reached("varlen_prep");
}
hipError_t launch_chunk_state(const Dims&, const void*, const void*, bool, const float*, const float*, float*, bool,
                              hipStream_t) {
  reached("chunk_state");
}
hipError_t launch_chunk_state_any(const Dims&, const void*, const void*, bool, const float*, const float*, void*, bool,
                                  bool, hipStream_t) {
  reached("chunk_state_any");
}
hipError_t launch_chunk_state_hg(const Dims&, const void*, const void*, const float*, const float*, void*, bool, bool,
                                 hipStream_t) {
  reached("chunk_state_hg");
}
hipError_t launch_chunk_state_cumsum_hg(const Dims&, const void*, const void*, const float*, const float*, float*,
                                        float*, void*, bool, bool, hipStream_t) {
  reached("chunk_state_cumsum_hg");
}
bool chunk_state_hg_varlen_supported(const Dims&) { return false; }
hipError_t launch_chunk_state_cumsum_hg_varlen(const Dims&, const void*, const void*, const float*, const float*,
                                               const int*, float*, float*, int*, float*, void*, hipStream_t) {
  reached("chunk_state_cumsum_hg_varlen");
}
hipError_t launch_state_passing(const Dims&, const float*, float*, const float*, const float*, float*, hipStream_t) {
  reached("state_passing");
}
hipError_t launch_state_passing_bf16(const Dims&, const float*, uint16_t*, const float*, const float*, float*,
                                     hipStream_t) {
  reached("state_passing_bf16");
}
hipError_t launch_state_passing_any(const Dims&, const void*, bool, void*, bool, const float*, const float*, float*,
                                    hipStream_t) {
  reached("state_passing_any");
}
hipError_t launch_state_fused(const Dims&, const void*, const void*, const float*, const float*, const float*, void*,
                              bool, float*, hipStream_t) {
  reached("state_fused");
}
hipError_t launch_chunk_scan_hg(const Dims&, const void*, const void*, const void*, bool, const float*, const float*,
                                const void*, bool, const float*, void*, bool, bool, hipStream_t, const int*) {
  reached("chunk_scan_hg");
}
hipError_t launch_chunk_scan(const Dims&, const void*, const void*, const void*, bool, const float*, const float*,
                             const void*, bool, const float*, void*, bool, bool, hipStream_t, const int*) {
  reached("chunk_scan");
}
hipError_t launch_varlen_states(const Dims&, const void*, const void*, bool, const float*, const float*, const int*,
                                const void*, bool, int64_t, const int64_t*, float*, bool, hipStream_t) {
  reached("varlen_states");
}
hipError_t launch_decode_step(int64_t, int64_t, int64_t, int64_t, int64_t, const void*, const float*, const float*,
                              const void*, const void*, const float*, bool, float*, void*, bool, hipStream_t) {
  reached("decode_step");
}
hipError_t launch_backward(const Dims&, const void*, const float*, const float*, const void*, const void*,
                           const float*, bool, const float*, const void*, bool, const float*, float*, float*, float*,
                           float*, float*, float*, float*, bool, void*, hipStream_t) {
  reached("backward");
}

}  // namespace ssd
