// abi_driver.cpp -- drives the C ABI's host-side validation and size
// arithmetic (ssd_api.cpp) over many shapes, extreme values included, in a
// build under AddressSanitizer and UndefinedBehaviorSanitizer (test
// infrastructure).  Every call is made with arguments that must be rejected
// before any launch (the launchers are stubs that abort), and the statuses
// must agree with the shape's validity as the workspace queries report it.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "ssd.h"

static uint64_t g_state = 0x243F6A8885A308D3ull;
static uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static int g_fail = 0;
#define EXPECT(cond, ...)                       \
  do {                                          \
    if (!(cond)) {                              \
      std::fprintf(stderr, __VA_ARGS__);        \
      std::fprintf(stderr, "\n");               \
      if (++g_fail > 20) std::exit(1);          \
    }                                           \
  } while (0)

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 100000;
  const int64_t extreme[] = {INT64_MIN, -(int64_t(1) << 40), -1, 0, 1, 3, 15, 17, 255, 257, 4097,
                             65535, 65536, int64_t(1) << 24, int64_t(1) << 31, int64_t(1) << 40,
                             int64_t(1) << 62, INT64_MAX};
  const int64_t sane[7][5] = {{1, 2, 8, 65535, 3},        {1, 255, 256, 8192, 300},
                              {1, 4, 80, 32767, 64},      {16, 64, 144, 256, 48},
                              {16, 64, 128, 256, 32},     {1, 2, 4, 80, 64},
                              {32, 64, 128, 256, 64}};
  void* F = reinterpret_cast<void*>(uintptr_t(0x100000));
  void* MIS = reinterpret_cast<void*>(uintptr_t(0x100004));  // not 16-byte aligned
  const ssd_dtype BAD_DT = static_cast<ssd_dtype>(99);
  const ssd_mma BAD_MMA = static_cast<ssd_mma>(99);
  long nvalid = 0;
  for (long it = 0; it < iters; ++it) {
    int64_t v[7];
    for (int f = 0; f < 7; ++f) {
      const uint64_t r = next_u64();
      v[f] = (r & 7) == 0 ? extreme[(r >> 3) % (sizeof(extreme) / sizeof(extreme[0]))] : sane[f][(r >> 3) % 5];
    }
    ssd_shape s = {v[0], v[1], v[2], v[3], v[4], v[5], v[6]};
    const size_t w = ssd_workspace_bytes(&s);
    const size_t wv = ssd_workspace_bytes_varlen(&s);
    const size_t wb = ssd_backward_workspace_bytes(&s);
    const bool valid = w > 0;
    nvalid += valid;
    EXPECT((wv > 0) == valid && (wb > 0) == valid, "workspace queries disagree on validity");
    EXPECT(!valid || wv >= w, "varlen workspace smaller than the forward's");
    const int sc = ssd_chunk_cumsum(&s, static_cast<const float*>(F), static_cast<const float*>(F), nullptr,
                                    nullptr, nullptr);
    EXPECT(valid ? sc == SSD_ERR_NULL : (sc == SSD_ERR_SHAPE || sc == SSD_ERR_UNSUPPORTED),
           "cumsum status %d (valid %d)", sc, (int)valid);
    const int want = valid ? SSD_ERR_DTYPE : sc;
    const float* Ff = static_cast<const float*>(F);
    float* Fw = static_cast<float*>(F);
    int st;
    st = ssd_chunk_state(&s, F, F, BAD_DT, Ff, Ff, F, SSD_F32, SSD_MMA_BF16, nullptr);
    EXPECT(st == want, "chunk_state %d want %d", st, want);
    st = ssd_chunk_cumsum_state(&s, F, F, BAD_DT, Ff, Ff, Fw, Fw, F, SSD_F32, SSD_MMA_BF16, nullptr);
    EXPECT(st == want, "chunk_cumsum_state %d want %d", st, want);
    st = ssd_state_passing(&s, F, BAD_DT, F, SSD_F32, Ff, nullptr, Fw, nullptr);
    EXPECT(st == want, "state_passing %d want %d", st, want);
    st = ssd_chunk_scan(&s, F, F, F, BAD_DT, Ff, Ff, F, SSD_F32, Ff, F, SSD_F32, SSD_MMA_BF16, nullptr);
    EXPECT(st == want, "chunk_scan %d want %d", st, want);
    st = ssd_chunk_scan(&s, F, F, F, SSD_BF16, Ff, Ff, F, SSD_F32, Ff, F, SSD_F32, BAD_MMA, nullptr);
    EXPECT(st == want, "chunk_scan (mma) %d want %d", st, want);
    st = ssd_chunk_state_passing(&s, F, F, BAD_DT, Ff, Ff, nullptr, F, SSD_BF16, Fw, SSD_MMA_BF16, nullptr);
    EXPECT(st == want, "chunk_state_passing %d want %d", st, want);
    st = ssd_forward(&s, F, Ff, Ff, F, F, Ff, BAD_DT, nullptr, F, SSD_BF16, Fw, F, ~size_t(0), SSD_MMA_BF16, nullptr);
    EXPECT(st == want, "forward %d want %d", st, want);
    st = ssd_forward_varlen(&s, F, Ff, Ff, F, F, Ff, BAD_DT, static_cast<const int32_t*>(F), nullptr, F, SSD_BF16,
                            Fw, 0, nullptr, nullptr, F, ~size_t(0), SSD_MMA_BF16, nullptr);
    EXPECT(st == want, "forward_varlen %d want %d", st, want);
    st = ssd_backward(&s, F, Ff, Ff, F, F, Ff, BAD_DT, nullptr, F, SSD_F32, nullptr, Fw, Fw, Fw, Fw, Fw, Fw, nullptr,
                      F, ~size_t(0), SSD_MMA_F32, nullptr);
    EXPECT(st == want, "backward %d want %d", st, want);
    st = ssd_decode_step(&s, F, Ff, Ff, F, F, Ff, BAD_DT, Fw, F, SSD_F32, nullptr);
    EXPECT(st != SSD_OK && st != SSD_ERR_HIP, "decode_step %d", st);
    if (valid) {
      // valid shape and dtypes: a workspace one byte short, a NULL workspace
      // and a misaligned input are each rejected before any launch
      for (int m = 0; m < 2; ++m) {
        const ssd_mma mma = m ? SSD_MMA_F32 : SSD_MMA_BF16;
        st = ssd_forward(&s, F, Ff, Ff, F, F, Ff, SSD_BF16, nullptr, F, SSD_BF16, Fw, F, 255, mma, nullptr);
        EXPECT(st == SSD_ERR_WORKSPACE, "forward, short workspace: %d", st);
        st = ssd_forward(&s, F, Ff, Ff, F, F, Ff, SSD_BF16, nullptr, F, SSD_BF16, Fw, nullptr, w, mma, nullptr);
        EXPECT(st == SSD_ERR_WORKSPACE, "forward, NULL workspace: %d", st);
        st = ssd_forward(&s, MIS, Ff, Ff, F, F, Ff, SSD_BF16, nullptr, F, SSD_BF16, Fw, F, w, mma, nullptr);
        EXPECT(st == SSD_ERR_ALIGN, "forward, misaligned x: %d", st);
      }
      st = ssd_forward_varlen(&s, F, Ff, Ff, F, F, Ff, SSD_BF16, static_cast<const int32_t*>(F), nullptr, F,
                              SSD_BF16, Fw, 0, nullptr, nullptr, F, wv - 1, SSD_MMA_BF16, nullptr);
      EXPECT(st == SSD_ERR_WORKSPACE || st == SSD_ERR_SHAPE, "forward_varlen, short workspace: %d", st);
      st = ssd_backward(&s, F, Ff, Ff, F, F, Ff, SSD_BF16, nullptr, F, SSD_F32, nullptr, Fw, Fw, Fw, Fw, Fw, Fw,
                        nullptr, F, wb - 1, SSD_MMA_F32, nullptr);
      EXPECT(st == SSD_ERR_WORKSPACE, "backward, short workspace: %d", st);
    }
  }
  for (int c = -3; c < 12; ++c) EXPECT(ssd_status_string(static_cast<ssd_status>(c & 7)) != nullptr, "status string");
  EXPECT(ssd_workspace_bytes(nullptr) == 0 && ssd_chunk_cumsum(nullptr, nullptr, nullptr, nullptr, nullptr,
                                                                nullptr) == SSD_ERR_NULL, "NULL shape");
  std::printf("abi_driver: %ld shapes (%ld valid), %d mismatches\n", iters, nvalid, g_fail);
  return g_fail ? 1 : 0;
}
