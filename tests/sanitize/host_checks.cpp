// Host-only driver for the C ABI's argument checks, workspace sizing and error
// reporting, built with AddressSanitizer and UndefinedBehaviorSanitizer on the
// CPU (tests/test_host_sanitizers.py). The kernel launch functions are replaced
// by stubs that touch no memory and report an error, so any call that passes its
// checks ends with FB_ERR_HIP instead of a launch; no GPU is needed.
#include <climits>
#include <cstdio>
#include <cstring>

#include "flashbob.h"
#include "kernels.hpp"

namespace fb {
#define FB_STUB(sig) \
  hipError_t sig { return hipErrorInvalidValue; }
FB_STUB(launch_attn_fwd(const FwdArgs&, DT, int, bool, int, hipStream_t))
FB_STUB(launch_attn_fwd_combine(const FwdArgs&, DT, int, hipStream_t))
FB_STUB(launch_pass1(const Pass1Args&, DT, int, bool, hipStream_t))
FB_STUB(launch_pass1_d64(const Pass1Args&, DT, bool, hipStream_t))
FB_STUB(launch_pass1_combine(const Pass1Args&, DT, int, hipStream_t))
FB_STUB(launch_pass1_q16(const Pass1Args&, DT, bool, hipStream_t))
FB_STUB(launch_pass1_q16_combine(const Pass1Args&, DT, hipStream_t))
FB_STUB(launch_fourpass_sweep(const Pass1Args&, int, DT, int, bool, hipStream_t))
FB_STUB(launch_first_bwd_dq(const Pass1Args&, DT, int, bool, hipStream_t))
FB_STUB(launch_first_bwd_dkdv(const Pass2Args&, DT, int, bool, hipStream_t))
FB_STUB(launch_pass2(const Pass2Args&, DT, int, bool, hipStream_t))
FB_STUB(launch_pass2_d128(const Pass2Args&, DT, hipStream_t))
FB_STUB(launch_pass2_reduce(const Pass2Args&, DT, int, hipStream_t))
FB_STUB(launch_pass2_convert(const Pass2Args&, DT, int, hipStream_t))
hipError_t launch_zero_f32(float*, size_t, hipStream_t) { return hipErrorInvalidValue; }
FB_STUB(launch_bwd_rowdot(const BwdArgs&, DT, int, int, hipStream_t))
FB_STUB(launch_bwd_dq(const BwdArgs&, DT, int, bool, int, hipStream_t))
FB_STUB(launch_bwd_dkdv(const BwdArgs&, DT, int, bool, int, hipStream_t))
FB_STUB(launch_probe_gq_atomics(float*, int, int, int, int, hipStream_t))
#undef FB_STUB
}  // namespace fb

static int failures = 0;

// pass1_asm_step_count over every sweep of many shapes: the scheduled block computes only
// whole key blocks that no query of its workgroup precedes, copies only whole blocks,
// and stops at a stage boundary unless it runs the whole sweep.
static int check_asm_step_counts() {
  int bad = 0;
  const int slots = 4, ahead = 3;
  for (int N = 1; N <= 1300; N += (N < 300 ? 1 : 37)) {
    for (int causal = 0; causal < 2; ++causal) {
      for (int nsplit = 1; nsplit <= 9; ++nsplit) {
        for (int qt = 0; qt < fb::row_tiles(N); ++qt) {
          int nkt = (N + 31) / 32;
          if (causal) nkt = nkt < (qt + 1) * 4 ? nkt : (qt + 1) * 4;
          for (int split = 0; split < nsplit; ++split) {
            const int kt_begin = (int)((long long)split * nkt / nsplit);
            const int kt_end = (int)((long long)(split + 1) * nkt / nsplit);
            const int nsteps = kt_end - kt_begin;
            const int n = fb::pass1_asm_step_count(N, causal != 0, qt, kt_begin, nsteps, slots, ahead);
            bool ok = n >= 0 && n <= nsteps && (n == nsteps || n % slots == 0);
            for (int j = 0; ok && j < n; ++j) {
              const int kt = kt_begin + j;
              ok = (kt + 1) * 32 <= N && (!causal || kt * 32 + 31 < qt * 128);
              if (ok && j + ahead < nsteps) ok = (kt_begin + j + ahead + 1) * 32 <= N;  // the block's copy
            }
            if (!ok && bad++ < 5)
              std::printf("FAIL asm step count: N=%d causal=%d nsplit=%d qt=%d split=%d -> %d of %d\n", N, causal,
                          nsplit, qt, split, n, nsteps);
          }
        }
      }
    }
  }
  return bad;
}
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::printf("FAIL line %d: %s (%s)\n", __LINE__, #cond, fb_last_error()); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static void* fake(int i) { return reinterpret_cast<void*>(0x100000 + 0x1000 * (size_t)i); }

static fb_status_t bob_ws(int B, int H, int N, int d, fb_dtype_t dt, float tau, void* ws, size_t ws_bytes) {
  return bob_attention_ws(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), tau, 0, B, H, N, d, dt,
                          fake(7), fake(8), fake(9), fake(10), ws, ws_bytes, nullptr);
}

int main() {
  failures += check_asm_step_counts();
  const fb_dtype_t dts[3] = {FB_F32, FB_F16, FB_BF16};
  const int ns[] = {1, 2, 31, 32, 33, 127, 128, 129, 1000, 16384, 262144, 1 << 22, INT_MAX - 255, INT_MAX - 127,
                    INT_MAX, -1, 0, INT_MIN};
  const int bhs[][2] = {{1, 1}, {8, 12}, {65535, 1}, {1, 65535}, {256, 256}, {0, 1}, {-3, 2}};
  // workspace sizing over extreme shapes: never crashes, 0 exactly when invalid
  for (fb_dtype_t dt : dts)
    for (int d : {32, 64, 96, 128})
      for (auto& bh : bhs)
        for (int n : ns)
          for (int s1 : {0, 1, 64}) {
            EXPECT(fb_set_tuning(s1, s1) == FB_OK);
            const size_t w = bob_workspace_bytes(bh[0], bh[1], n, d, dt);
            const long long rows = (long long)bh[0] * bh[1] * n;
            const bool valid = (d == 64 || d == 128) && bh[0] >= 1 && bh[1] >= 1 && n >= 1 &&
                               (long long)bh[0] * bh[1] <= 65535 && rows <= INT_MAX - 255;
            EXPECT((w != 0) == valid);
            if (valid) EXPECT(w >= (size_t)rows * d * (dt == FB_F32 ? 4 : 2));
          }
  EXPECT(fb_set_tuning(0, 0) == FB_OK);
  EXPECT(fb_set_tuning(-1, 0) == FB_ERR_ARG);
  EXPECT(fb_set_tuning(0, 65) == FB_ERR_ARG);
  EXPECT(std::strlen(fb_last_error()) > 0);
  EXPECT(fb_set_reduction(3) == FB_ERR_ARG);
  EXPECT(fb_set_reduction(-1) == FB_ERR_ARG);
  for (int mode = 0; mode < 3; ++mode) {  // workspace sizing in every reduction mode
    EXPECT(fb_set_reduction(mode) == FB_OK);
    EXPECT(fb_set_tuning(0, 4) == FB_OK);
    EXPECT(bob_workspace_bytes(1, 1, 16384, 64, FB_BF16) > 0);
    EXPECT(bob_workspace_bytes(1, 1, INT_MAX - 255, 128, FB_F16) > 0);
  }
  EXPECT(fb_set_reduction(0) == FB_OK);
  // the measurement probe: argument checks, then the (stubbed) launch
  {
    alignas(16) float gq[4];
    EXPECT(fb_probe_gq_atomics(nullptr, 1, 1, 256, 64, 1, nullptr) == FB_ERR_NULL);
    EXPECT(fb_probe_gq_atomics(gq, 1, 1, 256, 64, 0, nullptr) == FB_ERR_ARG);
    EXPECT(fb_probe_gq_atomics(gq, 1, 1, INT_MAX, 64, 1, nullptr) == FB_ERR_SHAPE);
    EXPECT(fb_probe_gq_atomics(gq, 1, 1, 256, 64, 1, nullptr) == FB_ERR_HIP);
  }
  EXPECT(fb_set_tuning(0, 0) == FB_OK);

  // argument checks of the workspace entry point
  EXPECT(bob_ws(1, 1, 128, 96, FB_BF16, 0.125f, fake(20), 1u << 30) == FB_ERR_HEADDIM);
  EXPECT(bob_ws(1, 1, INT_MAX, 64, FB_BF16, 0.125f, fake(20), 1u << 30) == FB_ERR_SHAPE);
  EXPECT(bob_ws(1, 1, 128, 64, (fb_dtype_t)3, 0.125f, fake(20), 1u << 30) == FB_ERR_DTYPE);
  EXPECT(bob_ws(1, 1, 128, 64, FB_BF16, 1.f / 0.f, fake(20), 1u << 30) == FB_ERR_ARG);
  EXPECT(bob_ws(1, 1, 128, 64, FB_BF16, 0.125f, nullptr, 1u << 30) == FB_ERR_WORKSPACE);
  EXPECT(bob_ws(1, 1, 128, 64, FB_BF16, 0.125f, fake(20), 64) == FB_ERR_WORKSPACE);
  // valid arguments reach the (stubbed) launch, which reports a HIP error
  EXPECT(bob_ws(1, 1, 128, 64, FB_BF16, 0.125f, fake(20), 1u << 30) == FB_ERR_HIP);
  EXPECT(std::strstr(fb_last_error(), "attn_fwd_stats") != nullptr);

  // allocation cap: refused before any HIP call
  EXPECT(fb_set_alloc_limit(4096) == FB_OK);
  EXPECT(bob_attention(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), 0.125f, 1, 2, 3, 4096, 128,
                       FB_F16, fake(7), fake(8), fake(9), fake(10), nullptr) == FB_ERR_OOM);
  EXPECT(attn_bwd(fake(0), fake(1), fake(2), fake(3), fake(4), (const float*)fake(5), 0.125f, 0, 1, 1, 4096, 64,
                  FB_BF16, fake(6), fake(7), fake(8), nullptr, nullptr) == FB_ERR_OOM);
  EXPECT(fb_set_alloc_limit(0) == FB_OK);

  // other entry points' checks
  EXPECT(attn_fwd(fake(0), fake(1), fake(2), nullptr, 0.125f, 0, 1, 1, 64, 64, FB_BF16, fake(3), (float*)fake(4),
                  (float*)fake(5), nullptr) == FB_ERR_NULL);
  EXPECT(attn_fwd(fake(0), fake(1), fake(2), nullptr, 0.125f, 0, 1, 1, 64, 64, FB_BF16, fake(0), (float*)fake(4),
                  nullptr, nullptr) == FB_ERR_ARG);
  EXPECT(bob_attention_with_stats(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), fake(7),
                                  (const float*)fake(8), (const float*)((char*)fake(9) + 2), 0.125f, 0, 1, 1, 64, 64,
                                  FB_BF16, fake(10), fake(11), fake(12), fake(13), nullptr, nullptr, fake(20),
                                  1u << 30, nullptr) == FB_ERR_ARG);
  EXPECT(bob_attention_fourpass_ws(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), fake(6), 0.125f, 0, 1, 1,
                                   64, 64, FB_F32, fake(7), fake(8), fake(9), fake(10), fake(20), 1u << 30,
                                   nullptr) == FB_ERR_DTYPE);

  // timing interface with nothing recorded
  fb_profile_start("bob_pass1");
  fb_kernel_time_t t[4];
  EXPECT(fb_profile_stop(t, 4) == 0);
  fb_profile_start(nullptr);
  EXPECT(fb_profile_stop(nullptr, 0) == 0);

  std::printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
