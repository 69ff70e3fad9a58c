// Measurement probe (not part of the BoB path): the float32 atomic traffic of the
// schedule that would form gQ in pass 2 instead of pass 1.
//
// In that schedule (the alternative to the two-pass design of the FlashBoB review
// page, Summary), pass 2 walks the query tiles of a 128-key tile and every step adds a
// 32 x d tile of gQ contributions, dS UK + Sbar K over its keys, into float32 gQ with
// hardware atomics: keys are split over workgroups, so no workgroup sees a query's whole
// sum. Even with the four waves of a workgroup summing their tiles first (through LDS),
// that is 32 d additions per (key tile, query tile) pair. The probe issues exactly
// those additions, with pass 2's grid (key tiles x heads x splits, each split taking its
// share of the query tiles in order) and no arithmetic besides them, so its time is a
// lower bound on what the atomics alone would add to that schedule.
#include "common.hpp"
#include "kernels.hpp"

namespace fb {

__global__ __launch_bounds__(kBlock) void probe_gq_atomics_kernel(float* __restrict__ gq, int N, int d, int nsplit) {
  const int bh = blockIdx.y, split = blockIdx.z;
  const int nqt = (N + kTile - 1) / kTile;
  const int it_begin = (int)((long long)split * nqt / nsplit);
  const int it_end = (int)((long long)(split + 1) * nqt / nsplit);
  const int per_thread = kTile * d / kBlock;  // 8 at d = 64, 16 at d = 128
  float* head = gq + (size_t)bh * N * d;
  for (int it = it_begin; it < it_end; ++it) {
    const int q0 = it * kTile;
    for (int k = 0; k < per_thread; ++k) {
      const int e = k * kBlock + (int)threadIdx.x;  // consecutive threads: consecutive columns
      const int row = q0 + e / d;
      if (row < N) unsafeAtomicAdd(head + (size_t)row * d + e % d, 1.0f);
    }
  }
}

hipError_t launch_probe_gq_atomics(float* gq, int BH, int N, int d, int nsplit, hipStream_t s) {
  hipLaunchKernelGGL(probe_gq_atomics_kernel, dim3(row_tiles(N), BH, nsplit), dim3(kBlock), 0, s, gq, N, d,
                     nsplit);
  return hipGetLastError();
}

}  // namespace fb
