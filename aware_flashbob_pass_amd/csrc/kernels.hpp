// Launch interfaces between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fb {

constexpr int kBlock = 256;     // 4 waves per workgroup
constexpr int kBlockRows = 128; // resident rows per workgroup (32 per wave)

enum class DT { F32 = 0, F16 = 1, BF16 = 2 };

// Statistics kernel: O, L (natural-log row LSE) and optionally D = rowsum(dO * O).
struct FwdArgs {
  const void *Q, *K, *V, *dO;
  void* O;
  float* L;
  float* D;  // null: skip D
  float tau;
  int N;
  int BH = 1;
  int nsplit = 1;
  float* part = nullptr;  // split records (nsplit > 1)
};

// Pass 1 (query-tile parallel): gQ, gdO, alpha, E; or per-split partials.
struct Pass1Args {
  const void *Q, *K, *V, *dO, *UQ, *UK, *UV, *O;
  const float *L, *D;
  void *gQ, *gdO;
  float *alpha, *E;
  float *l2, *c;  // per query for pass 2: L log2(e) and c = alpha D + E
  float* part;    // split records (nsplit > 1)
  float tau;
  int N, BH, nsplit;
  // Pass 2's merge counters ([B*H][row_tiles(N)]), zeroed by pass 1 for the
  // last-arriving-workgroup reduction (null otherwise).
  unsigned* p2_counters = nullptr;
};

// How pass 2 combines the partial gK, gV of a split query range.
enum Reduce : int {
  kReduceRecords = 0,    // per-split records, summed in split order by a merge kernel
  kReduceAtomic = 1,     // float32 atomic additions into acc32, then a conversion kernel
  kReduceLastBlock = 2,  // records; the last workgroup of a key tile to finish sums them
};

// Pass 2 (key-tile parallel): gK, gV; or per-split partials.
struct Pass2Args {
  const void *Q, *K, *V, *dO, *UQ, *UK, *UV;
  const float *L, *D, *alpha, *E;
  const float *l2, *c;  // L log2(e), c = alpha D + E (written by pass 1; staged 16-bit kernel)
  void *gK, *gV;
  float* part;
  float tau;
  int N, BH, nsplit;
  int reduce = kReduceRecords;  // with nsplit > 1 (16-bit BoB sweeps)
  float* acc32 = nullptr;       // kReduceAtomic: [2][B*H][N][d] float32 (gK / tau, gV), zeroed first
  unsigned* counters = nullptr; // kReduceLastBlock: [B*H][row_tiles(N)], zero on entry
};

// First backward: D = rowsum(dO * O), then dQ (query-parallel) and dK, dV (key-parallel).
struct BwdArgs {
  const void *Q, *K, *V, *O, *dO;
  const float* L;
  float* D;
  void *dQ, *dK, *dV;
  float tau;
  int N;
};

// Float count of one wave's partial record.
__host__ __device__ inline size_t pass1_record_floats(int d) { return (size_t)(4 * (d / 32) * 16 + 2) * 64; }
__host__ __device__ inline size_t fwd_record_floats(int d) { return (size_t)((d / 32) * 16 + 2) * 64; }
__host__ __device__ inline size_t pass2_record_floats(int d) { return (size_t)(2 * (d / 32) * 16) * 64; }
__host__ __device__ inline int row_tiles(int N) { return (N + kBlockRows - 1) / kBlockRows; }

// Steps of pass 1's scheduled block (the d = 64 bf16 sweep with tau folded) for the
// workgroup of query tile qt sweeping key blocks [kt_begin, kt_begin + nsteps) of 32
// keys, with `slots` LDS stages and copies `ahead` steps ahead. The block takes steps
// that need no mask: key blocks before the workgroup's first query (causal) and whole
// blocks of 32 keys. Its direct copies do not clamp rows past N, so none of them may
// reach a ragged last block either: the block stops `ahead` steps before it, and the
// compiled steps, whose copies clamp, issue that block's copy. It runs every step when
// none needs a mask, else a multiple of `slots` so the compiled steps start at stage 0.
__host__ __device__ inline int pass1_asm_step_count(int N, bool causal, int qt, int kt_begin, int nsteps, int slots,
                                                    int ahead) {
  const int whole = N / 32;  // whole 32-key blocks
  int n = nsteps;
  if (causal) n = qt * (kBlockRows / 32) - kt_begin;
  if (whole < kt_begin + nsteps) n = n < whole - kt_begin - ahead ? n : whole - kt_begin - ahead;  // ragged block
  n = n < 0 ? 0 : (n > nsteps ? nsteps : n);
  return n == nsteps ? nsteps : n / slots * slots;
}

// Kernels whose dynamic LDS exceeds 64 KiB must opt in (gfx950 has 160 KiB per CU).
template <class K>
inline hipError_t ensure_lds(K* kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

hipError_t launch_attn_fwd(const FwdArgs& a, DT dt, int d, bool causal, int BH, hipStream_t s);
hipError_t launch_attn_fwd_combine(const FwdArgs& a, DT dt, int d, hipStream_t s);
hipError_t launch_pass1(const Pass1Args& a, DT dt, int d, bool causal, hipStream_t s);
// The two-pass sweeps of 16-bit inputs, d = 64 and d = 128 (VGPR form, their own
// translation unit; called by launch_pass1).
hipError_t launch_pass1_d64(const Pass1Args& a, DT dt, bool causal, hipStream_t s);
hipError_t launch_pass1_combine(const Pass1Args& a, DT dt, int d, hipStream_t s);
// Measurement probe (probes.hip): the float32 atomic additions of a gQ-in-pass-2 schedule.
hipError_t launch_probe_gq_atomics(float* gq, int BH, int N, int d, int nsplit, hipStream_t s);
// Pass 1 with 16-query waves for 16-bit inputs at d = 128 (64 queries per workgroup,
// every score tile computed once) and its split merge.
__host__ __device__ inline int pass1_q16_tiles(int N) { return (N + 63) / 64; }
__host__ __device__ constexpr size_t pass1_q16_record_floats() { return (size_t)(4 * 8 * 4 + 2) * 64; }
hipError_t launch_pass1_q16(const Pass1Args& a, DT dt, bool causal, hipStream_t s);
hipError_t launch_pass1_q16_combine(const Pass1Args& a, DT dt, hipStream_t s);
// Four-pass ablation schedule, 16-bit inputs: sweep 0 writes alpha, sweep 1 E
// (alpha known), sweep 2 gQ and gdO (alpha and E known); each with its split merge.
hipError_t launch_fourpass_sweep(const Pass1Args& a, int sweep, DT dt, int d, bool causal, hipStream_t s);
// First backward on the staged 16-bit kernels (with its split merge when nsplit > 1):
// dQ = tau dS K written to a.gQ (reads Q, K, V, dO, L, D), and dK = tau dS^T Q,
// dV = P^T dO written to a.gK, a.gV (reads Q, K, V, dO, L, D).
hipError_t launch_first_bwd_dq(const Pass1Args& a, DT dt, int d, bool causal, hipStream_t s);
hipError_t launch_first_bwd_dkdv(const Pass2Args& a, DT dt, int d, bool causal, hipStream_t s);
__host__ __device__ inline size_t first_bwd_dq_record_floats(int d) { return (size_t)(d / 32) * 16 * 64; }
__host__ __device__ inline size_t fourpass_record_floats(int d) { return (size_t)2 * (d / 32) * 16 * 64; }
// 16-bit pass 2 at d = 64 is built for two waves per SIMD (two workgroups per CU).
inline int pass2_blocks_per_cu(DT dt, int d) { return (dt != DT::F32 && d == 64) ? 2 : 1; }
hipError_t launch_pass2(const Pass2Args& a, DT dt, int d, bool causal, hipStream_t s);
// The non-causal d = 128 BoB sweep of pass 2, 16-bit inputs (VGPR form, its own translation unit).
hipError_t launch_pass2_d128(const Pass2Args& a, DT dt, hipStream_t s);
hipError_t launch_pass2_reduce(const Pass2Args& a, DT dt, int d, hipStream_t s);
// kReduceAtomic: zero the float32 sums before pass 2, convert them to gK, gV after it.
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s);
hipError_t launch_pass2_convert(const Pass2Args& a, DT dt, int d, hipStream_t s);
hipError_t launch_bwd_rowdot(const BwdArgs& a, DT dt, int d, int BH, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, DT dt, int d, bool causal, int BH, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, DT dt, int d, bool causal, int BH, hipStream_t s);

}  // namespace fb
