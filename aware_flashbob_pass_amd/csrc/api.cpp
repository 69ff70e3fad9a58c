// C ABI of the attention BoB library: argument checks, workspace layout, split
// selection and stream-ordered launches. Declarations and contracts live in
// include/flashbob.h.
#include "flashbob.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"

using fb::DT;

namespace {

thread_local std::string g_err;

fb_status_t fail(fb_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

fb_status_t ok() {
  g_err.clear();
  return FB_OK;
}

// ---- tuning -------------------------------------------------------------------
std::mutex g_tune_mu;
int g_split1 = 0, g_split2 = 0;
int g_reduce = fb::kReduceRecords;  // pass 2's split reduction (fb_set_reduction)
constexpr int kMaxSplits = 64;
constexpr int kTargetBlocks = 256;   // one workgroup per compute unit
constexpr int kMinTilesPerSplit = 4; // 4 x 32 streamed rows per split at least

int auto_splits(int BH, int N, int target = kTargetBlocks, int tiles = -1) {
  const long long blocks = (long long)(tiles < 0 ? fb::row_tiles(N) : tiles) * BH;
  if (blocks >= target) return 1;
  const int steps = (N + 31) / 32;
  int s = (int)((target + blocks - 1) / blocks);
  s = std::min(s, std::max(1, steps / kMinTilesPerSplit));
  return std::max(1, std::min(s, kMaxSplits));
}

// Default split targets follow how many workgroups of each kernel one compute
// unit holds: the statistics kernel at least two (512 workgroups); 16-bit pass 2
// at d = 64 two (it is built for two waves per SIMD); pass 1 and the rest one.
// With an explicit pass-1 split the statistics kernel follows that value.
// 16-bit inputs at d = 128 run pass 1 with 16-query waves, 64 queries per workgroup.
bool pass1_uses_q16(fb::DT dt, int d) { return dt != fb::DT::F32 && d == 128; }

void splits_for(int BH, int N, fb::DT dt, int d, int* s0, int* s1, int* s2) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  *s1 = g_split1 > 0 ? g_split1
                     : auto_splits(BH, N, kTargetBlocks, pass1_uses_q16(dt, d) ? fb::pass1_q16_tiles(N) : -1);
  *s2 = g_split2 > 0 ? g_split2 : auto_splits(BH, N, fb::pass2_blocks_per_cu(dt, d) * kTargetBlocks);
  *s0 = g_split1 > 0 ? g_split1 : auto_splits(BH, N, 2 * kTargetBlocks);
}

// ---- library allocations -------------------------------------------------------
std::atomic<size_t> g_alloc_limit{0};  // 0: no cap

// Stream-ordered device allocation for the entry points that allocate. Refused
// with FB_ERR_OOM, before any HIP call, when `bytes` exceeds the caller's cap
// (fb_set_alloc_limit); then when it exceeds the free memory of the current
// device; then when hipMallocAsync itself fails.
fb_status_t device_alloc(void** p, size_t bytes, hipStream_t s, const char* what) {
  *p = nullptr;
  const size_t cap = g_alloc_limit.load();
  if (cap && bytes > cap)
    return fail(FB_ERR_OOM, "%s of %zu bytes exceeds the allocation limit of %zu bytes", what, bytes, cap);
  size_t free_b = 0, total_b = 0;
  hipError_t e = hipMemGetInfo(&free_b, &total_b);
  if (e != hipSuccess) return fail(FB_ERR_HIP, "hipMemGetInfo: %s", hipGetErrorString(e));
  if (bytes > free_b)
    return fail(FB_ERR_OOM, "%s of %zu bytes exceeds the %zu bytes free on the device", what, bytes, free_b);
  e = hipMallocAsync(p, bytes, s);
  if (e != hipSuccess || !*p) {
    (void)hipGetLastError();
    *p = nullptr;
    return fail(FB_ERR_OOM, "%s of %zu bytes failed: %s", what, bytes, hipGetErrorString(e));
  }
  return FB_OK;
}

// ---- fixed device scratch (bob_attention_noalloc) -------------------------------
// A file-scope device array serves as the workspace of the entry point that
// allocates nothing. Each GPU the library runs on holds its own copy from module
// load until the process ends. In host code `scratch` names only a host-side
// stand-in, so the device address of each GPU's copy is looked up once per device
// (with that device current) and every host use goes through that address.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fb_status_t hip_fail(hipError_t e, const char* what);

fb_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FB_ERR_ARG, "device %d out of range [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e == hipSuccess ? hipErrorInvalidSymbol : e, "hipGetSymbolAddress");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FB_OK;
}

// ---- kernel timing ------------------------------------------------------------
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::string g_prof_only;  // empty: every kernel
std::vector<ProfRec> g_prof;

template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    on = g_prof_on && (g_prof_only.empty() || g_prof_only == name);
  }
  if (!on) return launch();
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return launch();
  hipEventRecord(a, s);
  hipError_t e = launch();
  hipEventRecord(b, s);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back({name, a, b});
  return e;
}

// ---- argument checks -----------------------------------------------------------
constexpr int kMaxRows = 2147483647 - 255;  // B*H*N bound (see check_shape)

size_t esize(fb_dtype_t dt) { return dt == FB_F32 ? 4 : 2; }

fb_status_t check_shape(int B, int H, int N, int d, fb_dtype_t dtype, float tau) {
  if (dtype != FB_F32 && dtype != FB_F16 && dtype != FB_BF16) return fail(FB_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (d != 64 && d != 128) return fail(FB_ERR_HEADDIM, "head dim d=%d not supported (64 or 128)", d);
  if (B < 1 || H < 1 || N < 1) return fail(FB_ERR_SHAPE, "B, H, N must be >= 1 (got %d, %d, %d)", B, H, N);
  if ((long long)B * H > 65535) return fail(FB_ERR_SHAPE, "B*H=%lld exceeds 65535", (long long)B * H);
  // Rows of all heads are indexed with int arithmetic in the kernels and grids
  // (row_tiles(N) = (N + 127) / 128, resident row q0 + 31 < N + 128, launch ids
  // tile + tiles * head): bounding B*H*N by INT_MAX keeps every one of them in
  // range and the workspace size far inside size_t.
  if ((long long)B * H * N > (long long)kMaxRows)
    return fail(FB_ERR_SHAPE, "B*H*N=%lld exceeds %d", (long long)B * H * N, kMaxRows);
  if (!std::isfinite(tau)) return fail(FB_ERR_ARG, "tau must be finite");
  return FB_OK;
}

fb_status_t check_ptrs(std::initializer_list<std::pair<const char*, const void*>> ptrs, size_t align) {
  for (auto& p : ptrs) {
    if (!p.second) return fail(FB_ERR_NULL, "%s is NULL", p.first);
    if (reinterpret_cast<uintptr_t>(p.second) % align)
      return fail(FB_ERR_ARG, "%s is not %zu-byte aligned", p.first, align);
  }
  return FB_OK;
}

fb_status_t check_no_alias(std::initializer_list<std::pair<const char*, const void*>> outs,
                           std::initializer_list<std::pair<const char*, const void*>> ins) {
  std::vector<std::pair<const char*, const void*>> o(outs);
  for (size_t i = 0; i < o.size(); ++i) {
    if (!o[i].second) continue;
    for (auto& in : ins)
      if (in.second && in.second == o[i].second) return fail(FB_ERR_ARG, "output %s aliases input %s", o[i].first, in.first);
    for (size_t j = i + 1; j < o.size(); ++j)
      if (o[j].second == o[i].second) return fail(FB_ERR_ARG, "outputs %s and %s alias", o[i].first, o[j].first);
  }
  return FB_OK;
}

fb_status_t hip_fail(hipError_t e, const char* what) {
  return fail(FB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

DT to_dt(fb_dtype_t t) { return t == FB_BF16 ? DT::BF16 : (t == FB_F16 ? DT::F16 : DT::F32); }

// ---- workspace layout ------------------------------------------------------------
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t o, l, dd, alpha, e, l2, cc, part, acc32, counters, total;
  int s0, s1, s2;  // splits of the statistics kernel, pass 1, pass 2
  int reduce;      // pass 2's split reduction (16-bit inputs with s2 > 1)
};

WsLayout layout(int B, int H, int N, int d, fb_dtype_t dtype) {
  WsLayout w{};
  const size_t BH = (size_t)B * H;
  const size_t vec = align256(BH * N * sizeof(float));
  splits_for((int)BH, N, to_dt(dtype), d, &w.s0, &w.s1, &w.s2);
  if (dtype == FB_F32) w.s0 = 1;  // the float32 statistics kernel does not split
  size_t off = 0;
  w.o = off;
  off += align256(BH * N * d * esize(dtype));
  w.l = off;
  off += vec;
  w.dd = off;
  off += vec;
  w.alpha = off;
  off += vec;
  w.e = off;
  off += vec;
  w.l2 = off;  // L log2(e) and c = alpha D + E, written by pass 1 for pass 2
  off += vec;
  w.cc = off;
  off += vec;
  const size_t tiles = (size_t)fb::row_tiles(N) * BH * 4;  // waves
  const size_t p1 = w.s1 <= 1 ? 0
                    : pass1_uses_q16(to_dt(dtype), d)
                        ? (size_t)w.s1 * fb::pass1_q16_tiles(N) * BH * 4 * fb::pass1_q16_record_floats() * sizeof(float)
                        : (size_t)w.s1 * tiles * fb::pass1_record_floats(d) * sizeof(float);
  const size_t p2 = w.s2 > 1 ? (size_t)w.s2 * tiles * fb::pass2_record_floats(d) * sizeof(float) : 0;
  const size_t p0 = w.s0 > 1 ? (size_t)w.s0 * tiles * fb::fwd_record_floats(d) * sizeof(float) : 0;
  w.part = off;  // each kernel's records are consumed before the next kernel writes its own
  off += align256(std::max(p0, std::max(p1, p2)));
  {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    w.reduce = (dtype != FB_F32 && w.s2 > 1) ? g_reduce : fb::kReduceRecords;
  }
  w.acc32 = off;
  if (w.reduce == fb::kReduceAtomic) off += align256((size_t)2 * BH * N * d * sizeof(float));
  w.counters = off;
  if (w.reduce == fb::kReduceLastBlock) off += align256((size_t)fb::row_tiles(N) * BH * sizeof(unsigned));
  w.total = off;
  return w;
}

template <class F>
fb_status_t run(const char* name, hipStream_t s, F&& launch) {
  hipError_t e = timed(name, s, launch);
  if (e != hipSuccess) return hip_fail(e, name);
  return FB_OK;
}

// pass 2 (key-tile parallel) and its split reduction
fb_status_t column_pass(const void* Q, const void* K, const void* V, const void* dO, const void* UQ, const void* UK,
                        const void* UV, const float* L, const float* D, const float* alpha, const float* E, float tau,
                        bool causal, int BH, int N, int d, DT dt, void* gK, void* gV, char* ws, const WsLayout& w,
                        hipStream_t s) {
  fb::Pass2Args p2{};
  p2.Q = Q; p2.K = K; p2.V = V; p2.dO = dO; p2.UQ = UQ; p2.UK = UK; p2.UV = UV;
  p2.L = L; p2.D = D; p2.alpha = alpha; p2.E = E; p2.gK = gK; p2.gV = gV;
  p2.l2 = reinterpret_cast<const float*>(ws + w.l2);
  p2.c = reinterpret_cast<const float*>(ws + w.cc);
  p2.part = reinterpret_cast<float*>(ws + w.part);
  p2.tau = tau; p2.N = N; p2.BH = BH; p2.nsplit = w.s2;
  p2.reduce = w.reduce;
  p2.acc32 = reinterpret_cast<float*>(ws + w.acc32);
  p2.counters = reinterpret_cast<unsigned*>(ws + w.counters);  // zeroed by pass 1
  fb_status_t st;
  if (w.reduce == fb::kReduceAtomic) {
    st = run("bob_pass2_zero", s, [&] { return fb::launch_zero_f32(p2.acc32, (size_t)2 * BH * N * d, s); });
    if (st) return st;
  }
  st = run("bob_pass2", s, [&] { return fb::launch_pass2(p2, dt, d, causal, s); });
  if (st) return st;
  if (w.reduce == fb::kReduceAtomic) {
    st = run("bob_pass2_convert", s, [&] { return fb::launch_pass2_convert(p2, dt, d, s); });
    if (st) return st;
  } else if (w.s2 > 1 && w.reduce == fb::kReduceRecords) {
    st = run("bob_pass2_reduce", s, [&] { return fb::launch_pass2_reduce(p2, dt, d, s); });
    if (st) return st;
  }
  return FB_OK;
}

// pass 1 + pass 2 from O, L, D (all device pointers already checked)
fb_status_t two_pass(const void* Q, const void* K, const void* V, const void* dO, const void* UQ, const void* UK,
                     const void* UV, const void* O, const float* L, const float* D, float tau, bool causal, int B,
                     int H, int N, int d, fb_dtype_t dtype, void* gQ, void* gK, void* gV, void* gdO, float* alpha,
                     float* E, char* ws, const WsLayout& w, hipStream_t s) {
  const DT dt = to_dt(dtype);
  const int BH = B * H;
  fb::Pass1Args p1{};
  p1.Q = Q; p1.K = K; p1.V = V; p1.dO = dO; p1.UQ = UQ; p1.UK = UK; p1.UV = UV; p1.O = O;
  p1.L = L; p1.D = D; p1.gQ = gQ; p1.gdO = gdO; p1.alpha = alpha; p1.E = E;
  p1.l2 = reinterpret_cast<float*>(ws + w.l2);
  p1.c = reinterpret_cast<float*>(ws + w.cc);
  p1.part = reinterpret_cast<float*>(ws + w.part);
  p1.tau = tau; p1.N = N; p1.BH = BH; p1.nsplit = w.s1;
  if (w.reduce == fb::kReduceLastBlock) p1.p2_counters = reinterpret_cast<unsigned*>(ws + w.counters);
  const bool q16 = pass1_uses_q16(dt, d);
  fb_status_t st = run("bob_pass1", s, [&] {
    return q16 ? fb::launch_pass1_q16(p1, dt, causal, s) : fb::launch_pass1(p1, dt, d, causal, s);
  });
  if (st) return st;
  if (w.s1 > 1) {
    st = run("bob_pass1_combine", s, [&] {
      return q16 ? fb::launch_pass1_q16_combine(p1, dt, s) : fb::launch_pass1_combine(p1, dt, d, s);
    });
    if (st) return st;
  }
  return column_pass(Q, K, V, dO, UQ, UK, UV, L, D, alpha, E, tau, causal, BH, N, d, dt, gK, gV, ws, w, s);
}

// Four-pass ablation: alpha sweep, E sweep, row-output sweep, then pass 2.
fb_status_t four_pass(const void* Q, const void* K, const void* V, const void* dO, const void* UQ, const void* UK,
                      const void* UV, const void* O, const float* L, const float* D, float tau, bool causal, int B,
                      int H, int N, int d, fb_dtype_t dtype, void* gQ, void* gK, void* gV, void* gdO, float* alpha,
                      float* E, char* ws, const WsLayout& w, hipStream_t s) {
  const DT dt = to_dt(dtype);
  const int BH = B * H;
  fb::Pass1Args p1{};
  p1.Q = Q; p1.K = K; p1.V = V; p1.dO = dO; p1.UQ = UQ; p1.UK = UK; p1.UV = UV; p1.O = O;
  p1.L = L; p1.D = D; p1.gQ = gQ; p1.gdO = gdO; p1.alpha = alpha; p1.E = E;
  p1.l2 = reinterpret_cast<float*>(ws + w.l2);
  p1.c = reinterpret_cast<float*>(ws + w.cc);
  p1.part = reinterpret_cast<float*>(ws + w.part);
  p1.tau = tau; p1.N = N; p1.BH = BH; p1.nsplit = w.s1;
  if (w.reduce == fb::kReduceLastBlock) p1.p2_counters = reinterpret_cast<unsigned*>(ws + w.counters);
  static const char* names[3] = {"fourpass_alpha", "fourpass_energy", "fourpass_rows"};
  for (int sweep = 0; sweep < 3; ++sweep) {
    // The scalar sweeps (and the rows sweep at d = 64) run two workgroups per CU,
    // like the statistics kernel, so they take its split count. Record space: the
    // scalar records (64 floats per wave) fit in the statistics records; the rows
    // records (2 d / 32 tiles per wave) fit in the pass-1 records at up to twice
    // the pass-1 split count.
    if (sweep < 2) p1.nsplit = w.s0;
    else p1.nsplit = (d == 64 && w.s1 > 1) ? std::min(w.s0, 2 * w.s1) : w.s1;
    fb_status_t st = run(names[sweep], s, [&] { return fb::launch_fourpass_sweep(p1, sweep, dt, d, causal, s); });
    if (st) return st;
  }
  return column_pass(Q, K, V, dO, UQ, UK, UV, L, D, alpha, E, tau, causal, BH, N, d, dt, gK, gV, ws, w, s);
}

}  // namespace

extern "C" {

const char* fb_last_error(void) { return g_err.c_str(); }

fb_status_t fb_set_tuning(int pass1_splits, int pass2_splits) {
  if (pass1_splits < 0 || pass1_splits > kMaxSplits || pass2_splits < 0 || pass2_splits > kMaxSplits)
    return fail(FB_ERR_ARG, "splits must be in [0, %d]", kMaxSplits);
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_split1 = pass1_splits;
  g_split2 = pass2_splits;
  return ok();
}

fb_status_t fb_set_reduction(int mode) {
  if (mode < fb::kReduceRecords || mode > fb::kReduceLastBlock)
    return fail(FB_ERR_ARG, "reduction mode %d not in {0, 1, 2}", mode);
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_reduce = mode;
  return ok();
}

fb_status_t fb_probe_gq_atomics(float* gq, int B, int H, int N, int d, int splits, hipStream_t stream) {
  fb_status_t st = check_shape(B, H, N, d, FB_BF16, 1.f);
  if (st) return st;
  if (splits < 1 || splits > kMaxSplits) return fail(FB_ERR_ARG, "splits=%d not in [1, %d]", splits, kMaxSplits);
  if ((st = check_ptrs({{"gq", gq}}, 16))) return st;
  st = run("probe_gq_atomics", stream, [&] { return fb::launch_probe_gq_atomics(gq, B * H, N, d, splits, stream); });
  if (st) return st;
  return ok();
}

fb_status_t fb_set_alloc_limit(size_t bytes) {
  g_alloc_limit.store(bytes);
  return ok();
}

size_t bob_workspace_bytes(int B, int H, int N, int d, fb_dtype_t dtype) {
  if (check_shape(B, H, N, d, dtype, 1.f) != FB_OK) return 0;
  return layout(B, H, N, d, dtype).total;
}

fb_status_t bob_attention_ws(const void* Q, const void* K, const void* V, const void* dO, const void* UQ,
                             const void* UK, const void* UV, float tau, int causal, int B, int H, int N, int d,
                             fb_dtype_t dtype, void* gQ, void* gK, void* gV, void* gdO, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  fb_status_t st = check_shape(B, H, N, d, dtype, tau);
  if (st) return st;
  st = check_ptrs({{"Q", Q}, {"K", K}, {"V", V}, {"dO", dO}, {"UQ", UQ}, {"UK", UK}, {"UV", UV},
                   {"gQ", gQ}, {"gK", gK}, {"gV", gV}, {"gdO", gdO}}, 16);
  if (st) return st;
  st = check_no_alias({{"gQ", gQ}, {"gK", gK}, {"gV", gV}, {"gdO", gdO}},
                      {{"Q", Q}, {"K", K}, {"V", V}, {"dO", dO}, {"UQ", UQ}, {"UK", UK}, {"UV", UV}});
  if (st) return st;
  const WsLayout w = layout(B, H, N, d, dtype);
  if (!ws) return fail(FB_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(FB_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < w.total) return fail(FB_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, w.total);
  char* wsb = static_cast<char*>(ws);
  void* O = wsb + w.o;
  float* L = reinterpret_cast<float*>(wsb + w.l);
  float* D = reinterpret_cast<float*>(wsb + w.dd);
  fb::FwdArgs fa{Q, K, V, dO, O, L, D, tau, N, B * H, w.s0, reinterpret_cast<float*>(wsb + w.part)};
  st = run("attn_fwd_stats", stream, [&] { return fb::launch_attn_fwd(fa, to_dt(dtype), d, causal != 0, B * H, stream); });
  if (st) return st;
  if (w.s0 > 1) {
    st = run("attn_fwd_combine", stream, [&] { return fb::launch_attn_fwd_combine(fa, to_dt(dtype), d, stream); });
    if (st) return st;
  }
  st = two_pass(Q, K, V, dO, UQ, UK, UV, O, L, D, tau, causal != 0, B, H, N, d, dtype, gQ, gK, gV, gdO,
                reinterpret_cast<float*>(wsb + w.alpha), reinterpret_cast<float*>(wsb + w.e), wsb, w, stream);
  if (st) return st;
  return ok();
}

fb_status_t bob_attention_fourpass_ws(const void* Q, const void* K, const void* V, const void* dO, const void* UQ,
                                      const void* UK, const void* UV, float tau, int causal, int B, int H, int N, int d,
                                      fb_dtype_t dtype, void* gQ, void* gK, void* gV, void* gdO, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  fb_status_t st = check_shape(B, H, N, d, dtype, tau);
  if (st) return st;
  if (dtype == FB_F32) return fail(FB_ERR_DTYPE, "the four-pass schedule is implemented for bf16/fp16 inputs");
  st = check_ptrs({{"Q", Q}, {"K", K}, {"V", V}, {"dO", dO}, {"UQ", UQ}, {"UK", UK}, {"UV", UV},
                   {"gQ", gQ}, {"gK", gK}, {"gV", gV}, {"gdO", gdO}}, 16);
  if (st) return st;
  st = check_no_alias({{"gQ", gQ}, {"gK", gK}, {"gV", gV}, {"gdO", gdO}},
                      {{"Q", Q}, {"K", K}, {"V", V}, {"dO", dO}, {"UQ", UQ}, {"UK", UK}, {"UV", UV}});
  if (st) return st;
  const WsLayout w = layout(B, H, N, d, dtype);
  if (!ws) return fail(FB_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(FB_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < w.total) return fail(FB_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, w.total);
  char* wsb = static_cast<char*>(ws);
  void* O = wsb + w.o;
  float* L = reinterpret_cast<float*>(wsb + w.l);
  float* D = reinterpret_cast<float*>(wsb + w.dd);
  fb::FwdArgs fa{Q, K, V, dO, O, L, D, tau, N, B * H, w.s0, reinterpret_cast<float*>(wsb + w.part)};
  st = run("attn_fwd_stats", stream, [&] { return fb::launch_attn_fwd(fa, to_dt(dtype), d, causal != 0, B * H, stream); });
  if (st) return st;
  if (w.s0 > 1) {
    st = run("attn_fwd_combine", stream, [&] { return fb::launch_attn_fwd_combine(fa, to_dt(dtype), d, stream); });
    if (st) return st;
  }
  st = four_pass(Q, K, V, dO, UQ, UK, UV, O, L, D, tau, causal != 0, B, H, N, d, dtype, gQ, gK, gV, gdO,
                 reinterpret_cast<float*>(wsb + w.alpha), reinterpret_cast<float*>(wsb + w.e), wsb, w, stream);
  if (st) return st;
  return ok();
}

fb_status_t bob_attention(const void* Q, const void* K, const void* V, const void* dO, const void* UQ, const void* UK,
                          const void* UV, float tau, int causal, int B, int H, int N, int d, fb_dtype_t dtype,
                          void* gQ, void* gK, void* gV, void* gdO, hipStream_t stream) {
  fb_status_t st = check_shape(B, H, N, d, dtype, tau);
  if (st) return st;
  st = check_ptrs({{"Q", Q}, {"K", K}, {"V", V}, {"dO", dO}, {"UQ", UQ}, {"UK", UK}, {"UV", UV},
                   {"gQ", gQ}, {"gK", gK}, {"gV", gV}, {"gdO", gdO}}, 16);
  if (st) return st;
  st = check_no_alias({{"gQ", gQ}, {"gK", gK}, {"gV", gV}, {"gdO", gdO}},
                      {{"Q", Q}, {"K", K}, {"V", V}, {"dO", dO}, {"UQ", UQ}, {"UK", UK}, {"UV", UV}});
  if (st) return st;
  const size_t bytes = layout(B, H, N, d, dtype).total;
  void* ws = nullptr;
  st = device_alloc(&ws, bytes, stream, "workspace allocation");
  if (st) return st;
  st = bob_attention_ws(Q, K, V, dO, UQ, UK, UV, tau, causal, B, H, N, d, dtype, gQ, gK, gV, gdO, ws, bytes, stream);
  std::string msg = g_err;
  hipError_t ef = hipFreeAsync(ws, stream);
  if (st) {
    g_err = msg;
    return st;
  }
  if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync");
  return ok();
}

fb_status_t bob_attention_noalloc(const void* Q, const void* K, const void* V, const void* dO, const void* UQ,
                                  const void* UK, const void* UV, float tau, int causal, int B, int H, int N, int d,
                                  fb_dtype_t dtype, void* gQ, void* gK, void* gV, void* gdO, hipStream_t stream) {
  fb_status_t st = check_shape(B, H, N, d, dtype, tau);
  if (st) return st;
  const size_t bytes = layout(B, H, N, d, dtype).total;
  if (bytes > kScratchBytes)
    return fail(FB_ERR_WORKSPACE, "this shape needs %zu bytes of scratch, more than the %zu-byte maximum of "
                "bob_attention_noalloc (use bob_attention_ws)", bytes, kScratchBytes);
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st) return st;
  return bob_attention_ws(Q, K, V, dO, UQ, UK, UV, tau, causal, B, H, N, d, dtype, gQ, gK, gV, gdO, ws,
                          kScratchBytes, stream);
}

fb_status_t bob_attention_with_stats(const void* Q, const void* K, const void* V, const void* dO, const void* UQ,
                                     const void* UK, const void* UV, const void* O, const float* L, const float* D,
                                     float tau, int causal, int B, int H, int N, int d, fb_dtype_t dtype, void* gQ,
                                     void* gK, void* gV, void* gdO, float* alpha_out, float* E_out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  fb_status_t st = check_shape(B, H, N, d, dtype, tau);
  if (st) return st;
  st = check_ptrs({{"Q", Q}, {"K", K}, {"V", V}, {"dO", dO}, {"UQ", UQ}, {"UK", UK}, {"UV", UV}, {"O", O},
                   {"gQ", gQ}, {"gK", gK}, {"gV", gV}, {"gdO", gdO}}, 16);
  if (st) return st;
  st = check_ptrs({{"L", L}, {"D", D}}, 4);
  if (st) return st;
  if (alpha_out && (st = check_ptrs({{"alpha_out", alpha_out}}, 4))) return st;
  if (E_out && (st = check_ptrs({{"E_out", E_out}}, 4))) return st;
  st = check_no_alias({{"gQ", gQ}, {"gK", gK}, {"gV", gV}, {"gdO", gdO}, {"alpha_out", alpha_out}, {"E_out", E_out}},
                      {{"Q", Q}, {"K", K}, {"V", V}, {"dO", dO}, {"UQ", UQ}, {"UK", UK}, {"UV", UV}, {"O", O},
                       {"L", L}, {"D", D}});
  if (st) return st;
  const WsLayout w = layout(B, H, N, d, dtype);
  if (!ws) return fail(FB_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(FB_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < w.total) return fail(FB_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, w.total);
  char* wsb = static_cast<char*>(ws);
  float* alpha = alpha_out ? alpha_out : reinterpret_cast<float*>(wsb + w.alpha);
  float* E = E_out ? E_out : reinterpret_cast<float*>(wsb + w.e);
  st = two_pass(Q, K, V, dO, UQ, UK, UV, O, L, D, tau, causal != 0, B, H, N, d, dtype, gQ, gK, gV, gdO, alpha, E, wsb,
                w, stream);
  if (st) return st;
  return ok();
}

fb_status_t attn_fwd(const void* Q, const void* K, const void* V, const void* dO, float tau, int causal, int B, int H,
                     int N, int d, fb_dtype_t dtype, void* O, float* L, float* D_out, hipStream_t stream) {
  fb_status_t st = check_shape(B, H, N, d, dtype, tau);
  if (st) return st;
  st = check_ptrs({{"Q", Q}, {"K", K}, {"V", V}, {"O", O}}, 16);
  if (st) return st;
  st = check_ptrs({{"L", L}}, 4);
  if (st) return st;
  if (D_out) {
    if ((st = check_ptrs({{"D_out", D_out}}, 4))) return st;
    if ((st = check_ptrs({{"dO (needed for D_out)", dO}}, 16))) return st;
  }
  st = check_no_alias({{"O", O}, {"L", L}, {"D_out", D_out}}, {{"Q", Q}, {"K", K}, {"V", V}, {"dO", dO}});
  if (st) return st;
  fb::FwdArgs fa{Q, K, V, D_out ? dO : nullptr, O, L, D_out, tau, N};
  st = run("attn_fwd_stats", stream, [&] { return fb::launch_attn_fwd(fa, to_dt(dtype), d, causal != 0, B * H, stream); });
  if (st) return st;
  return ok();
}

fb_status_t attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* L,
                     float tau, int causal, int B, int H, int N, int d, fb_dtype_t dtype, void* dQ, void* dK, void* dV,
                     float* D_out, hipStream_t stream) {
  fb_status_t st = check_shape(B, H, N, d, dtype, tau);
  if (st) return st;
  st = check_ptrs({{"Q", Q}, {"K", K}, {"V", V}, {"O", O}, {"dO", dO}, {"dQ", dQ}, {"dK", dK}, {"dV", dV}}, 16);
  if (st) return st;
  st = check_ptrs({{"L", L}}, 4);
  if (st) return st;
  if (D_out && (st = check_ptrs({{"D_out", D_out}}, 4))) return st;
  st = check_no_alias({{"dQ", dQ}, {"dK", dK}, {"dV", dV}, {"D_out", D_out}},
                      {{"Q", Q}, {"K", K}, {"V", V}, {"O", O}, {"dO", dO}, {"L", L}});
  if (st) return st;
  const DT dt = to_dt(dtype);
  const int BH = B * H;
  // 16-bit inputs run the staged kernels, which may split the streamed range and
  // then need record buffers; float32 runs the single-buffered kernels.
  int s0 = 1, s1 = 1, s2 = 1;
  size_t rec_bytes = 0;
  if (dt != DT::F32) {
    splits_for(BH, N, dt, d, &s0, &s1, &s2);
    const size_t tiles = (size_t)fb::row_tiles(N) * BH * 4;  // waves
    const size_t r1 = s1 > 1 ? (size_t)s1 * tiles * fb::first_bwd_dq_record_floats(d) * sizeof(float) : 0;
    const size_t r2 = s2 > 1 ? (size_t)s2 * tiles * fb::pass2_record_floats(d) * sizeof(float) : 0;
    rec_bytes = align256(std::max(r1, r2));  // dQ's records are merged before dK/dV writes its own
  }
  const size_t d_bytes = D_out ? 0 : align256((size_t)BH * N * sizeof(float));
  void* tmp = nullptr;
  if (d_bytes + rec_bytes) {
    st = device_alloc(&tmp, d_bytes + rec_bytes, stream, "scratch allocation");
    if (st) return st;
  }
  float* D = D_out ? D_out : static_cast<float*>(tmp);
  float* part = reinterpret_cast<float*>(static_cast<char*>(tmp) + d_bytes);
  fb::BwdArgs ba{Q, K, V, O, dO, L, D, dQ, dK, dV, tau, N};
  st = run("attn_bwd_rowdot", stream, [&] { return fb::launch_bwd_rowdot(ba, dt, d, BH, stream); });
  if (dt == DT::F32) {
    if (!st) st = run("attn_bwd_dq", stream, [&] { return fb::launch_bwd_dq(ba, dt, d, causal != 0, BH, stream); });
    if (!st)
      st = run("attn_bwd_dkdv", stream, [&] { return fb::launch_bwd_dkdv(ba, dt, d, causal != 0, BH, stream); });
  } else {
    // the tensors the first backward does not read (UQ, UK, UV) point at valid inputs
    fb::Pass1Args p1{};
    p1.Q = Q; p1.K = K; p1.V = V; p1.dO = dO; p1.UQ = Q; p1.UK = K; p1.UV = V; p1.O = O;
    p1.L = L; p1.D = D; p1.gQ = dQ; p1.part = part;
    p1.tau = tau; p1.N = N; p1.BH = BH; p1.nsplit = s1;
    if (!st) st = run("attn_bwd_dq", stream, [&] { return fb::launch_first_bwd_dq(p1, dt, d, causal != 0, stream); });
    fb::Pass2Args p2{};
    p2.Q = Q; p2.K = K; p2.V = V; p2.dO = dO; p2.UQ = Q; p2.UK = K; p2.UV = V;
    p2.L = L; p2.D = D; p2.gK = dK; p2.gV = dV; p2.part = part;
    p2.tau = tau; p2.N = N; p2.BH = BH; p2.nsplit = s2;
    if (!st)
      st = run("attn_bwd_dkdv", stream, [&] { return fb::launch_first_bwd_dkdv(p2, dt, d, causal != 0, stream); });
    if (!st && s2 > 1)
      st = run("attn_bwd_dkdv_reduce", stream, [&] { return fb::launch_pass2_reduce(p2, dt, d, stream); });
  }
  if (tmp) {
    std::string msg = g_err;
    hipError_t ef = hipFreeAsync(tmp, stream);
    if (st) {
      g_err = msg;
      return st;
    }
    if (ef != hipSuccess) return hip_fail(ef, "hipFreeAsync");
  }
  if (st) return st;
  return ok();
}

void fb_profile_start(const char* only) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only = only ? only : "";
  for (auto& r : g_prof) {
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  g_prof.clear();
  g_prof_on = true;
}

int fb_profile_stop(fb_kernel_time_t* out, int max) {
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = false;
    recs.swap(g_prof);
  }
  std::map<std::string, std::pair<int, double>> agg;
  std::vector<std::string> order;
  int status = 0;
  for (auto& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) status = FB_ERR_HIP;
    if (!agg.count(r.name)) order.push_back(r.name);
    auto& v = agg[r.name];
    v.first += 1;
    v.second += ms;
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  if (status) {
    fail(FB_ERR_HIP, "event timing failed");
    return status;
  }
  int i = 0;
  for (auto& name : order) {
    if (out && i < max) {
      std::memset(out[i].name, 0, sizeof(out[i].name));
      std::strncpy(out[i].name, name.c_str(), sizeof(out[i].name) - 1);
      out[i].launches = agg[name].first;
      out[i].total_ms = agg[name].second;
    }
    ++i;
  }
  return i;
}

}  // extern "C"
