// Pass 1 for 16-bit inputs at d = 128 with 16-query waves.
//
// Same method step as bob_pass1_kernel (FlashBoB review page, Summary; Strengths on
// Prop. 4.1: one key sweep per query tile accumulates the six alpha-free sums into
// four tiles and applies alpha and E at the end):
//   A = W_a UK + W_b K,  B = W_a K,  C = P K,  X = P UV + (P G) V,
//   gQ = tau (A - alpha B - e0 C),  gdO = X - alpha O,  E = e0 - alpha D.
//
// At d = 128 the four float32 accumulators of a 32-query wave would fill the whole
// register file; a 32-query kernel would have to split the accumulated head dimension
// over two workgroups and compute every score tile twice (16 executed units per pass
// instead of 11). Here a wave owns 16 queries: its four accumulators take 128
// registers, each score tile is computed once, and a workgroup of 4 waves (one per
// SIMD) holds 64 queries.
//
// The file is compiled in the matrix-core VGPR form (score tiles in VGPRs, no copies
// out of AGPRs); the four accumulators stay in AGPRs through inline-assembly products
// (mfma16_acc), which supply their own hazard waits and settle after the sweep.
// Products are v_mfma_f32_16x16x32 (16-bit operands, float32 accumulation; lane
// layout checked on the MI355X with an in-bounds probe: A lane l holds row l % 16
// and k = 8 (l / 16) .. + 7, B lane l column l % 16 and the same k, D lane l
// column l % 16 and rows 4 (l / 16) .. + 3). With g = lane / 16:
//  - score tiles (keys x queries, two 16-key halves per 32-key step): lane l holds
//    query l % 16 and keys 16 kt + 4 g + s of half kt, slot s;
//  - those 8 values per lane are directly the B operand of the accumulating products
//    (contraction over the 32 keys, k-slot 4 kt + s, i.e. key 16 (k / 4) + 4 g + k % 4);
//    their A operand (16 head dims x those keys) comes from the row-major tile through
//    two transposing LDS loads (ds_read_b64_tr_b16), keys 4 g .. 4 g + 3 and
//    16 + 4 g .. 16 + 4 g + 3;
//  - accumulators (16 head dims x 16 queries per tile, 8 tiles per tensor): lane l
//    holds query l % 16 and dims 16 mt + 4 g .. + 3.
// Staging: three LDS stages of the K, V, UK, UV row-major tiles (32 keys, 32 KiB),
// filled two steps ahead with global_load_lds_dwordx4; one barrier per step.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace fb {

static constexpr int kQWaves = 4;
static constexpr int kQRows = 16;  // queries per wave
static constexpr int kQD = 128;
static constexpr int kQTileElems = 32 * kQD;   // one 32-key row-major tile
static constexpr int kQStageElems = 4 * kQTileElems;
static constexpr int kQNBuf = 3;
static constexpr int kQLayout = 1;  // LDS row swizzle of this kernel's tiles (common.hpp swz)

template <class TT>
__device__ inline f32x4 mfma_16x16x32(typename TT::vec a, typename TT::vec b, f32x4 c) {
  if constexpr (std::is_same_v<TT, BF16>)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ inline f32x4 q16_zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// A operand of an accumulating product: head dims 16 mt + (lane % 16), keys
// 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3 of the row-major tile (two transposing
// loads; source lane i of a 16-lane group addresses key row 4 g + i / 4 (+ 16) at dims
// 16 mt + 4 (i % 4) .. + 3 and receives dim 16 mt + i of the four rows).
template <class TT>
__device__ inline typename TT::vec q16_tr_op(const typename TT::elem* tile, int mt, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const int col = mt * 16 + (i & 3) * 4;
  const int row = g * 4 + (i >> 2);
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(tile + roff<TT, kQD, kQLayout>(row, col)));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(tile + roff<TT, kQD, kQLayout>(row + 16, col)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(typename TT::vec, v);
}

// A operand of a score product: key row m of the row-major tile, dims 32 ks + 8 g .. + 7.
template <class TT>
__device__ inline typename TT::vec q16_row_op(const typename TT::elem* tile, int m, int ks, int g) {
  return *reinterpret_cast<const typename TT::vec*>(tile + roff<TT, kQD, kQLayout>(m, ks * 32 + g * 8));
}

// gQ, gdO at dims 16 mt + 4 g .. + 3 of query qi.
template <class TT>
__device__ inline void q16_epilogue_quad(const f32x4& A, const f32x4& B, const f32x4& C, const f32x4& X, float alpha,
                                         float e0, int qi, int g, int bh, int mt, const Pass1Args& a) {
  using T = typename TT::elem;
  if (qi >= a.N) return;
  const size_t row = (size_t)bh * a.N + qi;
  const int dim = mt * 16 + g * 4;
  float o[4], q[4], x[4];
  load4<TT>(reinterpret_cast<const T*>(a.O) + row * kQD + dim, o);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    q[e] = a.tau * (A[e] - alpha * B[e] - e0 * C[e]);
    x[e] = X[e] - alpha * o[e];
  }
  store4<TT>(reinterpret_cast<T*>(a.gQ) + row * kQD + dim, q[0], q[1], q[2], q[3]);
  store4<TT>(reinterpret_cast<T*>(a.gdO) + row * kQD + dim, x[0], x[1], x[2], x[3]);
}

// alpha, E and, for pass 2, L log2(e) and c = alpha D + E of query qi.
__device__ inline void q16_write_scalars(float alpha, float e0, int qi, int bh, const Pass1Args& a) {
  if (qi >= a.N) return;
  const size_t row = (size_t)bh * a.N + qi;
  const float dq = a.D[row];
  const float E = e0 - alpha * dq;
  a.alpha[row] = alpha;
  a.E[row] = E;
  a.l2[row] = a.L[row] * kLog2e;
  a.c[row] = fmaf(alpha, dq, E);
}

// Record of one wave: acc[4 tensors][8 dim tiles][64 lanes][4], alpha_p[64], e0_p[64].
__device__ inline float* q16_record(const Pass1Args& a, int split, int bh, int qt, int wave) {
  const size_t rec = (((size_t)split * a.BH + bh) * pass1_q16_tiles(a.N) + qt) * kQWaves + wave;
  return a.part + rec * pass1_q16_record_floats();
}

template <class TT, bool CAUSAL>
__global__ __launch_bounds__(kBlock, 1) void bob_pass1_q16_kernel(Pass1Args a) {
  using T = typename TT::elem;
  using V = typename TT::vec;
  static_assert(TT::KPL == 8, "16-bit inputs only");
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 4, n = lane & 15;
  int qt, bh;
  tile_and_head<CAUSAL, true>(qt, bh);
  const int N = a.N, split = blockIdx.z;
  const size_t base = (size_t)bh * N * kQD;
  // pass 2's merge counters (kReduceLastBlock) count 128-key tiles: one per two of ours
  if (a.p2_counters && split == 0 && (qt & 1) == 0 && threadIdx.x == 0)
    a.p2_counters[(size_t)bh * row_tiles(N) + (qt >> 1)] = 0u;
  const T* src[4] = {reinterpret_cast<const T*>(a.K) + base, reinterpret_cast<const T*>(a.V) + base,
                     reinterpret_cast<const T*>(a.UK) + base, reinterpret_cast<const T*>(a.UV) + base};
  const int q0 = qt * (kQWaves * kQRows) + wave * kQRows;
  const int qi = q0 + n;

  // B operands held for the whole sweep: query qi (zero past N), dims 32 ks + 8 g .. + 7
  V bq[4], bdo[4], buq[4];
  {
    const T* q = reinterpret_cast<const T*>(a.Q) + base;
    const T* d = reinterpret_cast<const T*>(a.dO) + base;
    const T* u = reinterpret_cast<const T*>(a.UQ) + base;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (qi < N) {
        const size_t off = (size_t)qi * kQD + ks * 32 + g * 8;
        bq[ks] = *reinterpret_cast<const V*>(q + off);
        bdo[ks] = *reinterpret_cast<const V*>(d + off);
        buq[ks] = *reinterpret_cast<const V*>(u + off);
      } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          bq[ks][s] = TT::cvt(0.f);
          bdo[ks][s] = TT::cvt(0.f);
          buq[ks][s] = TT::cvt(0.f);
        }
      }
    }
  }
  const size_t rowv = (size_t)bh * N + (qi < N ? qi : 0);
  const float lq = a.L[rowv] * kLog2e;
  const float dq = a.D[rowv];
  const float cs = a.tau * kLog2e;
  const float tau = a.tau;

  f32x4 accA[8], accB[8], accC[8], accX[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    accA[mt] = q16_zero4();
    accB[mt] = q16_zero4();
    accC[mt] = q16_zero4();
    accX[mt] = q16_zero4();
  }
  float alpha_p = 0.f, e0_p = 0.f;

  int nkt = (N + 31) / 32;
  if (CAUSAL) nkt = min(nkt, (qt + 1) * (kQWaves * kQRows / 32));
  const int kt_begin = (int)((long long)split * nkt / a.nsplit);
  const int kt_end = (int)((long long)(split + 1) * nkt / a.nsplit);
  const int nsteps = kt_end - kt_begin;
  auto active = [&](int j) { return !CAUSAL || (kt_begin + j) * 32 <= q0 + kQRows - 1; };
  // Copies from inline assembly (the compiler's own waits then never drain them early):
  // whole 32-key blocks in the scalar-base form, the ragged last block through
  // stage_direct, which repeats row N - 1. Each step ends with every copy landed.
  constexpr int CP = stage_copies<kQD, kQWaves>();
  unsigned coff[CP];
#pragma unroll
  for (int p = 0; p < CP; ++p) coff[p] = stage_lane_offset<kQD, kQWaves, kQLayout>(p, wave, lane);
  const unsigned lds_wave = lds_addr(lds) + (unsigned)wave * 1024u;
  auto issue = [&](int stg, int j) {
    const int r0 = (kt_begin + j) * 32;
    if (r0 + 32 <= N) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        stage_block_saddr<kQD, kQWaves>(src[t] + (size_t)r0 * kQD, coff,
                                        lds_wave + (unsigned)((stg * kQStageElems + t * kQTileElems) * (int)sizeof(T)));
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        stage_direct<TT, kQD, kQWaves, true, kQLayout>(src[t], r0, N, lds + stg * kQStageElems + t * kQTileElems,
                                                      wave, lane);
    }
  };
  settle_regs(bq, bdo, buq);
  settle_regs(lq, dq);
  for (int j = 0; j < kQNBuf - 1 && j < nsteps; ++j) issue(j, j);
  wait_vmem();
  __syncthreads();

  auto step = [&](auto S_c, int j) {
    constexpr int S = decltype(S_c)::value;
    if (j + kQNBuf - 1 < nsteps) issue((S + kQNBuf - 1) % kQNBuf, j + kQNBuf - 1);  // last read in step j - 1
    if (active(j)) {
      const T* st = lds + S * kQStageElems;
      const T *tk = st, *tv = st + kQTileElems, *tuk = st + 2 * kQTileElems, *tuv = st + 3 * kQTileElems;
      f32x4 sc[2], gc[2], pc[2], hc[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        sc[kt] = q16_zero4();
        gc[kt] = q16_zero4();
        pc[kt] = q16_zero4();
        hc[kt] = q16_zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int m = kt * 16 + n;
          const V ak = q16_row_op<TT>(tk, m, ks, g);
          const V av = q16_row_op<TT>(tv, m, ks, g);
          const V auk = q16_row_op<TT>(tuk, m, ks, g);
          const V auv = q16_row_op<TT>(tuv, m, ks, g);
          sc[kt] = mfma_16x16x32<TT>(ak, bq[ks], sc[kt]);
          gc[kt] = mfma_16x16x32<TT>(ak, buq[ks], gc[kt]);
          gc[kt] = mfma_16x16x32<TT>(auk, bq[ks], gc[kt]);
          pc[kt] = mfma_16x16x32<TT>(av, bdo[ks], pc[kt]);
          hc[kt] = mfma_16x16x32<TT>(auv, bdo[ks], hc[kt]);
        }
      }
      // log2-domain scores, masked where the key is out of range or after the query
      const int k0 = (kt_begin + j) * 32;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s = 0; s < 4; ++s) sc[kt][s] = sc[kt][s] * cs - lq;
      if (k0 + 32 > N || (CAUSAL && k0 + 31 > q0)) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int key = k0 + kt * 16 + g * 4 + s;
            if (!(key < N && (!CAUSAL || key <= qi))) sc[kt][s] = -INFINITY;
          }
      }
      V wa, wb, pp, pg;  // k-slot 4 kt + s
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float p = fast_exp2(sc[kt][s]);
          const float gv = gc[kt][s] * tau;
          const float t1 = pc[kt][s] - dq;
          const float vpg = p * gv;
          const float vwb = p * fmaf(gv, t1, hc[kt][s]);
          alpha_p += vpg;
          e0_p += vwb;
          const int k = kt * 4 + s;
          wa[k] = TT::cvt(p * t1);
          wb[k] = TT::cvt(vwb);
          pp[k] = TT::cvt(p);
          pg[k] = TT::cvt(vpg);
        }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const V ok = q16_tr_op<TT>(tk, mt, lane);
        const V ouk = q16_tr_op<TT>(tuk, mt, lane);
        const V ov = q16_tr_op<TT>(tv, mt, lane);
        const V ouv = q16_tr_op<TT>(tuv, mt, lane);
        mfma16_acc<TT>(accA[mt], ouk, wa);  // W_a UK
        mfma16_acc<TT>(accB[mt], ok, wa);   // W_a K
        mfma16_acc<TT>(accX[mt], ouv, pp);  // P UV
        mfma16_acc<TT>(accA[mt], ok, wb);   // W_b K
        mfma16_acc<TT>(accC[mt], ok, pp);   // P K
        mfma16_acc<TT>(accX[mt], ov, pg);   // (P G) V
      }
    }
    wait_vmem();
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  int j = 0;
  for (; j + kQNBuf <= nsteps; j += kQNBuf) {
    step(I0{}, j);
    step(I1{}, j + 1);
    step(I2{}, j + 2);
  }
  if (j < nsteps) step(I0{}, j);
  if (j + 1 < nsteps) step(I1{}, j + 1);
  acc16_settle<8>(accA, accB, accC, accX);

  if (a.nsplit == 1) {
    // the four lane groups of a query: (x0 + x1) + (x2 + x3) on every lane
    float alpha = alpha_p + __shfl_xor(alpha_p, 16);
    alpha += __shfl_xor(alpha, 32);
    float e0 = e0_p + __shfl_xor(e0_p, 16);
    e0 += __shfl_xor(e0, 32);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      q16_epilogue_quad<TT>(accA[mt], accB[mt], accC[mt], accX[mt], alpha, e0, qi, g, bh, mt, a);
    if (g == 0) q16_write_scalars(alpha, e0, qi, bh, a);
    return;
  }
  float* R = q16_record(a, split, bh, qt, wave);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    reinterpret_cast<f32x4*>(R)[(0 * 8 + mt) * 64 + lane] = accA[mt];
    reinterpret_cast<f32x4*>(R)[(1 * 8 + mt) * 64 + lane] = accB[mt];
    reinterpret_cast<f32x4*>(R)[(2 * 8 + mt) * 64 + lane] = accC[mt];
    reinterpret_cast<f32x4*>(R)[(3 * 8 + mt) * 64 + lane] = accX[mt];
  }
  R[128 * 64 + lane] = alpha_p;
  R[128 * 64 + 64 + lane] = e0_p;
}

// Merge of the split records in split order. A workgroup takes one wave's record and
// four of its dim tiles (grid z = which four); thread t handles record lane t / 4 and
// dim tile 4 z + t % 4 (16 contiguous bytes of each tensor) and sums the row partials
// of its query over the splits and the four lane groups.
template <class TT>
__global__ __launch_bounds__(kBlock) void bob_pass1_q16_combine_kernel(Pass1Args a) {
  const int L = threadIdx.x >> 2, mt = (threadIdx.x & 3) + 4 * blockIdx.z;
  const int g = L >> 4, n = L & 15;
  const int qt = blockIdx.x / kQWaves, wave = blockIdx.x % kQWaves, bh = blockIdx.y;
  const int qi = qt * (kQWaves * kQRows) + wave * kQRows + n;
  f32x4 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = q16_zero4();
  float al[4] = {0.f, 0.f, 0.f, 0.f}, el[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* R = q16_record(a, sp, bh, qt, wave);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += reinterpret_cast<const f32x4*>(R)[(k * 8 + mt) * 64 + L];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      al[q] += R[128 * 64 + n + 16 * q];
      el[q] += R[128 * 64 + 64 + n + 16 * q];
    }
  }
  const float alpha = (al[0] + al[1]) + (al[2] + al[3]);
  const float e0 = (el[0] + el[1]) + (el[2] + el[3]);
  q16_epilogue_quad<TT>(acc[0], acc[1], acc[2], acc[3], alpha, e0, qi, g, bh, mt, a);
  if (g == 0 && mt == 0) q16_write_scalars(alpha, e0, qi, bh, a);
}

template <class TT, bool CAUSAL>
static hipError_t launch_q16_t(const Pass1Args& a, hipStream_t s) {
  const size_t lds = (size_t)kQNBuf * kQStageElems * sizeof(typename TT::elem);
  hipError_t e = ensure_lds(&bob_pass1_q16_kernel<TT, CAUSAL>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_pass1_q16_kernel<TT, CAUSAL>), dim3(pass1_q16_tiles(a.N), a.BH, a.nsplit), dim3(kBlock),
                     lds, s, a);
  return hipGetLastError();
}

hipError_t launch_pass1_q16(const Pass1Args& a, DT dt, bool causal, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return causal ? launch_q16_t<BF16, true>(a, s) : launch_q16_t<BF16, false>(a, s);
    case DT::F16: return causal ? launch_q16_t<F16, true>(a, s) : launch_q16_t<F16, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pass1_q16_combine(const Pass1Args& a, DT dt, hipStream_t s) {
  const dim3 grid(pass1_q16_tiles(a.N) * kQWaves, a.BH, 2);
  switch (dt) {
    case DT::BF16: hipLaunchKernelGGL(bob_pass1_q16_combine_kernel<BF16>, grid, dim3(kBlock), 0, s, a); break;
    case DT::F16: hipLaunchKernelGGL(bob_pass1_q16_combine_kernel<F16>, grid, dim3(kBlock), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fb
