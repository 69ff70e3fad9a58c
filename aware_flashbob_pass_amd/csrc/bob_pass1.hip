// BoB pass 1: query-tile parallel. Produces gQ, gdO and the two row scalars.
//
// FlashBoB review page (Summary; Strengths on Prop. 4.1): the softmax double
// backward has a hierarchical affine structure in which two row scalars,
// alpha and E, enter every output affinely, so one sweep over the keys per
// query tile can accumulate alpha-free sums and apply the scalars at the end.
// Written out for row i (sums over keys j; G = tau (UQ K^T + Q UK^T),
// H = dO UV^T, dP = dO V^T, P = exp(tau Q K^T - L)):
//   alpha_i = sum_j P G,                   E_i = sum_j W_b - alpha_i D_i,
//   W_a = P (dP - D),  W_b = P (G (dP - D) + H),
//   gQ_i  = tau [ (W_a UK + W_b K) - alpha_i W_a K - e0_i P K ],  e0_i = sum_j W_b,
//   gdO_i = (P UV + (P G) V) - alpha_i O_i.
// The six alpha-free contractions W_a UK, W_b K, W_a K, P K, P UV and
// (P G) V accumulate into four float32 register tiles (A, B, C, X below); the
// pages name six alpha-free accumulators without listing them, and this is our
// reading of them.
//
// Each workgroup owns 128 queries (4 waves x 32) and a contiguous range of key
// tiles (the whole key range, or one of `nsplit` parts of it). With splits,
// each wave writes its raw accumulators and row partial sums as a record and
// a combine kernel sums the records in split order and applies the epilogue.
//
// This file holds the float32 kernel, the split merges, the four-pass modes and
// the launches; the staged 16-bit kernel template is in pass1_kernel.hpp and its
// two-pass instances are built in bob_pass1_vgpr.hip.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "pass1_common.hpp"
#include "pass1_kernel.hpp"

namespace fb {

// Single-buffered variant (transposed LDS copies); used for float32 inputs.
template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kBlock) void bob_pass1_simple_kernel(Pass1Args a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB;
  extern __shared__ __align__(16) unsigned char smem[];
  T* k_r = reinterpret_cast<T*>(smem);
  T* v_r = k_r + G::ROW_ELEMS;
  T* uk_r = v_r + G::ROW_ELEMS;
  T* uv_r = uk_r + G::ROW_ELEMS;
  T* k_t = uv_r + G::ROW_ELEMS;
  T* v_t = k_t + G::T_ELEMS;
  T* uk_t = v_t + G::T_ELEMS;
  T* uv_t = uk_t + G::T_ELEMS;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  const int N = a.N, bh = blockIdx.y, split = blockIdx.z;
  const size_t base = (size_t)bh * N * D;
  const T* Q = reinterpret_cast<const T*>(a.Q) + base;
  const T* K = reinterpret_cast<const T*>(a.K) + base;
  const T* Vm = reinterpret_cast<const T*>(a.V) + base;
  const T* dO = reinterpret_cast<const T*>(a.dO) + base;
  const T* UQ = reinterpret_cast<const T*>(a.UQ) + base;
  const T* UK = reinterpret_cast<const T*>(a.UK) + base;
  const T* UV = reinterpret_cast<const T*>(a.UV) + base;
  const int q0 = blockIdx.x * kBlockRows + wave * kTile;
  const int qi = q0 + n;

  V bq[G::DK], bdo[G::DK], buq[G::DK];
  load_resident<TT, D>(Q, qi, N, g, bq);
  load_resident<TT, D>(dO, qi, N, g, bdo);
  load_resident<TT, D>(UQ, qi, N, g, buq);
  const size_t rowv = (size_t)bh * N + (qi < N ? qi : 0);
  const float lq = a.L[rowv] * kLog2e;
  const float dq = a.D[rowv];
  const float cs = a.tau * kLog2e;
  const float tau = a.tau;

  f32x16 accA[MB], accB[MB], accC[MB], accX[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accA[mb] = zero16();
    accB[mb] = zero16();
    accC[mb] = zero16();
    accX[mb] = zero16();
  }
  float alpha_p = 0.f, e0_p = 0.f;

  int nkt = (N + kTile - 1) / kTile;
  if (CAUSAL) nkt = min(nkt, (int)(blockIdx.x + 1) * (kBlockRows / kTile));
  const int kt_begin = (int)((long long)split * nkt / a.nsplit);
  const int kt_end = (int)((long long)(split + 1) * nkt / a.nsplit);

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int k0 = kt * kTile;
    __syncthreads();
    stage_tile<TT, D>(K, k0, N, k_r, k_t, tid, kBlock);
    stage_tile<TT, D>(Vm, k0, N, v_r, v_t, tid, kBlock);
    stage_tile<TT, D>(UK, k0, N, uk_r, uk_t, tid, kBlock);
    stage_tile<TT, D>(UV, k0, N, uv_r, uv_t, tid, kBlock);
    __syncthreads();
    if (CAUSAL && k0 > q0 + kTile - 1) continue;

    // score tiles (keys x queries): S, G, dP, H
    f32x16 s = zero16(), gg = zero16(), dp = zero16(), h = zero16();
#pragma unroll
    for (int t = 0; t < G::DK; ++t) {
      const V ak = lds_row_op<TT, D>(k_r, n, t, g);
      const V auk = lds_row_op<TT, D>(uk_r, n, t, g);
      const V av = lds_row_op<TT, D>(v_r, n, t, g);
      const V auv = lds_row_op<TT, D>(uv_r, n, t, g);
      s = TT::mfma(ak, bq[t], s);
      gg = TT::mfma(ak, buq[t], gg);
      gg = TT::mfma(auk, bq[t], gg);
      dp = TT::mfma(av, bdo[t], dp);
      h = TT::mfma(auv, bdo[t], h);
    }

    // element-wise weights
    V wa[G::NK], wb[G::NK], pp[G::NK], pg[G::NK];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + kappa(r, g);
      const bool ok = key < N && (!CAUSAL || key <= qi);
      const float p = ok ? fast_exp2(s[r] * cs - lq) : 0.f;
      const float gv = gg[r] * tau;
      const float dpv = dp[r];
      const float t1 = dpv - dq;
      const float vpg = p * gv;
      const float vwb = p * (gv * t1 + h[r]);
      alpha_p += vpg;
      e0_p += vwb;
      const int kk = r / TT::KPL, ss = r % TT::KPL;
      vset<TT>(wa[kk], ss, p * t1);
      vset<TT>(wb[kk], ss, vwb);
      vset<TT>(pp[kk], ss, p);
      vset<TT>(pg[kk], ss, vpg);
    }

    // alpha-free accumulators (head dims x queries)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int dim = mb * 32 + n;
#pragma unroll
      for (int t = 0; t < G::NK; ++t) {
        const V tk = lds_t_op<TT, D>(k_t, dim, t, g);
        const V tuk = lds_t_op<TT, D>(uk_t, dim, t, g);
        const V tv = lds_t_op<TT, D>(v_t, dim, t, g);
        const V tuv = lds_t_op<TT, D>(uv_t, dim, t, g);
        accA[mb] = TT::mfma(tuk, wa[t], accA[mb]);
        accA[mb] = TT::mfma(tk, wb[t], accA[mb]);
        accB[mb] = TT::mfma(tk, wa[t], accB[mb]);  // W_a K
        accC[mb] = TT::mfma(tk, pp[t], accC[mb]);
        accX[mb] = TT::mfma(tuv, pp[t], accX[mb]);
        accX[mb] = TT::mfma(tv, pg[t], accX[mb]);
      }
    }
  }

  if (a.nsplit == 1) {
    pass1_epilogue<TT, D>(accA, accB, accC, accX, alpha_p, e0_p, qi, g, bh, a);
    return;
  }
  pass1_write_record<TT, D>(accA, accB, accC, accX, alpha_p, e0_p, split, bh, blockIdx.x, wave, lane, a);
}

template <class TT, int D, int MODE>
__global__ __launch_bounds__(kBlock) void fourpass_combine_kernel(Pass1Args a) {
  constexpr int MB = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  const int bh = blockIdx.y;
  const int qi = blockIdx.x * kBlockRows + wave * kTile + n;
  f32x16 Q[MB], X[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    Q[mb] = zero16();
    X[mb] = zero16();
  }
  float s_p = 0.f;
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* R = fourpass_record<TT, D, MODE>(a, sp, bh, blockIdx.x, wave);
    if constexpr (MODE == kDqPass) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) Q[mb] += load_tile16(R + mb * 1024, lane);
    } else if constexpr (MODE == kRowsPass) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        Q[mb] += load_tile16(R + (0 * MB + mb) * 1024, lane);
        X[mb] += load_tile16(R + (1 * MB + mb) * 1024, lane);
      }
    } else {
      s_p += R[lane];
    }
  }
  fourpass_epilogue<TT, D, MODE>(Q, X, s_p, qi, g, bh, a);
}

// Sum the split records of one wave in split order and apply the epilogue. A
// workgroup takes one wave's record and one 32-wide head-dim block (grid x = query
// tile x wave, z = block); thread t sums slots 4 (t / 64) .. 4 (t / 64) + 3 of
// record lane t % 64, so consecutive threads read consecutive 16 bytes of the
// quad-major record tiles and four times as many waves are in flight as with one
// thread per record lane. The sums are formed in the same order as in
// one-lane-per-thread form (split by split, then the row's lane pair), and block 0
// writes the row scalars.
template <class TT, int D>
__global__ __launch_bounds__(kBlock) void bob_pass1_combine_kernel(Pass1Args a) {
  constexpr int MB = P1<TT, D>::MBA;
  constexpr int ACC = P1<TT, D>::ACC_FLOATS;
  const int L = threadIdx.x & 63, r4 = threadIdx.x >> 6;
  const int g = L >> 5, n = L & 31;
  const int qt = blockIdx.x >> 2, wave = blockIdx.x & 3;
  const int bh = blockIdx.y, mbl = blockIdx.z;
  const int qi = qt * kBlockRows + wave * kTile + n;
  f32x4 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float alo = 0.f, ahi = 0.f, elo = 0.f, ehi = 0.f;
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* R = pass1_record<TT, D>(a, sp, bh, qt, wave);
    f32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = tile_quad(R + (k * MB + mbl) * 1024, L, r4);
    alo += R[ACC + n];
    ahi += R[ACC + 32 + n];
    elo += R[ACC + 64 + n];
    ehi += R[ACC + 96 + n];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] += v[k];
  }
  const float alpha = alo + ahi, e0 = elo + ehi;
  pass1_epilogue_quad<TT, D>(acc[0], acc[1], acc[2], acc[3], alpha, e0, qi, g, bh, mbl, r4, a);
  if (blockIdx.z == 0 && r4 == 0) pass1_write_scalars(alpha, e0, qi, g, bh, a);
}

template <class TT, int D, bool CAUSAL>
static hipError_t launch_p1_t(const Pass1Args& a, hipStream_t s) {
  const size_t lds = pass1_lds_bytes<TT, D>();
  dim3 grid(row_tiles(a.N), a.BH, a.nsplit);
  if constexpr (TT::KPL == 1) {
    hipError_t e = ensure_lds(&bob_pass1_simple_kernel<TT, D, CAUSAL>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bob_pass1_simple_kernel<TT, D, CAUSAL>), grid, dim3(kBlock), lds, s, a);
  } else if constexpr (D == 64) {
    return launch_pass1_d64(a, std::is_same_v<TT, BF16> ? DT::BF16 : DT::F16, CAUSAL, s);
  } else if constexpr (D == 128) {
    return hipErrorInvalidValue;  // 16-bit d = 128 runs bob_pass1_q16_kernel (launch_pass1_q16)
  } else {
    hipError_t e = ensure_lds(&bob_pass1_kernel<TT, D, CAUSAL, kTwoPass>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bob_pass1_kernel<TT, D, CAUSAL, kTwoPass>), grid, dim3(kBlock), lds, s, a);
  }
  return hipGetLastError();
}

template <class TT>
static hipError_t launch_p1_tt(const Pass1Args& a, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch_p1_t<TT, 64, true>(a, s) : launch_p1_t<TT, 64, false>(a, s);
  return causal ? launch_p1_t<TT, 128, true>(a, s) : launch_p1_t<TT, 128, false>(a, s);
}

hipError_t launch_pass1(const Pass1Args& a, DT dt, int d, bool causal, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_p1_tt<BF16>(a, d, causal, s);
    case DT::F16: return launch_p1_tt<F16>(a, d, causal, s);
    default: return launch_p1_tt<F32>(a, d, causal, s);
  }
}

template <class TT, int D>
static hipError_t launch_c1_t(const Pass1Args& a, hipStream_t s) {
  dim3 grid(row_tiles(a.N) * 4, a.BH, P1<TT, D>::MBA);  // one workgroup per wave record
  hipLaunchKernelGGL((bob_pass1_combine_kernel<TT, D>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pass1_combine(const Pass1Args& a, DT dt, int d, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return d == 64 ? launch_c1_t<BF16, 64>(a, s) : launch_c1_t<BF16, 128>(a, s);
    case DT::F16: return d == 64 ? launch_c1_t<F16, 64>(a, s) : launch_c1_t<F16, 128>(a, s);
    default: return d == 64 ? launch_c1_t<F32, 64>(a, s) : launch_c1_t<F32, 128>(a, s);
  }
}

// ---- four-pass ablation launchers (16-bit inputs) ----------------------------
template <class TT, int D, bool CAUSAL, int MODE>
static hipError_t launch_fp_t(const Pass1Args& a, hipStream_t s) {
  const size_t lds = pass1_lds_bytes<TT, D>();
  hipError_t e = ensure_lds(&bob_pass1_kernel<TT, D, CAUSAL, MODE>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_pass1_kernel<TT, D, CAUSAL, MODE>), dim3(row_tiles(a.N), a.BH, a.nsplit), dim3(kBlock), lds,
                     s, a);
  if ((e = hipGetLastError()) != hipSuccess || a.nsplit == 1) return e;
  hipLaunchKernelGGL((fourpass_combine_kernel<TT, D, MODE>), dim3(row_tiles(a.N), a.BH), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

template <class TT, int MODE>
static hipError_t launch_fp_m(const Pass1Args& a, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch_fp_t<TT, 64, true, MODE>(a, s) : launch_fp_t<TT, 64, false, MODE>(a, s);
  return causal ? launch_fp_t<TT, 128, true, MODE>(a, s) : launch_fp_t<TT, 128, false, MODE>(a, s);
}

template <class TT>
static hipError_t launch_fp_tt(const Pass1Args& a, int sweep, int d, bool causal, hipStream_t s) {
  switch (sweep) {
    case 0: return launch_fp_m<TT, kAlphaPass>(a, d, causal, s);
    case 1: return launch_fp_m<TT, kEnergyPass>(a, d, causal, s);
    default: return launch_fp_m<TT, kRowsPass>(a, d, causal, s);
  }
}

hipError_t launch_first_bwd_dq(const Pass1Args& a, DT dt, int d, bool causal, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_fp_m<BF16, kDqPass>(a, d, causal, s);
    case DT::F16: return launch_fp_m<F16, kDqPass>(a, d, causal, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fourpass_sweep(const Pass1Args& a, int sweep, DT dt, int d, bool causal, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_fp_tt<BF16>(a, sweep, d, causal, s);
    case DT::F16: return launch_fp_tt<F16>(a, sweep, d, causal, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fb
