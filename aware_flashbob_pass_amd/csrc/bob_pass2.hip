// BoB pass 2: key-tile parallel. Produces gK and gV.
//
// After pass 1 every query row's scalars L, D, alpha, E are known (review page,
// Summary: only the two length-N vectors alpha and E cross the pass boundary,
// besides the statistics). For key j, summing over queries i:
//   dS   = P (dP - D),
//   Sbar = P (G (dP - D) - alpha dP + H - E),      (cotangent of the scores)
//   dPbar = P (G - alpha),                          (cotangent of dP)
//   gK_j = tau sum_i (dS_ij UQ_i + Sbar_ij Q_i),    gV_j = sum_i dPbar_ij dO_i,
// with G = tau (UQ K^T + Q UK^T), H = dO UV^T, dP = dO V^T, P = exp(tau Q K^T - L).
//
// Each workgroup owns 128 keys (4 waves x 32), keeps K, V, UK, UV rows of its
// keys in registers as matrix-core B operands, and streams 32-query tiles of
// Q, dO, UQ (row-major and transposed copies) and the four row scalars
// through LDS. With splits of the query range, each wave writes raw
// accumulators and a reduce kernel sums them in split order.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace fb {

// gK_j and gV_j at the 4 head dims of slots 4 r4 .. 4 r4 + 3 of head-dim block mb.
template <class TT, int D>
__device__ inline void pass2_epilogue_quad(const f32x4& dK, const f32x4& dV, int kj, int g, int bh, int mb, int r4,
                                           const Pass2Args& a) {
  using T = typename TT::elem;
  if (kj >= a.N) return;
  const size_t row = (size_t)bh * a.N + kj;
  const int dim = mb * 32 + kappa(r4 * 4, g);
  const float tau = a.tau;
  store4<TT>(reinterpret_cast<T*>(a.gK) + row * D + dim, tau * dK[0], tau * dK[1], tau * dK[2], tau * dK[3]);
  store4<TT>(reinterpret_cast<T*>(a.gV) + row * D + dim, dV[0], dV[1], dV[2], dV[3]);
}

template <class TT, int D>
__device__ inline void pass2_epilogue_block(const f32x16& dK, const f32x16& dV, int kj, int g, int bh, int mb,
                                            const Pass2Args& a) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    const f32x4 k4 = {dK[r4 * 4], dK[r4 * 4 + 1], dK[r4 * 4 + 2], dK[r4 * 4 + 3]};
    const f32x4 v4 = {dV[r4 * 4], dV[r4 * 4 + 1], dV[r4 * 4 + 2], dV[r4 * 4 + 3]};
    pass2_epilogue_quad<TT, D>(k4, v4, kj, g, bh, mb, r4, a);
  }
}

template <class TT, int D>
__device__ inline void pass2_epilogue(const f32x16 (&dK)[Geo<TT, D>::MB], const f32x16 (&dV)[Geo<TT, D>::MB],
                                      int kj, int g, int bh, const Pass2Args& a) {
#pragma unroll
  for (int mb = 0; mb < Geo<TT, D>::MB; ++mb) pass2_epilogue_block<TT, D>(dK[mb], dV[mb], kj, g, bh, mb, a);
}

template <class TT, int D>
__device__ inline void pass2_write_record(const f32x16 (&dK)[Geo<TT, D>::MB], const f32x16 (&dV)[Geo<TT, D>::MB],
                                          int split, int bh, int kt, int wave, int lane, const Pass2Args& a) {
  constexpr int MB = Geo<TT, D>::MB;
  const size_t rec = (((size_t)split * a.BH + bh) * row_tiles(a.N) + kt) * 4 + wave;
  float* R = a.part + rec * pass2_record_floats(D);  // [2][MB][64 lanes][16]
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    store_acc16(R + ((0 * MB + mb) * 64 + lane) * 16, dK[mb]);
    store_acc16(R + ((1 * MB + mb) * 64 + lane) * 16, dV[mb]);
  }
}

// Single-buffered variant (transposed LDS copies); used for float32 inputs.
template <class TT, int D, bool CAUSAL>
__global__ __launch_bounds__(kBlock) void bob_pass2_simple_kernel(Pass2Args a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB;
  extern __shared__ __align__(16) unsigned char smem[];
  T* q_r = reinterpret_cast<T*>(smem);
  T* do_r = q_r + G::ROW_ELEMS;
  T* uq_r = do_r + G::ROW_ELEMS;
  T* q_t = uq_r + G::ROW_ELEMS;
  T* do_t = q_t + G::T_ELEMS;
  T* uq_t = do_t + G::T_ELEMS;
  float* sc = reinterpret_cast<float*>(uq_t + G::T_ELEMS);  // [4][32]: L*log2e, D, alpha, E

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  const int N = a.N, bh = blockIdx.y, split = blockIdx.z;
  const size_t base = (size_t)bh * N * D;
  const size_t vbase = (size_t)bh * N;
  const T* Q = reinterpret_cast<const T*>(a.Q) + base;
  const T* dO = reinterpret_cast<const T*>(a.dO) + base;
  const T* UQ = reinterpret_cast<const T*>(a.UQ) + base;
  const int k0w = blockIdx.x * kBlockRows + wave * kTile;
  const int kj = k0w + n;

  V bk[G::DK], bv[G::DK], buk[G::DK], buv[G::DK];
  load_resident<TT, D>(reinterpret_cast<const T*>(a.K) + base, kj, N, g, bk);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.V) + base, kj, N, g, bv);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.UK) + base, kj, N, g, buk);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.UV) + base, kj, N, g, buv);
  const float cs = a.tau * kLog2e;
  const float tau = a.tau;

  f32x16 accK[MB], accV[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accK[mb] = zero16();
    accV[mb] = zero16();
  }

  const int nqt = (N + kTile - 1) / kTile;
  const int qt_first = CAUSAL ? (int)blockIdx.x * (kBlockRows / kTile) : 0;
  const int span = nqt - qt_first;
  const int it_begin = qt_first + (int)((long long)split * span / a.nsplit);
  const int it_end = qt_first + (int)((long long)(split + 1) * span / a.nsplit);

  for (int it = it_begin; it < it_end; ++it) {
    const int i0 = it * kTile;
    __syncthreads();
    stage_tile<TT, D>(Q, i0, N, q_r, q_t, tid, kBlock);
    stage_tile<TT, D>(dO, i0, N, do_r, do_t, tid, kBlock);
    stage_tile<TT, D>(UQ, i0, N, uq_r, uq_t, tid, kBlock);
    if (tid < 4 * kTile) {
      const int which = tid / kTile, rr = tid % kTile;
      const int qrow = i0 + rr;
      float v = 0.f;
      if (qrow < N) {
        if (which == 0) v = a.L[vbase + qrow] * kLog2e;
        else if (which == 1) v = a.D[vbase + qrow];
        else if (which == 2) v = a.alpha[vbase + qrow];
        else v = a.E[vbase + qrow];
      }
      sc[tid] = v;
    }
    __syncthreads();
    if (CAUSAL && i0 + kTile - 1 < k0w) continue;  // every query before every key of this wave

    // score tiles (queries x keys): S, G, dP, H
    f32x16 s = zero16(), gg = zero16(), dp = zero16(), h = zero16();
#pragma unroll
    for (int t = 0; t < G::DK; ++t) {
      const V aq = lds_row_op<TT, D>(q_r, n, t, g);
      const V auq = lds_row_op<TT, D>(uq_r, n, t, g);
      const V ado = lds_row_op<TT, D>(do_r, n, t, g);
      s = TT::mfma(aq, bk[t], s);
      gg = TT::mfma(auq, bk[t], gg);
      gg = TT::mfma(aq, buk[t], gg);
      dp = TT::mfma(ado, bv[t], dp);
      h = TT::mfma(ado, buv[t], h);
    }

    V wds[G::NK], wsb[G::NK], wdp[G::NK];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = kappa(r, g);
      const int qrow = i0 + qr;
      const bool ok = qrow < N && kj < N && (!CAUSAL || kj <= qrow);
      const float lq = sc[qr], dq = sc[kTile + qr], al = sc[2 * kTile + qr], eq = sc[3 * kTile + qr];
      const float p = ok ? fast_exp2(s[r] * cs - lq) : 0.f;
      const float gv = gg[r] * tau;
      const float dpv = dp[r];
      const float t1 = dpv - dq;
      const int kk = r / TT::KPL, ss = r % TT::KPL;
      vset<TT>(wds[kk], ss, p * t1);
      vset<TT>(wsb[kk], ss, p * (gv * t1 - al * dpv + h[r] - eq));
      vset<TT>(wdp[kk], ss, p * (gv - al));
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int dim = mb * 32 + n;
#pragma unroll
      for (int t = 0; t < G::NK; ++t) {
        const V tuq = lds_t_op<TT, D>(uq_t, dim, t, g);
        const V tq = lds_t_op<TT, D>(q_t, dim, t, g);
        const V tdo = lds_t_op<TT, D>(do_t, dim, t, g);
        accK[mb] = TT::mfma(tuq, wds[t], accK[mb]);
        accK[mb] = TT::mfma(tq, wsb[t], accK[mb]);
        accV[mb] = TT::mfma(tdo, wdp[t], accV[mb]);
      }
    }
  }

  if (a.nsplit == 1) {
    pass2_epilogue<TT, D>(accK, accV, kj, g, bh, a);
    return;
  }
  pass2_write_record<TT, D>(accK, accV, split, bh, blockIdx.x, wave, lane, a);
}

// Staged variant for 16-bit inputs: three LDS stages of row-major Q, dO, UQ
// tiles plus their four row scalars, copied two steps ahead from inline
// assembly so that the end of a step waits only for the copies of the next one
// (the compiler does not see them and inserts no wait of its own); transposed
// operands come from the transposing LDS load. Each step forms its score tiles,
// its weights and its accumulating products in turn. At d = 64 the kernel fits
// 256 registers, so two waves share each SIMD (two workgroups per CU) and each
// one's matrix-core work overlaps the other's vector work; that beat forming
// the next step's tiles during the current step at one wave per SIMD.
template <class TT, int D, bool CAUSAL, bool FIRST = false>
__global__ __launch_bounds__(kBlock, (D == 64 ? 2 : 1)) void bob_pass2_kernel(Pass2Args a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB, DK = G::DK, NK = G::NK;
  constexpr int NT = 3, NBUF = 3, AHEAD = NBUF - 1;
  constexpr int STAGE_ELEMS = NT * G::ROW_ELEMS + 4 * kTile * 4 / (int)sizeof(T);  // tiles + 4 x 32 floats
  static_assert(TT::KPL == 8 && NK == 2, "16-bit inputs only");
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  int kt, bh;
  tile_and_head<CAUSAL, false>(kt, bh);
  const int N = a.N, split = blockIdx.z;
  const size_t base = (size_t)bh * N * D;
  const size_t vbase = (size_t)bh * N;
  const T* src[NT] = {reinterpret_cast<const T*>(a.Q) + base, reinterpret_cast<const T*>(a.dO) + base,
                      reinterpret_cast<const T*>(a.UQ) + base};
  // FIRST (the first backward g: dK = tau dS^T Q, dV = P^T dO) needs S and dP only:
  // no UQ tile, no UK / UV rows, and only the L and D row scalars.
  constexpr int NSCAL = FIRST ? 2 : 4;
  constexpr int COPIES = (FIRST ? 2 : 3) * stage_copies<D, kBlock / 64>() + 1;  // per wave and stage
  const float* vsrc[4] = {(FIRST ? a.L : a.l2) + vbase, a.D + vbase, FIRST ? nullptr : a.alpha + vbase,
                          FIRST ? nullptr : a.c + vbase};
  const int k0w = kt * kBlockRows + wave * kTile;
  const int kj = k0w + n;

  V bk[DK], bv[DK], buk[DK], buv[DK];
  load_resident<TT, D>(reinterpret_cast<const T*>(a.K) + base, kj, N, g, bk);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.V) + base, kj, N, g, bv);
  if constexpr (!FIRST) {
    load_resident<TT, D>(reinterpret_cast<const T*>(a.UK) + base, kj, N, g, buk);
    load_resident<TT, D>(reinterpret_cast<const T*>(a.UV) + base, kj, N, g, buv);
  }
  const float cs = a.tau * kLog2e;
  const float tau = a.tau;

  f32x16 accK[MB], accV[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accK[mb] = zero16();
    accV[mb] = zero16();
  }

  const int nqt = (N + kTile - 1) / kTile;
  const int qt_first = CAUSAL ? kt * (kBlockRows / kTile) : 0;
  const int span = nqt - qt_first;
  const int it_begin = qt_first + (int)((long long)split * span / a.nsplit);
  const int it_end = qt_first + (int)((long long)(split + 1) * span / a.nsplit);
  const int nsteps = it_end - it_begin;

  auto tile = [&](int j, int t) { return lds + (j % NBUF) * STAGE_ELEMS + t * G::ROW_ELEMS; };
  auto scal = [&](int j) { return reinterpret_cast<float*>(lds + (j % NBUF) * STAGE_ELEMS + NT * G::ROW_ELEMS); };
  auto active = [&](int j) { return !CAUSAL || (it_begin + j) * kTile + kTile - 1 >= k0w; };

  // Each stage also holds the row scalars of its 32 queries (rows >= N repeat row
  // N - 1): L log2(e), D, alpha and c = alpha D + E as pass 1 wrote them, so that
  // Sbar = P (Pbar - E) = dPbar (dP - D) + P (H - c) (Pbar = G (dP - D) - alpha dP
  // + H); the first backward stages L and D and scales L here. Wave w copies
  // scalar w % NSCAL with its lanes 0..31, so every wave issues the same number of
  // copies per stage (with NSCAL = 2 two waves write the same values).
  auto issue = [&](int stg, int j) {
    const int i0 = (it_begin + j) * kTile;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (!FIRST || t < 2) stage_direct<TT, D, kBlock / 64, true>(src[t], i0, N, tile(stg, t), wave, lane);
    const int which = wave % NSCAL;
    if (lane < kTile) glds4<true>(vsrc[which] + min(i0 + lane, N - 1), scal(stg) + which * kTile);
  };
  settle_regs(bk, bv);
  if constexpr (!FIRST) settle_regs(buk, buv);
  for (int j = 0; j < AHEAD && j < nsteps; ++j) issue(j, j);
  wait_vmem();
  __syncthreads();

  f32x16 sc, gc, pc, hc;  // score tiles of the current step
  auto scores_kstep = [&](int j, int t, f32x16& s_, f32x16& g_, f32x16& p_, f32x16& h_) {
    const V aq = lds_row_op<TT, D>(tile(j, 0), n, t, g);
    const V ado = lds_row_op<TT, D>(tile(j, 1), n, t, g);
    const V auq = lds_row_op<TT, D>(tile(j, 2), n, t, g);
    s_ = TT::mfma(aq, bk[t], s_);
    if constexpr (!FIRST) {
      g_ = TT::mfma(auq, bk[t], g_);
      g_ = TT::mfma(aq, buk[t], g_);
    }
    p_ = TT::mfma(ado, bv[t], p_);
    if constexpr (!FIRST) h_ = TT::mfma(ado, buv[t], h_);
  };
  auto step = [&](auto S_c, int j) {
    constexpr int S = decltype(S_c)::value;
    constexpr int SC = (S + AHEAD) % NBUF;
    const bool copies = j + AHEAD < nsteps;
    if (copies) issue(SC, j + AHEAD);  // buffer SC was last read in step j - 1
    const int i0 = (it_begin + j) * kTile;
    if (active(j)) {
      sc = zero16();
      gc = zero16();
      pc = zero16();
      hc = zero16();
#pragma unroll
      for (int t = 0; t < DK; ++t) scores_kstep(S, t, sc, gc, pc, hc);
      // Row scalars of the streamed queries: lane group g holds rows kappa(r, g), which
      // for r = 4 r4 .. 4 r4 + 3 are the 4 consecutive rows 8 r4 + 4 g .. + 3.
      const float* sv = scal(S);
      auto row4 = [&](int which, int r4) {
        return *reinterpret_cast<const f32x4*>(sv + which * kTile + r4 * 8 + g * 4);
      };
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 l4 = FIRST ? row4(0, r4) * kLog2e : row4(0, r4);
#pragma unroll
        for (int e = 0; e < 4; ++e) sc[r4 * 4 + e] = sc[r4 * 4 + e] * cs - l4[e];
      }
      if (i0 + kTile > N || (CAUSAL && i0 < k0w + kTile - 1)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = i0 + kappa(r, g);
          if (!(qrow < N && (!CAUSAL || kj <= qrow))) sc[r] = -INFINITY;
        }
      }
      V wds[NK], wsb[NK], wdp[NK];
      f32x4 d4, a4, c4;  // D, alpha, c of the current group of 4 rows (loaded at its first row)
      auto elementwise = [&](int r) {
        if ((r & 3) == 0) {
          d4 = row4(1, r >> 2);
          if constexpr (!FIRST) {
            a4 = row4(2, r >> 2);
            c4 = row4(3, r >> 2);
          }
        }
        const float dq = d4[r & 3];
        const float p = fast_exp2(sc[r]);
        const float dpv = pc[r];
        const float t1 = dpv - dq;
        const int kk = r >> 3, ss = r & 7;
        vset<TT>(wds[kk], ss, p * t1);  // dS
        if constexpr (FIRST) {
          vset<TT>(wdp[kk], ss, p);  // P
        } else {
          const float dpb = p * (gc[r] * tau - a4[r & 3]);           // dPbar = P (G - alpha)
          vset<TT>(wsb[kk], ss, fmaf(dpb, t1, p * (hc[r] - c4[r & 3])));  // Sbar
          vset<TT>(wdp[kk], ss, dpb);
        }
      };
#pragma unroll
      for (int t = 0; t < DK; ++t)
#pragma unroll
        for (int r = t * 8 / DK; r < (t + 1) * 8 / DK; ++r) elementwise(r);
#pragma unroll
      for (int t = 0; t < NK; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const V tuq = lds_tr_op<TT, D>(tile(S, 2), mb, t, lane);
          const V tq = lds_tr_op<TT, D>(tile(S, 0), mb, t, lane);
          const V tdo = lds_tr_op<TT, D>(tile(S, 1), mb, t, lane);
          if (t == 0) {
#pragma unroll
            for (int r = 8 + mb * 8 / MB; r < 8 + (mb + 1) * 8 / MB; ++r) elementwise(r);
          }
          if constexpr (FIRST) {
            accK[mb] = TT::mfma(tq, wds[t], accK[mb]);  // dS^T Q
          } else {
            accK[mb] = TT::mfma(tuq, wds[t], accK[mb]);  // dS^T UQ
            accK[mb] = TT::mfma(tq, wsb[t], accK[mb]);   // Sbar^T Q
          }
          accV[mb] = TT::mfma(tdo, wdp[t], accV[mb]);    // P^T dO or dPbar^T dO
        }
    }
    if (copies) wait_vmem_keep<COPIES>();  // this step's copies may stay in flight
    else wait_vmem();
    __syncthreads();
  };
  int j = 0;
  for (; j + NBUF <= nsteps; j += NBUF) unroll_steps(step, j, std::make_integer_sequence<int, NBUF>{});
  unroll_steps_until(step, j, nsteps, std::make_integer_sequence<int, NBUF - 1>{});

  if (a.nsplit == 1) {
    pass2_epilogue<TT, D>(accK, accV, kj, g, bh, a);
    return;
  }
  pass2_write_record<TT, D>(accK, accV, split, bh, kt, wave, lane, a);
}

// Sum the split records of one wave in split order and write one 32-wide head-dim
// block of gK, gV. A workgroup takes one wave's record and one block (grid x = key
// tile x wave, z = block); thread t sums slots 4 (t % 4) .. 4 (t % 4) + 3 of record
// lane t / 4, so consecutive threads read consecutive 16 bytes and four times as
// many waves are in flight as with one thread per record lane.
template <class TT, int D>
__global__ __launch_bounds__(kBlock) void bob_pass2_reduce_kernel(Pass2Args a) {
  constexpr int MB = Geo<TT, D>::MB;
  const int L = threadIdx.x >> 2, r4 = threadIdx.x & 3;
  const int g = L >> 5, n = L & 31;
  const int kt = blockIdx.x >> 2, wave = blockIdx.x & 3;
  const int bh = blockIdx.y, mb = blockIdx.z;
  const int kj = kt * kBlockRows + wave * kTile + n;
  const int kt_count = row_tiles(a.N);
  f32x4 dK = {0.f, 0.f, 0.f, 0.f}, dV = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* R = a.part + ((((size_t)sp * a.BH + bh) * kt_count + kt) * 4 + wave) * pass2_record_floats(D);
    const f32x4 k4 = *reinterpret_cast<const f32x4*>(R + ((0 * MB + mb) * 64 + L) * 16 + r4 * 4);
    const f32x4 v4 = *reinterpret_cast<const f32x4*>(R + ((1 * MB + mb) * 64 + L) * 16 + r4 * 4);
    dK += k4;
    dV += v4;
  }
  pass2_epilogue_quad<TT, D>(dK, dV, kj, g, bh, mb, r4, a);
}

template <class TT, int D>
static size_t pass2_lds_bytes() {
  using G = Geo<TT, D>;
  if constexpr (TT::KPL == 1)
    return (size_t)3 * (G::ROW_ELEMS + G::T_ELEMS) * sizeof(typename TT::elem) + 4 * kTile * sizeof(float);
  return (size_t)3 * (3 * G::ROW_ELEMS * sizeof(typename TT::elem) + 4 * kTile * sizeof(float));
}

template <class TT, int D, bool CAUSAL>
static hipError_t launch_p2_t(const Pass2Args& a, hipStream_t s) {
  const size_t lds = pass2_lds_bytes<TT, D>();
  dim3 grid(row_tiles(a.N), a.BH, a.nsplit);
  if constexpr (TT::KPL == 1) {
    hipError_t e = ensure_lds(&bob_pass2_simple_kernel<TT, D, CAUSAL>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bob_pass2_simple_kernel<TT, D, CAUSAL>), grid, dim3(kBlock), lds, s, a);
  } else {
    hipError_t e = ensure_lds(&bob_pass2_kernel<TT, D, CAUSAL>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bob_pass2_kernel<TT, D, CAUSAL>), grid, dim3(kBlock), lds, s, a);
  }
  return hipGetLastError();
}

template <class TT>
static hipError_t launch_p2_tt(const Pass2Args& a, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch_p2_t<TT, 64, true>(a, s) : launch_p2_t<TT, 64, false>(a, s);
  return causal ? launch_p2_t<TT, 128, true>(a, s) : launch_p2_t<TT, 128, false>(a, s);
}

template <class TT, int D, bool CAUSAL>
static hipError_t launch_fb_dkdv_t(const Pass2Args& a, hipStream_t s) {
  const size_t lds = pass2_lds_bytes<TT, D>();
  hipError_t e = ensure_lds(&bob_pass2_kernel<TT, D, CAUSAL, true>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bob_pass2_kernel<TT, D, CAUSAL, true>), dim3(row_tiles(a.N), a.BH, a.nsplit), dim3(kBlock), lds,
                     s, a);
  return hipGetLastError();
}

template <class TT>
static hipError_t launch_fb_dkdv_tt(const Pass2Args& a, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch_fb_dkdv_t<TT, 64, true>(a, s) : launch_fb_dkdv_t<TT, 64, false>(a, s);
  return causal ? launch_fb_dkdv_t<TT, 128, true>(a, s) : launch_fb_dkdv_t<TT, 128, false>(a, s);
}

hipError_t launch_first_bwd_dkdv(const Pass2Args& a, DT dt, int d, bool causal, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_fb_dkdv_tt<BF16>(a, d, causal, s);
    case DT::F16: return launch_fb_dkdv_tt<F16>(a, d, causal, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pass2(const Pass2Args& a, DT dt, int d, bool causal, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return launch_p2_tt<BF16>(a, d, causal, s);
    case DT::F16: return launch_p2_tt<F16>(a, d, causal, s);
    default: return launch_p2_tt<F32>(a, d, causal, s);
  }
}

template <class TT, int D>
static hipError_t launch_r2_t(const Pass2Args& a, hipStream_t s) {
  dim3 grid(row_tiles(a.N) * 4, a.BH, Geo<TT, D>::MB);  // one workgroup per wave record
  hipLaunchKernelGGL((bob_pass2_reduce_kernel<TT, D>), grid, dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pass2_reduce(const Pass2Args& a, DT dt, int d, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return d == 64 ? launch_r2_t<BF16, 64>(a, s) : launch_r2_t<BF16, 128>(a, s);
    case DT::F16: return d == 64 ? launch_r2_t<F16, 64>(a, s) : launch_r2_t<F16, 128>(a, s);
    default: return d == 64 ? launch_r2_t<F32, 64>(a, s) : launch_r2_t<F32, 128>(a, s);
  }
}

}  // namespace fb
