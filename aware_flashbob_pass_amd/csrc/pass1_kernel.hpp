// The staged pass-1 kernel template (16-bit inputs) and its four-pass modes.
// Included by bob_pass1.hip (the four-pass modes and the first backward's dQ sweep) and
// by bob_pass1_vgpr.hip (the two-pass instances, built with the matrix-core VGPR form:
// see that file).
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "pass1_asm.hpp"
#include "pass1_common.hpp"

namespace fb {

// 24 wait states after the last accumulating product before anything reads the four
// accumulator tiles (see acc_settle in common.hpp).
template <int MB>
__device__ inline void pass1_acc_settle(f32x16 (&A)[MB], f32x16 (&B)[MB], f32x16 (&C)[MB], f32x16 (&X)[MB]) {
  acc_settle<MB>(A, B);
  acc_settle<MB>(C, X);
}

// ---- four-pass ablation schedule (modes of the pipelined kernel) -----------------
enum : int { kTwoPass = 0, kAlphaPass = 1, kEnergyPass = 2, kRowsPass = 3, kDqPass = 4 };
// kDqPass is not part of BoB: it is the query-side half of the first backward g
// (dQ = tau dS K with dS = P (dP - D)), run by the same staged sweep so that the
// autograd path's first backward uses the same kernels as the rest.

// Record of one wave: the row partial (alpha or E sweeps) or the two row-output
// accumulators (rows sweep), lane-contiguous.
template <class TT, int D, int MODE>
__device__ inline float* fourpass_record(const Pass1Args& a, int split, int bh, int qt, int wave) {
  constexpr size_t REC = MODE == kRowsPass ? (size_t)2 * (D / 32) * 16 * 64
                         : MODE == kDqPass  ? (size_t)(D / 32) * 16 * 64
                                            : 64;
  const size_t rec = (((size_t)split * a.BH + bh) * row_tiles(a.N) + qt) * 4 + wave;
  return a.part + rec * REC;
}

template <class TT, int D, int MODE>
__device__ inline void fourpass_epilogue(const f32x16 (&Q)[D / 32], const f32x16 (&X)[D / 32], float s_p, int qi,
                                         int g, int bh, const Pass1Args& a) {
  using T = typename TT::elem;
  const float total = pair_sum32(s_p);
  if (qi >= a.N) return;
  const size_t row = (size_t)bh * a.N + qi;
  if constexpr (MODE == kAlphaPass) {
    if (g == 0) a.alpha[row] = total;
  } else if constexpr (MODE == kEnergyPass) {
    if (g == 0) {  // alpha is known from the alpha sweep
      a.E[row] = total;
      a.l2[row] = a.L[row] * kLog2e;
      a.c[row] = fmaf(a.alpha[row], a.D[row], total);
    }
  } else if constexpr (MODE == kDqPass) {
    T* dQ = reinterpret_cast<T*>(a.gQ) + row * D;
    const float tau = a.tau;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = mb * 32 + kappa(r4 * 4, g);
        const int r = r4 * 4;
        store4<TT>(dQ + dim, tau * Q[mb][r], tau * Q[mb][r + 1], tau * Q[mb][r + 2], tau * Q[mb][r + 3]);
      }
  } else {
    T* gQ = reinterpret_cast<T*>(a.gQ) + row * D;
    T* gdO = reinterpret_cast<T*>(a.gdO) + row * D;
    const float tau = a.tau;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = mb * 32 + kappa(r4 * 4, g);
        const int r = r4 * 4;
        store4<TT>(gQ + dim, tau * Q[mb][r], tau * Q[mb][r + 1], tau * Q[mb][r + 2], tau * Q[mb][r + 3]);
        store4<TT>(gdO + dim, X[mb][r], X[mb][r + 1], X[mb][r + 2], X[mb][r + 3]);
      }
  }
}

template <class TT, int D, int MODE>
__device__ inline void fourpass_write_record(const f32x16 (&Q)[D / 32], const f32x16 (&X)[D / 32], float s_p,
                                             int split, int bh, int qt, int wave, int lane, const Pass1Args& a) {
  float* R = fourpass_record<TT, D, MODE>(a, split, bh, qt, wave);
  if constexpr (MODE == kDqPass) {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) store_tile16(R + mb * 1024, lane, Q[mb]);
  } else if constexpr (MODE == kRowsPass) {
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb) {
      store_tile16(R + (0 * (D / 32) + mb) * 1024, lane, Q[mb]);
      store_tile16(R + (1 * (D / 32) + mb) * 1024, lane, X[mb]);
    }
  } else {
    R[lane] = s_p;
  }
}

// Interleaving request for one pipelined pass-1 step (one basic block): each
// matrix-core op is followed by a share of the element-wise vector work and by
// the LDS reads of the NEXT k-step (operands are fetched one k-step ahead).
// Masks: 0x008 matrix core, 0x002 vector ALU, 0x100 LDS read.
template <int DK, int MB>
__device__ inline void pass1_schedule() {
#pragma unroll
  for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // k-step 0 operands
#pragma unroll
  for (int i = 0; i < 5 * DK; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < 6 * MB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
#pragma unroll
  for (int i = 0; i < 6 * MB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// Pipelined variant for 16-bit inputs. LDS holds three stages of row-major
// K, V, UK, UV tiles (32 keys each); the registers of every thread prefetch the
// stage two steps ahead, so each step has a single barrier and no exposed
// global-load latency. Within a step, the score tiles of the NEXT step are
// formed on the matrix cores while the element-wise work of the current step
// runs on the vector ALUs, and the accumulating contractions read their
// transposed operands with the transposing LDS load (lds_tr_op).
//
// MODE selects the schedule: kTwoPass is the method's pass 1 above. The other
// modes are the natural four-pass schedule that the affine structure collapses
// (review page, Summary and Strengths on Prop. 4.1), kept for measuring what
// the collapse saves: kAlphaPass sweeps the keys for alpha only (S and G),
// kEnergyPass sweeps again for E with alpha known, and kRowsPass forms
// gQ = tau (dS UK + Sbar K) and gdO = P UV + dPbar V with alpha and E known.
// Waves per SIMD each pass-1 kernel is built for: the two-pass kernel (d = 64; d = 128
// runs bob_pass1_q16_kernel) keeps four float32 accumulator tiles in AGPRs beside its
// score tiles in VGPRs (one wave); the other modes hold at most two accumulator tiles,
// or at d = 128 at most the alpha sweep's score tiles, and take the register form at two.
__host__ __device__ constexpr int p1_waves_per_simd(int mode, int d) {
  return (mode == kTwoPass || (d == 128 && mode != kAlphaPass)) ? 1 : 2;
}

// FOLD (two-pass sweep, bf16, tau a positive power of two): the resident Q and UQ
// rows are scaled by tau once, which is exact, so the score products give tau S and
// G = tau (UQ K^T + Q UK^T) directly (the same float32 values as scaling afterwards)
// and each step saves the 16 multiplications of G by tau.
// ASML (that sweep): steps that need no mask (whole key blocks that no query of the
// workgroup precedes) run as one inline-assembly block with a fixed schedule
// (pass1_asm_steps). kAsmAll: every step of the sweep needs none (non-causal, N a
// multiple of 32), so the kernel has no compiled steps; kAsmPrefix: the compiled steps
// take the rest (a causal sweep's diagonal blocks, a ragged last block).
enum : int { kAsmNone = 0, kAsmAll = 1, kAsmPrefix = 2 };
template <class TT, int D, bool CAUSAL, int MODE, bool FOLD = false, int ASML = kAsmNone>
__global__ __launch_bounds__(kBlock, p1_waves_per_simd(MODE, D)) void bob_pass1_kernel(Pass1Args a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB, DK = G::DK, NK = G::NK;
  // d = 64: four LDS stages, copies issued three steps ahead from inline assembly
  // and awaited one step before use; d = 128 (no register room for the deeper
  // unroll) keeps three stages, two steps ahead, compiler-visible copies.
  constexpr bool DEEP = D == 64;
  constexpr int NT = 4, NBUF = ASML != kAsmNone ? FB_PASS1_ASM_SLOTS : DEEP ? 4 : 3;
  constexpr int AHEAD = ASML != kAsmNone ? FB_PASS1_ASM_AHEAD : NBUF - 1;
  // The two-pass sweeps keep their four accumulator tiles in AGPRs from inline
  // assembly and are compiled with the VGPR form for everything else
  // (bob_pass1_vgpr.hip), so the element-wise work reads the score tiles where the
  // matrix cores wrote them. The d = 64 sweeps also form the next step's score tiles
  // during the current step (software pipelining; 247 VGPRs causal, 255 non-causal).
  constexpr bool PIPE = D == 64 && MODE == kTwoPass;
  constexpr bool ASM_ACC = MODE == kTwoPass;
  constexpr bool TWO = MODE == kTwoPass;
  constexpr bool NEED_DP = MODE != kAlphaPass;  // the alpha sweep needs S and G only
  constexpr bool NEED_G = MODE != kDqPass;      // the first backward needs S and dP only
  constexpr bool NEED_H = NEED_DP && NEED_G;
  // direct copies one wave issues per step (K always, V for dP, UK for G, UV for H)
  constexpr int COPIES = (1 + NEED_DP + NEED_G + NEED_H) * stage_copies<D, kBlock / 64>();
  constexpr int MBA = TWO ? P1<TT, D>::MBA : MB;
  static_assert(TT::KPL == 8 && NK == 2, "16-bit inputs only");
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  int qt, bh;
  tile_and_head<CAUSAL, true>(qt, bh);
  const int N = a.N, split = blockIdx.z;
  // pass 2's merge counter of key tile qt starts at zero (kReduceLastBlock)
  if (a.p2_counters && blockIdx.z == 0 && threadIdx.x == 0) a.p2_counters[(size_t)bh * row_tiles(N) + qt] = 0u;
  const size_t base = (size_t)bh * N * D;
  const T* src[NT] = {reinterpret_cast<const T*>(a.K) + base, reinterpret_cast<const T*>(a.V) + base,
                      reinterpret_cast<const T*>(a.UK) + base, reinterpret_cast<const T*>(a.UV) + base};
  const int q0 = qt * kBlockRows + wave * kTile;
  const int qi = q0 + n;

  int nkt = (N + kTile - 1) / kTile;
  if (CAUSAL) nkt = min(nkt, (qt + 1) * (kBlockRows / kTile));
  const int kt_begin = (int)((long long)split * nkt / a.nsplit);
  const int kt_end = (int)((long long)(split + 1) * nkt / a.nsplit);
  const int nsteps = kt_end - kt_begin;

  auto stage = [&](int j, int t) { return lds + ((j % NBUF) * NT + t) * G::ROW_ELEMS; };
  auto active = [&](int j) { return !CAUSAL || (kt_begin + j) * kTile <= q0 + kTile - 1; };

  // tiles a mode reads: K always, V for dP, UK for G, UV for H
  constexpr bool NEED_TILE[NT] = {true, NEED_DP, NEED_G, NEED_H};
  auto issue = [&](int stg, int j) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (NEED_TILE[t])
        stage_direct<TT, D, kBlock / 64, DEEP>(src[t], (kt_begin + j) * kTile, N,
                                                lds + (stg * NT + t) * G::ROW_ELEMS, wave, lane);
  };
  // Copies first, then the resident rows, so that their latencies overlap: the
  // compiler's own waits for those loads only get stricter with older copies in flight.
  // Without splits the epilogue needs the wave's rows of O (gdO = X - alpha O): they
  // are copied into LDS beside the stages, so the end of the sweep reads no global memory.
  T* o_lds = lds + NBUF * NT * G::ROW_ELEMS + wave * kTile * D;
  if constexpr (TWO && D == 64) {
    if (a.nsplit == 1) {
      const T* osrc = reinterpret_cast<const T*>(a.O) + base;
#pragma unroll
      for (int c = 0; c < kTile * D / (64 * 8); ++c) {  // 64 lanes x 16 bytes a copy
        const int slot = c * 64 + lane, row = slot / (D / 8), ch = slot % (D / 8);
        glds16<DEEP>(osrc + (size_t)min(q0 + row, N - 1) * D + ch * 8, o_lds + c * 64 * 8);
      }
    }
  }
  for (int j = 0; j < AHEAD && j < nsteps; ++j) issue(j, j);

  V bq[DK], bdo[DK], buq[DK];
  load_resident<TT, D>(reinterpret_cast<const T*>(a.Q) + base, qi, N, g, bq);
  load_resident<TT, D>(reinterpret_cast<const T*>(a.dO) + base, qi, N, g, bdo);
  if constexpr (NEED_G) load_resident<TT, D>(reinterpret_cast<const T*>(a.UQ) + base, qi, N, g, buq);
  static_assert(!FOLD || (MODE == kTwoPass && std::is_same_v<TT, BF16>), "tau folding: bf16 two-pass sweep only");
  if constexpr (FOLD) {
#pragma unroll
    for (int t = 0; t < DK; ++t)
#pragma unroll
      for (int s = 0; s < TT::KPL; ++s) {
        bq[t][s] = TT::cvt(TT::tof(bq[t][s]) * a.tau);
        buq[t][s] = TT::cvt(TT::tof(buq[t][s]) * a.tau);
      }
  }
  const size_t rowv = (size_t)bh * N + (qi < N ? qi : 0);
  const float lq = a.L[rowv] * kLog2e;
  const float dq = a.D[rowv];
  const float cs = FOLD ? kLog2e : a.tau * kLog2e;
  const float tau = a.tau;
  const float al = (MODE == kEnergyPass || MODE == kRowsPass) ? a.alpha[rowv] : 0.f;
  const float er = MODE == kRowsPass ? a.E[rowv] : 0.f;

  f32x16 accA[MBA], accB[MBA], accC[MBA], accX[MBA];
#pragma unroll
  for (int mb = 0; mb < MBA; ++mb) {
    accA[mb] = zero16();
    accB[mb] = zero16();
    accC[mb] = zero16();
    accX[mb] = zero16();
  }
  float alpha_p = 0.f, e0_p = 0.f;

  // The stage copies are invisible to the compiler (inline assembly), so make it
  // complete its own loads of the resident rows and row scalars here: otherwise it
  // could wait for them inside the loop with a vmcnt(0) that also drains the copies.
  if constexpr (DEEP) {
    settle_regs(bq, bdo, lq, dq, al, er);
    if constexpr (NEED_G) settle_regs(buq);
  }
  wait_vmem();
  __syncthreads();

  // score tiles of the current step (c) and of the next step (x)
  f32x16 sc = zero16(), gc = zero16(), pc = zero16(), hc = zero16();
  if (PIPE && nsteps > 0 && active(0)) {
#pragma unroll
    for (int t = 0; t < DK; ++t) {
      const V ak = lds_row_op<TT, D>(stage(0, 0), n, t, g);
      const V av = lds_row_op<TT, D>(stage(0, 1), n, t, g);
      const V auk = lds_row_op<TT, D>(stage(0, 2), n, t, g);
      const V auv = lds_row_op<TT, D>(stage(0, 3), n, t, g);
      sc = TT::mfma(ak, bq[t], sc);
      if constexpr (NEED_G) {
        gc = TT::mfma(ak, buq[t], gc);
        gc = TT::mfma(auk, bq[t], gc);
      }
      if constexpr (NEED_DP) pc = TT::mfma(av, bdo[t], pc);
      if constexpr (NEED_H) hc = TT::mfma(auv, bdo[t], hc);
    }
  }

  // One pipeline step; S = j % NBUF is a compile-time constant so that every LDS
  // address is a loop-invariant per-lane offset plus an immediate. Step j reads
  // stage S (and S + 1 for the next step's scores) and copies step j + AHEAD into
  // stage S + AHEAD (last read in step j - 1). With DEEP it then waits, before its
  // barrier, only for the copies of step j - 1 (step j + 2, read from step j + 1
  // on), so each copy has two steps to land; otherwise for all of them.
  auto step = [&](auto S_c, int j) {
    constexpr int S = decltype(S_c)::value;
    constexpr int SN = (S + 1) % NBUF, SC = (S + AHEAD) % NBUF;
    const T* ck = lds + (S * NT + 0) * G::ROW_ELEMS;
    const T* cv = lds + (S * NT + 1) * G::ROW_ELEMS;
    const T* cuk = lds + (S * NT + 2) * G::ROW_ELEMS;
    const T* cuv = lds + (S * NT + 3) * G::ROW_ELEMS;
    const T* nk = lds + (SN * NT + 0) * G::ROW_ELEMS;
    const T* nv = lds + (SN * NT + 1) * G::ROW_ELEMS;
    const T* nuk = lds + (SN * NT + 2) * G::ROW_ELEMS;
    const T* nuv = lds + (SN * NT + 3) * G::ROW_ELEMS;
    const bool copies = j + AHEAD < nsteps;
    if (copies) issue(SC, j + AHEAD);
    const bool act = active(j);
    const bool act_next = (j + 1 < nsteps) && active(j + 1);
    const int k0 = (kt_begin + j) * kTile;
    f32x16 sx = zero16(), gx = zero16(), px = zero16(), hx = zero16();

    if (act) {
      if constexpr (!PIPE) {
        sc = zero16();
        gc = zero16();
        pc = zero16();
        hc = zero16();
#pragma unroll
        for (int t = 0; t < DK; ++t) {
          const V ak = lds_row_op<TT, D>(ck, n, t, g);
          const V av = lds_row_op<TT, D>(cv, n, t, g);
          const V auk = lds_row_op<TT, D>(cuk, n, t, g);
          const V auv = lds_row_op<TT, D>(cuv, n, t, g);
          sc = TT::mfma(ak, bq[t], sc);
          if constexpr (NEED_G) {
            gc = TT::mfma(ak, buq[t], gc);
            gc = TT::mfma(auk, bq[t], gc);
          }
          if constexpr (NEED_DP) pc = TT::mfma(av, bdo[t], pc);
          if constexpr (NEED_H) hc = TT::mfma(auv, bdo[t], hc);
        }
      }
      // log2-domain scores, masked where the key is out of range or after the query
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = sc[r] * cs - lq;
      if (k0 + kTile > N || (CAUSAL && k0 + kTile - 1 > q0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kappa(r, g);
          if (!(key < N && (!CAUSAL || key <= qi))) sc[r] = -INFINITY;
        }
      }
      V wa[NK], wb[NK], pp[NK], pg[NK];
      auto elementwise = [&](int r) {
        const float p = fast_exp2(sc[r]);
        const float gv = FOLD ? gc[r] : gc[r] * tau;
        const int kk = r >> 3, ss = r & 7;
        if constexpr (MODE == kAlphaPass) {
          alpha_p += p * gv;
        } else if constexpr (MODE == kEnergyPass) {
          const float dpv = pc[r];
          e0_p += p * (fmaf(gv, dpv - dq, hc[r]) - al * dpv);  // P Pbar: E directly
        } else if constexpr (MODE == kDqPass) {
          vset<TT>(wa[kk], ss, p * (pc[r] - dq));  // dS
        } else if constexpr (MODE == kRowsPass) {
          const float dpv = pc[r];
          const float t1 = dpv - dq;
          const float pbar = fmaf(gv, t1, hc[r]) - al * dpv;
          vset<TT>(wa[kk], ss, p * t1);             // dS
          vset<TT>(wb[kk], ss, p * (pbar - er));    // Sbar
          vset<TT>(pp[kk], ss, p);                  // P
          vset<TT>(pg[kk], ss, p * (gv - al));      // dPbar
        } else {
          const float dpv = pc[r];
          const float t1 = dpv - dq;
          const float vpg = p * gv;
          const float vwb = p * fmaf(gv, t1, hc[r]);
          alpha_p += vpg;
          e0_p += vwb;
          // The sums are ordered, so the compiler may not reassociate them; left free it
          // schedules each chain late and keeps all 32 of the step's terms live (about 50
          // values spilled per step in the non-causal sweep). Pinning each addition here
          // keeps a term's live range short. The causal sweep measured 2% slower pinned.
          if constexpr (!CAUSAL) asm volatile("" : "+v"(alpha_p), "+v"(e0_p));
          vset<TT>(wa[kk], ss, p * t1);
          vset<TT>(wb[kk], ss, vwb);
          vset<TT>(pp[kk], ss, p);
          vset<TT>(pg[kk], ss, vpg);
        }
      };
      // phase 1: next step's score tiles (matrix cores) with rows 0..7 (vector ALUs);
      // the last step also forms "next" tiles from a stale stage, never used.
      // LDS operands are fetched one k-step ahead of the matrix-core ops using them.
      V ro[2][4];
      auto fetch_row = [&](int t, V (&o)[4]) {
        o[0] = lds_row_op<TT, D>(nk, n, t, g);
        o[1] = lds_row_op<TT, D>(nv, n, t, g);
        o[2] = lds_row_op<TT, D>(nuk, n, t, g);
        o[3] = lds_row_op<TT, D>(nuv, n, t, g);
      };
      if constexpr (PIPE) {
        fetch_row(0, ro[0]);
#pragma unroll
        for (int t = 0; t < DK; ++t) {
          if (t + 1 < DK) fetch_row(t + 1, ro[(t + 1) & 1]);
          const V(&o)[4] = ro[t & 1];
          sx = TT::mfma(o[0], bq[t], sx);
          if constexpr (NEED_G) gx = TT::mfma(o[0], buq[t], gx);
          if constexpr (NEED_DP) px = TT::mfma(o[1], bdo[t], px);
          if constexpr (NEED_G) gx = TT::mfma(o[2], bq[t], gx);
          if constexpr (NEED_H) hx = TT::mfma(o[3], bdo[t], hx);
#pragma unroll
          for (int r = t * 8 / DK; r < (t + 1) * 8 / DK; ++r) elementwise(r);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) elementwise(r);
      }
      // phases 2-3: alpha-free accumulators; rows 8..15 ride along the first half
      V to[2][4];
      auto fetch_tr = [&](int q, V (&o)[4]) {
        const int t = q / MBA, mb = q % MBA;
        o[0] = lds_tr_op<TT, D>(ck, mb, t, lane);
        o[1] = lds_tr_op<TT, D>(cuk, mb, t, lane);
        o[2] = lds_tr_op<TT, D>(cv, mb, t, lane);
        o[3] = lds_tr_op<TT, D>(cuv, mb, t, lane);
      };
      if constexpr (MODE == kAlphaPass || MODE == kEnergyPass) {
        // scalar sweeps: no accumulating contractions
#pragma unroll
        for (int r = 8; r < 16; ++r) elementwise(r);
      } else {
      if constexpr (PIPE) fetch_tr(0, to[0]);
#pragma unroll
      for (int q = 0; q < NK * MBA; ++q) {
        const int t = q / MBA, mb = q % MBA;
        // d = 128 fetches each k-step's operands just before use (register budget)
        if constexpr (PIPE) {
          if (q + 1 < NK * MBA) fetch_tr(q + 1, to[(q + 1) & 1]);
        } else {
          fetch_tr(q, to[q & 1]);
        }
        if (t == 0) {
#pragma unroll
          for (int r = 8 + mb * 8 / MBA; r < 8 + (mb + 1) * 8 / MBA; ++r) elementwise(r);
        }
        const V(&o)[4] = to[q & 1];
        if constexpr (MODE == kDqPass) {
          accA[mb] = TT::mfma(o[0], wa[t], accA[mb]);  // dS K
        } else if constexpr (MODE == kRowsPass) {
          accA[mb] = TT::mfma(o[1], wa[t], accA[mb]);  // dS UK
          accX[mb] = TT::mfma(o[3], pp[t], accX[mb]);  // P UV
          accA[mb] = TT::mfma(o[0], wb[t], accA[mb]);  // Sbar K
          accX[mb] = TT::mfma(o[2], pg[t], accX[mb]);  // dPbar V
        } else {
          if constexpr (ASM_ACC) {  // AGPR accumulators from inline assembly
            mfma_acc<TT>(accA[mb], o[1], wa[t]);
            mfma_acc<TT>(accB[mb], o[0], wa[t]);  // W_a K
            mfma_acc<TT>(accX[mb], o[3], pp[t]);
            mfma_acc<TT>(accA[mb], o[0], wb[t]);
            mfma_acc<TT>(accC[mb], o[0], pp[t]);
            mfma_acc<TT>(accX[mb], o[2], pg[t]);
          } else {
            accA[mb] = TT::mfma(o[1], wa[t], accA[mb]);
            accB[mb] = TT::mfma(o[0], wa[t], accB[mb]);  // W_a K
            accX[mb] = TT::mfma(o[3], pp[t], accX[mb]);
            accA[mb] = TT::mfma(o[0], wb[t], accA[mb]);
            accC[mb] = TT::mfma(o[0], pp[t], accC[mb]);
            accX[mb] = TT::mfma(o[2], pg[t], accX[mb]);
          }
        }
      }
      }
      // the interleave request pays off in the causal sweep only (non-causal: 1% slower with it)
      if constexpr (PIPE && TWO && CAUSAL) pass1_schedule<DK, MBA>();
    } else if (PIPE && act_next) {
#pragma unroll
      for (int t = 0; t < DK; ++t) {
        const V ak = lds_row_op<TT, D>(nk, n, t, g);
        const V av = lds_row_op<TT, D>(nv, n, t, g);
        const V auk = lds_row_op<TT, D>(nuk, n, t, g);
        const V auv = lds_row_op<TT, D>(nuv, n, t, g);
        sx = TT::mfma(ak, bq[t], sx);
        if constexpr (NEED_G) {
          gx = TT::mfma(ak, buq[t], gx);
          gx = TT::mfma(auk, bq[t], gx);
        }
        if constexpr (NEED_DP) px = TT::mfma(av, bdo[t], px);
        if constexpr (NEED_H) hx = TT::mfma(auv, bdo[t], hx);
      }
    }
    if constexpr (PIPE) {
      sc = sx;
      gc = gx;
      pc = px;
      hc = hx;
    }
    if (DEEP && copies) wait_vmem_keep<COPIES>();  // this step's copies may stay in flight
    else wait_vmem();
    __syncthreads();
    // The scalar sweeps' element-wise work has no memory effects; pin its sum to the
    // step so the compiler cannot sink several steps' work (and keep their score
    // tiles live) past the barriers.
    if constexpr (MODE == kAlphaPass) asm volatile("" : "+v"(alpha_p)::"memory");
    if constexpr (MODE == kEnergyPass) asm volatile("" : "+v"(e0_p)::"memory");
  };
  int j = 0;
  if constexpr (ASML != kAsmNone) {
    static_assert(FOLD && D == 64 && (ASML == kAsmPrefix || !CAUSAL), "scheduled loop: folded d = 64 two-pass sweep");
    // steps with no mask and no copy of a ragged block (kAsmAll: the caller guarantees
    // every step qualifies)
    const int nasm = ASML == kAsmAll ? nsteps
                                     : pass1_asm_step_count(N, CAUSAL, qt, kt_begin, nsteps, NBUF, AHEAD);
    if (nasm > 0) {
      const size_t ahead = (size_t)(kt_begin + AHEAD) * kTile * D;  // copy sources of step 0
      pass1_asm_steps(sc, gc, pc, hc, bq, buq, bdo, accA, accB, accC, accX, alpha_p, e0_p, lq, dq, src[0] + ahead,
                      src[1] + ahead, src[2] + ahead, src[3] + ahead, lds, wave, lane, nasm, nsteps);
      // the compiled steps take the plain dP tile (the block leaves dP - D in it)
      if (FB_PASS1_ASM_DBIAS && nasm < nsteps) {
#pragma unroll
        for (int r = 0; r < 16; ++r) pc[r] += dq;
      }
      j = nasm;
    }
  }
  if constexpr (ASML != kAsmAll) {
    for (; j + NBUF <= nsteps; j += NBUF) unroll_steps(step, j, std::make_integer_sequence<int, NBUF>{});
    unroll_steps_until(step, j, nsteps, std::make_integer_sequence<int, NBUF - 1>{});
  }

  if constexpr (TWO) {
    if constexpr (ASM_ACC) pass1_acc_settle<MBA>(accA, accB, accC, accX);
    if (a.nsplit == 1) {
      if constexpr (D == 64) pass1_epilogue<TT, D>(accA, accB, accC, accX, alpha_p, e0_p, qi, g, bh, a, o_lds + n * D,
                                                    lq, dq);
      else pass1_epilogue<TT, D>(accA, accB, accC, accX, alpha_p, e0_p, qi, g, bh, a);
      return;
    }
    pass1_write_record<TT, D>(accA, accB, accC, accX, alpha_p, e0_p, split, bh, qt, wave, lane, a);
  } else {
    const float sp = MODE == kAlphaPass ? alpha_p : e0_p;
    if (a.nsplit == 1) {
      fourpass_epilogue<TT, D, MODE>(accA, accX, sp, qi, g, bh, a);
      return;
    }
    fourpass_write_record<TT, D, MODE>(accA, accX, sp, split, bh, qt, wave, lane, a);
  }
}

// LDS of the scheduled loop: FB_PASS1_ASM_SLOTS stages of K, V, UK, UV.
inline size_t pass1_asm_lds_bytes() { return (size_t)FB_PASS1_ASM_SLOTS * 4 * 32 * 64 * 2; }
// LDS after the stages of the two-pass d = 64 kernel: each wave's rows of O (16-bit).
inline size_t pass1_o_lds_bytes() { return (size_t)4 * 32 * 64 * 2; }

template <class TT, int D>
inline size_t pass1_lds_bytes() {
  using G = Geo<TT, D>;
  if constexpr (TT::KPL == 1) return (size_t)4 * (G::ROW_ELEMS + G::T_ELEMS) * sizeof(typename TT::elem);
  return (size_t)(D == 64 ? 4 : 3) * 4 * G::ROW_ELEMS * sizeof(typename TT::elem);  // stages of K, V, UK, UV
}

}  // namespace fb
