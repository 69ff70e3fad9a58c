// Statistics kernel: one online-softmax forward sweep per query tile.
//
// BoB recomputes every score tile from the forward's row statistics (the
// score-recomputation model of the FlashBoB review page, Strengths: Theorem 4.5),
// so the call starts with a FlashAttention-style forward that produces
//   O = softmax(tau Q K^T) V,  L_i = log sum_j exp(tau q_i . k_j),
// and, fused into its epilogue, D_i = sum_t dO_it O_it formed from the float32
// O before rounding (D = rowsum(P * dP) = rowsum(dO * O) in exact arithmetic).
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

// 1: non-causal 16-bit d = 64 sweeps take the skewed kernel; 0 builds them with
// attn_fwd_kernel instead (for comparing the two on the same inputs).
#ifndef FB_FWD_SKEW
#define FB_FWD_SKEW 1
#endif

namespace fb {

// Stage ring of the skewed statistics sweep: slots and copy distance in steps.
constexpr int kFwdSkewSlots = 6;
constexpr int kFwdSkewAhead = 5;

// O, L and (optionally) D of one wave from its unnormalised O^T accumulators,
// running max m (log2 units, equal in lanes n and n + 32) and per-lane partial
// denominators l.
template <class TT, int D, bool WITH_D>
__device__ inline void fwd_epilogue(const f32x16 (&acc)[Geo<TT, D>::MB], float m, float l, int qi, int g, int bh,
                                    const FwdArgs& a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  const int N = a.N;
  const size_t base = (size_t)bh * N * D;
  const float lt = pair_sum32(l);
  const float inv = 1.f / lt;
  if (qi >= N) return;
  T* O = reinterpret_cast<T*>(a.O) + base + (size_t)qi * D;
  const T* dO = WITH_D ? reinterpret_cast<const T*>(a.dO) + base + (size_t)qi * D : nullptr;
  float dot = 0.f;
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dim = mb * 32 + kappa(r4 * 4, g);
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[mb][r4 * 4 + e] * inv;
      store4<TT>(O + dim, o[0], o[1], o[2], o[3]);
      if constexpr (WITH_D) {
        float x[4];
        load4<TT>(dO + dim, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) dot += x[e] * o[e];
      }
    }
  // lanes n and n + 32 own the same query, so the exchange stays paired
  if (g == 0) a.L[(size_t)bh * N + qi] = m * kLn2 + __logf(lt);
  if constexpr (WITH_D) {
    dot = pair_sum32(dot);
    if (g == 0) a.D[(size_t)bh * N + qi] = dot;
  }
}

// Staged variant for 16-bit inputs (same staging scheme as pass 1): K and V
// tiles in three row-major LDS stages loaded two steps ahead; each step forms
// its score tile, runs the online softmax and accumulates P V, reading V^T
// operands with the transposing LDS load. Declared for two waves per SIMD (the
// register form; d = 128 then needs 188 VGPRs and no AGPRs), which hides more
// than forming the next step's tile early did.
// The reference maximum m of a row is not tracked per step: each step forms its
// weights 2^(s - m) with the current m and only when some lane's sum of them
// reaches lazy_limit (or is not finite, as on a row's first step, where m is
// -1e30) does it take the step's row maximum, rescale the sums and form the
// weights again. The result is unchanged because the denominator l and the
// accumulators share m, and the maximum's tree, pair exchange and compare run
// only on those steps. Every weight of a step that is not redone is at most its
// lane's sum, so the limit bounds the weight operands: bf16 has the float32
// exponent range and takes 2^32; fp16 operands must stay below 65504, its
// largest finite value, and take 2^15. After a redo every weight is at most 1.
// The end of a statistics sweep: O, L (and D) of the wave's rows when the keys are not
// split, else the wave's split record (accumulators, m, l) for the merge.
template <class TT, int D, bool WITH_D>
__device__ inline void fwd_finish(const f32x16 (&acc)[Geo<TT, D>::MB], float m, float l, int qt, int bh, int split,
                                  int wave, int lane, const FwdArgs& a) {
  constexpr int MB = Geo<TT, D>::MB;
  const int N = a.N;
  if (a.nsplit == 1) {
    fwd_epilogue<TT, D, WITH_D>(acc, m, l, qt * kBlockRows + wave * kTile + (lane & 31), lane >> 5, bh, a);
    return;
  }
  const size_t rec = (((size_t)split * a.BH + bh) * row_tiles(N) + qt) * 4 + wave;
  float* R = a.part + rec * fwd_record_floats(D);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) store_tile16(R + mb * 1024, lane, acc[mb]);  // [MB] quad-major tiles
  R[MB * 16 * 64 + lane] = m;
  R[MB * 16 * 64 + 64 + lane] = l;
}

template <class TT>
__device__ constexpr float lazy_limit() {
  return std::is_same_v<TT, F16> ? 32768.f : 4294967296.f;  // 2^15 : 2^32
}

// True when the step sum x reached `limit` or is not finite. The sum of
// exponentials is never negative, so its bit pattern orders like its value,
// and +inf and every NaN pattern (either sign) compare above any finite limit.
// An integer compare keeps this exact under -fno-honor-nans, which lets the
// compiler assume a float compare never sees a NaN.
__device__ inline bool lazy_redo(float x, float limit) { return __float_as_uint(x) >= __float_as_uint(limit); }

template <class TT, int D, bool CAUSAL, bool WITH_D>
__global__ __launch_bounds__(kBlock, 2) void attn_fwd_kernel(FwdArgs a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB, DK = G::DK, NK = G::NK;
  constexpr int NT = 2, NBUF = 3;
  static_assert(TT::KPL == 8 && NK == 2, "16-bit inputs only");
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  int qt, bh;
  tile_and_head<CAUSAL, true>(qt, bh);
  const int N = a.N, split = blockIdx.z;
  const size_t base = (size_t)bh * N * D;
  const T* src[NT] = {reinterpret_cast<const T*>(a.K) + base, reinterpret_cast<const T*>(a.V) + base};
  const int q0 = qt * kBlockRows + wave * kTile;
  const int qi = q0 + n;

  V bq[DK];
  load_resident<TT, D>(reinterpret_cast<const T*>(a.Q) + base, qi, N, g, bq);
  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
  float m = -1e30f, l = 0.f;
  const float cs = a.tau * kLog2e;
  const bool fold = cs > 0.f;           // wave-uniform
  const float cm = fold ? cs : 1.f;     // multiplier of the score in the exponent

  int nkt = (N + kTile - 1) / kTile;
  if (CAUSAL) nkt = min(nkt, (qt + 1) * (kBlockRows / kTile));
  const int kt_begin = (int)((long long)split * nkt / a.nsplit);
  const int kt_end = (int)((long long)(split + 1) * nkt / a.nsplit);
  const int nsteps = kt_end - kt_begin;
  auto stage = [&](int j, int t) { return lds + ((j % NBUF) * NT + t) * G::ROW_ELEMS; };
  auto active = [&](int j) { return !CAUSAL || (kt_begin + j) * kTile <= q0 + kTile - 1; };

  // Copies from inline assembly: whole 32-key blocks in the scalar-base form, the ragged
  // last block through stage_direct (which repeats row N - 1); each step ends with every
  // copy landed.
  constexpr int CP = stage_copies<D, kBlock / 64>();
  unsigned coff[CP];
#pragma unroll
  for (int p = 0; p < CP; ++p) coff[p] = stage_lane_offset<D, kBlock / 64>(p, wave, lane);
  const unsigned lds_wave = lds_addr(lds) + (unsigned)wave * 1024u;
  auto issue = [&](int stg, int j) {
    const int r0 = (kt_begin + j) * kTile;
    if (r0 + kTile <= N) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        stage_block_saddr<D, kBlock / 64>(src[t] + (size_t)r0 * D, coff,
                                          lds_wave + (unsigned)((stg * NT + t) * G::ROW_ELEMS * (int)sizeof(T)));
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        stage_direct<TT, D, kBlock / 64, true>(src[t], r0, N, lds + (stg * NT + t) * G::ROW_ELEMS, wave, lane);
    }
  };
  settle_regs(bq);
  for (int j = 0; j < 2 && j < nsteps; ++j) issue(j, j);
  wait_vmem();
  __syncthreads();

  f32x16 sc;  // score tile of the current step
  auto step = [&](auto S_c, int j) {
    constexpr int S = decltype(S_c)::value;
    constexpr int SC = (S + 2) % NBUF;
    if (j + 2 < nsteps) issue(SC, j + 2);  // buffer SC was last read in step j - 1
    const int k0 = (kt_begin + j) * kTile;
    if (active(j)) {
      sc = zero16();
#pragma unroll
      for (int t = 0; t < DK; ++t) sc = TT::mfma(lds_row_op<TT, D>(stage(S, 0), n, t, g), bq[t], sc);
      // With cs > 0 the scale stays folded into the exponent (p = 2^(raw cs - m)): the
      // maximum of the raw scores times cs equals the maximum of the scaled scores
      // (rounding is monotonic) and masked raw scores of -inf still give p = 0. With
      // cs <= 0 the scores are scaled first and the exponent multiplies by 1.
      if (!fold) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] *= cs;
      }
      if (k0 + kTile > N || (CAUSAL && k0 + kTile - 1 > q0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kappa(r, g);
          if (!(key < N && (!CAUSAL || key <= qi))) sc[r] = -INFINITY;
        }
      }
      V pp[NK];
      float ls = 0.f;  // this step's part of the denominator
      auto weights = [&]() {
        ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(sc[r], cm, -m));
          ls += p;
          vset<TT>(pp[r >> 3], r & 7, p);
        }
      };
      weights();
      if (__ballot(lazy_redo(ls, lazy_limit<TT>()))) {  // rare: move m to the row maximum
        float mx = max16(sc);
        if (fold) mx *= cs;
        mx = pair_max32(mx);
        const float mnew = fmaxf(m, mx);
        const float f = fast_exp2(m - mnew);
        l *= f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] *= f;
        m = mnew;
        weights();
      }
      l += ls;
#pragma unroll
      for (int t = 0; t < NK; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = TT::mfma(lds_tr_op<TT, D>(stage(S, 1), mb, t, lane), pp[t], acc[mb]);
    }
    wait_vmem();
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  int j = 0;
  for (; j + NBUF <= nsteps; j += NBUF) {
    step(I0{}, j);
    step(I1{}, j + 1);
    step(I2{}, j + 2);
  }
  if (j < nsteps) step(I0{}, j);
  if (j + 1 < nsteps) step(I1{}, j + 1);

  fwd_finish<TT, D, WITH_D>(acc, m, l, qt, bh, split, wave, lane, a);
}

// Two-step skew of the same sweep. Step j issues the score products of step j + 2
// and the P V products of step j, and forms the weights of step j + 1 from the score
// tile step j - 1 issued: no part of a step waits for another part of it, so the
// compiler can place the exponentials among the products. Score tiles and weights
// are double-buffered. The stage ring has NBUF slots and the copies, issued from
// inline assembly, run AHEAD stages ahead; step j reads K of stage j + 2 and V of
// stage j, and its end waits only for stage j + 3.
// The weights take one form, p = 2^(fma(s, tau log2 e, -m)), on every step; a step
// whose keys need a mask (the ragged last block, the causal diagonal) or whose
// weights reach the lazy limit forms them again on a slow path, which applies the
// mask and, for the limit, moves m to the row maximum as attn_fwd_kernel does. A
// redo of step j + 1's weights rescales the accumulators after step j's products,
// which were formed with the same reference as the sums.
template <class TT, int D, bool CAUSAL, bool WITH_D>
__global__ __launch_bounds__(kBlock, 2) void attn_fwd_skew_kernel(FwdArgs a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  constexpr int MB = G::MB, DK = G::DK, NK = G::NK;
  constexpr int NT = 2, NBUF = kFwdSkewSlots, AHEAD = kFwdSkewAhead;
  constexpr int COPIES = NT * stage_copies<D, kBlock / 64>();  // per wave and stage
  static_assert(TT::KPL == 8 && NK == 2, "16-bit inputs only");
  static_assert(NBUF % 2 == 0 && AHEAD >= 3 && AHEAD < NBUF, "stage ring");
  extern __shared__ __align__(16) unsigned char smem[];
  T* lds = reinterpret_cast<T*>(smem);

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  int qt, bh;
  tile_and_head<CAUSAL, true>(qt, bh);
  const int N = a.N, split = blockIdx.z;
  const size_t base = (size_t)bh * N * D;
  const T* src[NT] = {reinterpret_cast<const T*>(a.K) + base, reinterpret_cast<const T*>(a.V) + base};
  const int q0 = qt * kBlockRows + wave * kTile;
  const int qi = q0 + n;

  int nkt = (N + kTile - 1) / kTile;
  if (CAUSAL) nkt = min(nkt, (qt + 1) * (kBlockRows / kTile));
  const int kt_begin = (int)((long long)split * nkt / a.nsplit);
  const int kt_end = (int)((long long)(split + 1) * nkt / a.nsplit);
  const int nsteps = kt_end - kt_begin;
  auto stage = [&](int slot, int t) __attribute__((always_inline)) { return lds + (slot * NT + t) * G::ROW_ELEMS; };
  auto active = [&](int j) __attribute__((always_inline)) { return !CAUSAL || (kt_begin + j) * kTile <= q0 + kTile - 1; };
  // Copies of whole 32-key blocks take the scalar-base form: the block's address is
  // wave-uniform, the lane's byte offset within it (the slot stage_direct gives the lane,
  // with its swizzle) is computed once, and the LDS destination is the wave's part of the
  // stage. The ragged last block keeps stage_direct, which repeats row N - 1.
  constexpr int CP = stage_copies<D, kBlock / 64>();
  unsigned coff[CP];
#pragma unroll
  for (int p = 0; p < CP; ++p) coff[p] = stage_lane_offset<D, kBlock / 64>(p, wave, lane);
  const unsigned lds_wave = lds_addr(lds) + (unsigned)wave * 1024u;
  auto issue = [&](int slot, int j) __attribute__((always_inline)) {
    const int r0 = (kt_begin + j) * kTile;
    if (r0 + kTile <= N) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        stage_block_saddr<D, kBlock / 64>(src[t] + (size_t)r0 * D, coff,
                                          lds_wave + (unsigned)((slot * NT + t) * G::ROW_ELEMS * (int)sizeof(T)));
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        stage_direct<TT, D, kBlock / 64, true>(src[t], r0, N, stage(slot, t), wave, lane);
    }
  };

  V bq[DK];
  load_resident<TT, D>(reinterpret_cast<const T*>(a.Q) + base, qi, N, g, bq);
  settle_regs(bq);
  for (int j = 0; j < AHEAD && j < nsteps; ++j) issue(j, j);
  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = zero16();
  float m = -1e30f, l = 0.f;
  const float cs = a.tau * kLog2e;
  wait_vmem();
  __syncthreads();

  f32x16 sb[2];
  V pp[2][NK];
  auto scores = [&](f32x16& s, int slot) __attribute__((always_inline)) {
    s = zero16();
#pragma unroll
    for (int t = 0; t < DK; ++t) s = TT::mfma(lds_row_op<TT, D>(stage(slot, 0), n, t, g), bq[t], s);
  };
  // Weights of step j from its score tile, with their sum added to l.
  auto weights = [&](const f32x16& sc, V (&p)[NK], int j) __attribute__((always_inline)) {
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = fast_exp2(fmaf(sc[r], cs, -m));
      ls += pr;
      vset<TT>(p[r >> 3], r & 7, pr);
    }
    const int k0 = (kt_begin + j) * kTile;
    const bool masked = k0 + kTile > N || (CAUSAL && k0 + kTile - 1 > q0);  // wave-uniform
    // the ballot first, so that the sum and its test stay with the products and exponentials
    const bool redo = __ballot(lazy_redo(ls, lazy_limit<TT>())) != 0;
    if (redo || masked) {
      bool keep[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kappa(r, g);
        keep[r] = !masked || (key < N && (!CAUSAL || key <= qi));
      }
      auto form = [&]() __attribute__((always_inline)) {
        ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = keep[r] ? fast_exp2(fmaf(sc[r], cs, -m)) : 0.f;
          ls += pr;
          vset<TT>(p[r >> 3], r & 7, pr);
        }
      };
      if (masked) form();
      if (__ballot(lazy_redo(ls, lazy_limit<TT>()))) {  // move m to the row maximum
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (keep[r]) mx = fmaxf(mx, sc[r] * cs);
        mx = pair_max32(mx);
        const float mnew = fmaxf(m, mx);
        const float f = fast_exp2(m - mnew);
        l *= f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] *= f;
        m = mnew;
        form();
      }
    }
    l += ls;
  };

  if (nsteps > 0 && active(0)) scores(sb[0], 0);
  if (nsteps > 1 && active(1)) scores(sb[1], 1);
  if (nsteps > 0 && active(0)) weights(sb[0], pp[0], 0);

  // FULL: steps j + 1 .. j + AHEAD exist (no tail checks)
  auto step = [&](auto I_c, int j, auto full_c) __attribute__((always_inline)) {
    constexpr int I = decltype(I_c)::value;
    constexpr bool FULL = decltype(full_c)::value;
    constexpr int SJ = I % NBUF, SJ2 = (I + 2) % NBUF, SJA = (I + AHEAD) % NBUF;
    const bool copy = FULL || j + AHEAD < nsteps;
    if (copy) issue(SJA, j + AHEAD);  // slot SJA was last read in step j + AHEAD - NBUF < j
    if ((FULL || j + 2 < nsteps) && active(j + 2)) scores(sb[I % 2], SJ2);
    if (active(j)) {
#pragma unroll
      for (int t = 0; t < NK; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb] = TT::mfma(lds_tr_op<TT, D>(stage(SJ, 1), mb, t, lane), pp[I % 2][t], acc[mb]);
    }
    if ((FULL || j + 1 < nsteps) && active(j + 1)) weights(sb[(I + 1) % 2], pp[(I + 1) % 2], j + 1);
    if (copy) wait_vmem_keep<(AHEAD - 3) * COPIES>();  // stage j + 3 has landed
    else wait_vmem();
    __syncthreads();
  };
  using Full = std::true_type;
  using Tail = std::false_type;
  auto full = [&](auto I_c, int j) __attribute__((always_inline)) { step(I_c, j, Full{}); };
  auto tail = [&](auto I_c, int j) __attribute__((always_inline)) { step(I_c, j, Tail{}); };
  int j = 0;
  for (; j + NBUF + AHEAD <= nsteps; j += NBUF) unroll_steps(full, j, std::make_integer_sequence<int, NBUF>{});
  unroll_steps_until(tail, j, nsteps, std::make_integer_sequence<int, NBUF + AHEAD>{});

  fwd_finish<TT, D, WITH_D>(acc, m, l, qt, bh, split, wave, lane, a);
}

// Merge the split records of one wave (fixed split order) and apply the epilogue.
// A workgroup takes one wave's record (grid x = query tile x wave); the 8 threads
// 8 n .. 8 n + 7 hold row n of it: record lanes n and n + 32 (g) times slots
// 4 r4 .. 4 r4 + 3 of every head-dim block (quad-major tiles: for one r4, the 8 rows
// of a wave read two runs of 128 contiguous bytes), four times as many waves are in
// flight as with one thread per record lane, and D = dO . O of the row is summed
// over those 8 adjacent lanes.
template <class TT, int D, bool WITH_D>
__global__ __launch_bounds__(kBlock) void attn_fwd_combine_kernel(FwdArgs a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  constexpr int MB = G::MB;
  constexpr int MOFF = MB * 16 * 64;  // m[64], then l[64], after the accumulators
  const int t = threadIdx.x, n = t >> 3, g = (t >> 2) & 1, r4 = t & 3;
  const int L = g * 32 + n;
  const int qt = blockIdx.x >> 2, wave = blockIdx.x & 3, bh = blockIdx.y;
  const int N = a.N;
  const int qi = qt * kBlockRows + wave * kTile + n;
  auto rec = [&](int sp) {
    return a.part + ((((size_t)sp * a.BH + bh) * row_tiles(N) + qt) * 4 + wave) * fwd_record_floats(D);
  };
  float M = -1e30f;  // m is the same in record lanes n and n + 32
  for (int sp = 0; sp < a.nsplit; ++sp) M = fmaxf(M, rec(sp)[MOFF + L]);
  f32x4 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float llo = 0.f, lhi = 0.f;
  for (int sp = 0; sp < a.nsplit; ++sp) {
    const float* R = rec(sp);
    const float w = fast_exp2(R[MOFF + L] - M);
    llo += w * R[MOFF + 64 + n];
    lhi += w * R[MOFF + 96 + n];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] += w * tile_quad(R + mb * 1024, L, r4);
  }
  const float lt = llo + lhi;
  const float inv = 1.f / lt;
  const size_t row = (size_t)bh * N + qi;
  float dot = 0.f;
  if (qi < N) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int dim = mb * 32 + kappa(r4 * 4, g);
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = acc[mb][e] * inv;
      store4<TT>(reinterpret_cast<T*>(a.O) + row * D + dim, o[0], o[1], o[2], o[3]);
      if constexpr (WITH_D) {
        float x[4];
        load4<TT>(reinterpret_cast<const T*>(a.dO) + row * D + dim, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) dot += x[e] * o[e];
      }
    }
  }
  if constexpr (WITH_D) {
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    dot += __shfl_xor(dot, 4);
  }
  if (qi >= N || (t & 7) != 0) return;
  a.L[row] = M * kLn2 + __logf(lt);
  if constexpr (WITH_D) a.D[row] = dot;
}

// Single-buffered variant (transposed LDS copy of V); used for float32 inputs.
template <class TT, int D, bool CAUSAL, bool WITH_D>
__global__ __launch_bounds__(kBlock) void attn_fwd_simple_kernel(FwdArgs a) {
  using G = Geo<TT, D>;
  using T = typename TT::elem;
  using V = typename TT::vec;
  extern __shared__ __align__(16) unsigned char smem[];
  T* krow = reinterpret_cast<T*>(smem);
  T* vt = krow + G::ROW_ELEMS;

  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int g = lane >> 5, n = lane & 31;
  const int N = a.N, bh = blockIdx.y;
  const size_t base = (size_t)bh * N * D;
  const T* Q = reinterpret_cast<const T*>(a.Q) + base;
  const T* K = reinterpret_cast<const T*>(a.K) + base;
  const T* Vm = reinterpret_cast<const T*>(a.V) + base;
  const int q0 = blockIdx.x * kBlockRows + wave * kTile;
  const int qi = q0 + n;

  V bq[G::DK];
  load_resident<TT, D>(Q, qi, N, g, bq);
  f32x16 acc[G::MB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) acc[mb] = zero16();
  float m = -1e30f, l = 0.f;
  const float cs = a.tau * kLog2e;

  int nkt = (N + kTile - 1) / kTile;
  if (CAUSAL) nkt = min(nkt, (int)(blockIdx.x + 1) * (kBlockRows / kTile));
  for (int kt = 0; kt < nkt; ++kt) {
    const int k0 = kt * kTile;
    __syncthreads();
    stage_tile<TT, D>(K, k0, N, krow, nullptr, tid, kBlock);
    stage_tile<TT, D>(Vm, k0, N, nullptr, vt, tid, kBlock);
    __syncthreads();
    if (CAUSAL && k0 > q0 + kTile - 1) continue;  // every key after every query of this wave

    f32x16 s = zero16();
#pragma unroll
    for (int t = 0; t < G::DK; ++t) s = TT::mfma(lds_row_op<TT, D>(krow, n, t, g), bq[t], s);

    float mx = -1e30f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + kappa(r, g);
      const bool ok = key < N && (!CAUSAL || key <= qi);
      s[r] = ok ? s[r] * cs : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = pair_max32(mx);
    const float mnew = fmaxf(m, mx);
    const float sc = fast_exp2(m - mnew);
    l *= sc;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) acc[mb] *= sc;
    V pp[G::NK];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(s[r] - mnew);
      l += p;
      vset<TT>(pp[r / TT::KPL], r % TT::KPL, p);
    }
    m = mnew;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int t = 0; t < G::NK; ++t) acc[mb] = TT::mfma(lds_t_op<TT, D>(vt, mb * 32 + n, t, g), pp[t], acc[mb]);
  }

  const float lt = pair_sum32(l);
  const float inv = 1.f / lt;
  if (qi < N) {
    T* O = reinterpret_cast<T*>(a.O) + base + (size_t)qi * D;
    const T* dO = WITH_D ? reinterpret_cast<const T*>(a.dO) + base + (size_t)qi * D : nullptr;
    float dot = 0.f;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dim = mb * 32 + kappa(r4 * 4, g);
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[mb][r4 * 4 + e] * inv;
        store4<TT>(O + dim, o[0], o[1], o[2], o[3]);
        if constexpr (WITH_D) {
          float x[4];
          load4<TT>(dO + dim, x);
#pragma unroll
          for (int e = 0; e < 4; ++e) dot += x[e] * o[e];
        }
      }
    // lanes n and n + 32 own the same query, so the exchanges below stay paired
    if (g == 0) a.L[(size_t)bh * N + qi] = m * kLn2 + __logf(lt);
    if constexpr (WITH_D) {
      dot = pair_sum32(dot);
      if (g == 0) a.D[(size_t)bh * N + qi] = dot;
    }
  }
}

template <class TT, int D, bool CAUSAL, bool WITH_D>
static hipError_t launch_fwd_t(const FwdArgs& a, int BH, hipStream_t s) {
  using G = Geo<TT, D>;
  if constexpr (TT::KPL == 1) {
    const size_t lds = (size_t)(G::ROW_ELEMS + G::T_ELEMS) * sizeof(typename TT::elem);
    hipError_t e = ensure_lds(&attn_fwd_simple_kernel<TT, D, CAUSAL, WITH_D>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_fwd_simple_kernel<TT, D, CAUSAL, WITH_D>), dim3(row_tiles(a.N), BH), dim3(kBlock), lds,
                       s, a);
  } else {
    // The skew pays off on long non-causal sweeps at d = 64: at d = 128 it needs more than
    // 256 registers, and causal sweeps are too short for its longer prologue and tail.
    if constexpr (FB_FWD_SKEW && D == 64 && !CAUSAL) {
      const size_t lds = (size_t)kFwdSkewSlots * 2 * G::ROW_ELEMS * sizeof(typename TT::elem);
      hipError_t e = ensure_lds(&attn_fwd_skew_kernel<TT, D, CAUSAL, WITH_D>, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_fwd_skew_kernel<TT, D, CAUSAL, WITH_D>), dim3(row_tiles(a.N), BH, a.nsplit),
                         dim3(kBlock), lds, s, a);
    } else {
      const size_t lds = (size_t)3 * 2 * G::ROW_ELEMS * sizeof(typename TT::elem);
      hipError_t e = ensure_lds(&attn_fwd_kernel<TT, D, CAUSAL, WITH_D>, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_fwd_kernel<TT, D, CAUSAL, WITH_D>), dim3(row_tiles(a.N), BH, a.nsplit),
                         dim3(kBlock), lds, s, a);
    }
  }
  return hipGetLastError();
}

template <class TT, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, bool causal, int BH, hipStream_t s) {
  const bool wd = a.D != nullptr;
  if (causal) return wd ? launch_fwd_t<TT, D, true, true>(a, BH, s) : launch_fwd_t<TT, D, true, false>(a, BH, s);
  return wd ? launch_fwd_t<TT, D, false, true>(a, BH, s) : launch_fwd_t<TT, D, false, false>(a, BH, s);
}

template <class TT>
static hipError_t launch_fwd_tt(const FwdArgs& a, int d, bool causal, int BH, hipStream_t s) {
  return d == 64 ? launch_fwd_d<TT, 64>(a, causal, BH, s) : launch_fwd_d<TT, 128>(a, causal, BH, s);
}

hipError_t launch_attn_fwd(const FwdArgs& a, DT dt, int d, bool causal, int BH, hipStream_t s) {
  if (dt == DT::F32 && a.nsplit != 1) return hipErrorInvalidValue;
  switch (dt) {
    case DT::BF16: return launch_fwd_tt<BF16>(a, d, causal, BH, s);
    case DT::F16: return launch_fwd_tt<F16>(a, d, causal, BH, s);
    default: return launch_fwd_tt<F32>(a, d, causal, BH, s);
  }
}

template <class TT, int D>
static hipError_t launch_fc_t(const FwdArgs& a, hipStream_t s) {
  dim3 grid(row_tiles(a.N) * 4, a.BH);  // one workgroup per wave record
  if (a.D) {
    hipLaunchKernelGGL((attn_fwd_combine_kernel<TT, D, true>), grid, dim3(kBlock), 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_fwd_combine_kernel<TT, D, false>), grid, dim3(kBlock), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_combine(const FwdArgs& a, DT dt, int d, hipStream_t s) {
  switch (dt) {
    case DT::BF16: return d == 64 ? launch_fc_t<BF16, 64>(a, s) : launch_fc_t<BF16, 128>(a, s);
    case DT::F16: return d == 64 ? launch_fc_t<F16, 64>(a, s) : launch_fc_t<F16, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fb
