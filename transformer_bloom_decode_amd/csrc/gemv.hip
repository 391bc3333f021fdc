// Decode GEMV on the vector ALU for up to 4 activation rows (the batch-1..4 decode
// step and LM head): each wave streams one or two weight rows in 1 KB non-temporal
// loads (whole rows, or half rows on a pair of waves, at once when the grid leaves wave
// slots empty); the block's output rows are finished by the fused epilogue (or an
// argmax for the LM head).  The pages'
// analysis ("DeepSpeed Inference ...", Section III.A) is that small-batch inference is
// bound by reading the weights once; this kernel is built around streaming W at full
// bandwidth.  Its planning (rows per wave, pieces in flight) and launch live here too.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// ---------------------------------------------------------------------------
// decode GEMV on the vector ALU (M <= 4 activation rows)
// ---------------------------------------------------------------------------
// Each wave owns R consecutive weight rows over the full K (or, with KS > 1, over its
// part of K, below).  Per step every lane loads one 16-byte piece of each of its rows,
// so a wave load instruction covers 1 KB of one row contiguously; the loads are
// non-temporal (streamed weights are not kept in the caches that hold activations and
// the KV cache).  Weights are widened to float32 in registers and multiplied by the
// matching activation values with fmaf; each lane keeps R*M running sums, reduced
// across the wave at the end.  U steps are loaded ahead of the one being multiplied.
template <typename TW> struct VOps;

template <> struct VOps<bf16_t> {
  static constexpr int kPerLane = 8;                      // elements per 16-byte piece
  static __device__ __forceinline__ void widen(u32x4 w, float f[8]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) { f[2 * t] = lo_bf(w[t]); f[2 * t + 1] = hi_bf(w[t]); }
  }
};

template <> struct VOps<int8_t> {
  static constexpr int kPerLane = 16;
  static __device__ __forceinline__ void widen(u32x4 w, float f[16]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * t + b] = (float)(int)(int8_t)(w[t] >> (8 * b));
  }
};

// Activation pieces: 8 elements of a bf16 row, or 4 of a float32 row, per 16 bytes.
template <typename TX> struct XOps;
template <> struct XOps<bf16_t> {
  static constexpr int kPer16 = 8;
  static __device__ __forceinline__ void widen(u32x4 v, float *f) {
#pragma unroll
    for (int t = 0; t < 4; ++t) { f[2 * t] = lo_bf(v[t]); f[2 * t + 1] = hi_bf(v[t]); }
  }
};
template <> struct XOps<float> {
  static constexpr int kPer16 = 4;
  static __device__ __forceinline__ void widen(u32x4 v, float *f) {
#pragma unroll
    for (int t = 0; t < 4; ++t) f[t] = __uint_as_float(v[t]);
  }
};
template <> struct XOps<int8_t> {   // W8A8 activation codes (the row scale comes later)
  static constexpr int kPer16 = 16;
  static __device__ __forceinline__ void widen(u32x4 v, float *f) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int b = 0; b < 4; ++b) f[4 * t + b] = (float)(int)(int8_t)(v[t] >> (8 * b));
  }
};
template <> struct XOps<f16_t> {
  static constexpr int kPer16 = 8;
  static __device__ __forceinline__ void widen(u32x4 v, float *f) {
#pragma unroll
    for (int t = 0; t < 4; ++t) { f[2 * t] = f16lo(v[t]); f[2 * t + 1] = f16hi(v[t]); }
  }
};

// Folded LayerNorm ("DeepSpeed Inference ...", Section III.D fuses each LayerNorm with
// the GeMM that follows it), one activation row.  The consumer GEMV reads g * x and
// finishes y_n = rstd (sum_k W[n][k] (g x)_k - mean c_n) + d_n, with c_n = sum_k W[n][k]
// g_k and d_n = sum_k W[n][k] b_k + bias_n precomputed (ep.ln_cd) and mean, rstd of x
// from the sums that the blocks of the residual GEMV before it accumulated: every wave
// copies the accumulators (1 KB) straight into its own LDS region before it requests
// the weights, and forms the totals from there after its dot products (no barrier).

// The residual GEMV's share: each block adds the float64 sums of its new x[n] and
// x[n]^2 (xn: this lane's value, 0 for lanes without an output) to slot
// blockIdx % kStatSlots.
__device__ __forceinline__ void fold_stats_add(const EpiParams &ep, float xn) {
  __shared__ double red[2][4];
  double s1 = xn, s2 = (double)xn * xn;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s1 += __shfl_xor(s1, o, 64);
    s2 += __shfl_xor(s2, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = s1;
    red[1][threadIdx.x >> 6] = s2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long *a = ep.fold_stats + 2 * (blockIdx.x % kStatSlots);
    stat_add(a, (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]), kStatFrac1);
    stat_add(a + 1, (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]), kStatFrac2);
  }
}

// DB: double-buffered (the next U pieces per row are issued before the current ones
// are used) or single-buffered (U pieces per row issued at once, then used; with U >=
// the row's pieces, a wave issues its whole row in one go, which keeps the most bytes
// in flight when the grid is too small to fill every wave slot).  TX: activation type
// (bf16, or float32 when the model keeps float32 activations).
// KS: waves per weight row.  KS = 2 splits each row's K range in halves between the two
// waves of a pair (rows per block 4 R / 2): the half-length waves finish in half the
// time, so the drain of the last round of waves is shorter; the second half's dot
// product reaches the first through LDS and is added after the first's, in that order.
template <typename TW, typename TP, typename TX, int MR, int R, int U, bool DB, int KS = 1>
__global__ __launch_bounds__(256) void k_gemv_valu(const TX *__restrict__ X,
                                                   const TW *__restrict__ W, int M, int N, int K,
                                                   EpiParams ep) {
  using VO = VOps<TW>;
  using XO = XOps<TX>;
  constexpr int E = VO::kPerLane;
  constexpr int XP = E / XO::kPer16;                      // 16-byte activation pieces per step
  __shared__ float am_v[4][MR];
  __shared__ int am_i[4][MR];
  static_assert(KS == 1 || (KS == 2 && !DB), "the K split runs on single-buffered rows");
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int wrow = KS == 1 ? wid : (wid >> 1);   // the wave's row group in the block
  const int half = KS == 1 ? 0 : (wid & 1);      // its part of the K range
  const int row0 = (blockIdx.x * (4 / KS) + wrow) * R;
  const TW *wr[R];
#pragma unroll
  for (int i = 0; i < R; ++i) wr[i] = W + (size_t)min(row0 + i, N - 1) * K;
  const TX *xr[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) xr[m] = X + (size_t)min(m, M - 1) * K;

  // A folded LayerNorm (one row against bf16 weights; ln_fold_supported): one copy of
  // its accumulators per wave
  constexpr bool kFold = MR == 1 && sizeof(TW) == 2;
  __shared__ __attribute__((aligned(16))) unsigned long long lst[kFold ? 4 * kStatWords : 1];
  unsigned long long *wst = lst + (kFold ? kStatWords * __builtin_amdgcn_readfirstlane(wid) : 0);
  // lane l < R*MR finishes output (row0 + l / MR, activation row l % MR).  One row of
  // bf16 / fp16 activations against bf16 weights (the batch-1 decode step): the lane's
  // epilogue operands are requested now, with the weights (measured on MI355X: the
  // residual projections waited for them at the end of every wave); the other variants
  // keep their registers for the weights and load them in the epilogue.
  constexpr bool kPre = MR == 1 && sizeof(TW) == 2 && sizeof(TX) == 2;
  const int on = row0 + lane / MR, om = lane % MR;
  const bool has_out =
      half == 0 && lane < R * MR && on < N && om < M && ep.mode != EPI_ARGMAX;
  EpiPre pre{};
  if constexpr (kPre) {
    if (has_out) pre = epi_prefetch<TP>(ep, om, on);
  }
  float fold_c = 0.f, fold_d = 0.f;   // c_n and d_n of the lane's output row
  if constexpr (kFold) {
    if (ep.ln_stats) {
      if (half == 0 && lane < R && row0 + lane < N) {
        fold_c = ep.ln_cd[row0 + lane];
        fold_d = ep.ln_cd[N + row0 + lane];
      }
      static_assert(kStatWords * 8 % 1024 == 0, "whole 1 KB copies");
#pragma unroll
      for (int j = 0; j < kStatWords * 8 / 1024; ++j)
        __builtin_amdgcn_global_load_lds(
            (const void *)((const unsigned char *)ep.ln_stats + j * 1024 + lane * 16),
            (__attribute__((address_space(3))) void *)((unsigned char *)wst + j * 1024), 16, 0,
            0);
    }
  }

  float acc[R][MR];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[i][m] = 0.f;

  const int step = 64 * E;                                // elements per wave step
  const int nsteps_all = (K + step - 1) / step;
  const int sbeg = half * ((nsteps_all + KS - 1) / KS);   // the wave's steps [sbeg, nsteps)
  const int nsteps = KS == 1 ? nsteps_all : min(nsteps_all, sbeg + (nsteps_all + KS - 1) / KS);
  u32x4 cw[U][R], cx[U][MR][XP];

  auto load = [&](int s0, u32x4(&w)[U][R], u32x4(&x)[U][MR][XP]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s0 + u) * step + lane * E;
      const bool ok = (s0 + u) < nsteps && k < K;
#pragma unroll
      for (int i = 0; i < R; ++i)
        w[u][i] = ok ? __builtin_nontemporal_load((const u32x4 *)(wr[i] + k)) : zero4();
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int p = 0; p < XP; ++p)
          x[u][m][p] = ok ? *(const u32x4 *)(xr[m] + k + XO::kPer16 * p) : zero4();
    }
  };

  auto compute = [&]() {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xf[MR][E];
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int p = 0; p < XP; ++p) XO::widen(cx[u][m][p], &xf[m][XO::kPer16 * p]);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float wf[E];
        VO::widen(cw[u][i], wf);
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[i][m] = fmaf(wf[e], xf[m][e], acc[i][m]);
      }
    }
  };

  if constexpr (DB) {
    u32x4 nw[U][R], nx[U][MR][XP];
    load(0, cw, cx);
    for (int s0 = 0; s0 < nsteps; s0 += U) {
      if (s0 + U < nsteps) load(s0 + U, nw, nx);
      compute();
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int i = 0; i < R; ++i) cw[u][i] = nw[u][i];
#pragma unroll
        for (int m = 0; m < MR; ++m)
#pragma unroll
          for (int p = 0; p < XP; ++p) cx[u][m][p] = nx[u][m][p];
      }
    }
  } else {
    for (int s0 = sbeg; s0 < nsteps; s0 += U) {
      load(s0, cw, cx);
      compute();
    }
  }

#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[i][m] = wave_sum(acc[i][m]);
  if constexpr (KS == 2) {
    __shared__ float kpart[2][R * MR];   // second halves' dot products, per row group
    if (half == 1 && lane == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < MR; ++m) kpart[wrow][i * MR + m] = acc[i][m];
    }
    __syncthreads();
    if (half == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[i][m] += kpart[wrow][i * MR + m];
    }
  }

  float ln_mean = 0.f, ln_rstd = 0.f;
  if constexpr (kFold) {
    if (ep.ln_stats) {
      // vmcnt(0): the wave's copies have landed in its LDS region
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
      double s1, s2;
      stat_totals_wave(wst, s1, s2);
      const double md = s1 / K;
      const double var = s2 / K - md * md;
      ln_mean = (float)md;
      ln_rstd = 1.0f / sqrtf((float)(var > 0.0 ? var : 0.0) + ep.ln_eps);
    }
  }

  if (ep.mode == EPI_ARGMAX) {
    // best of this wave's R rows per activation row, then of the block's 4 waves
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float bv = -INFINITY;
        int bi = min(row0, N - 1);
#pragma unroll
        for (int i = 0; i < R; ++i)
          if (row0 + i < N) argmax_take(bv, bi, acc[i][m], row0 + i);
        am_v[wid][m] = bv;
        am_i[wid][m] = bi;
      }
    }
    __syncthreads();
    if (threadIdx.x < MR && threadIdx.x < M) {
      const int m = threadIdx.x;
      float bv = am_v[0][m];
      int bi = am_i[0][m];
      for (int w = 1; w < 4; ++w) argmax_take(bv, bi, am_v[w][m], am_i[w][m]);
      ep.am_val[(size_t)m * ep.am_stride + blockIdx.x] = bv;
      ep.am_idx[(size_t)m * ep.am_stride + blockIdx.x] = bi;
    }
    return;
  }
  float xn = 0.f;   // the updated residual value of the lane's output (EPI_RESID)
  if (lane < R * MR) {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int m = 0; m < MR; ++m)
        if (lane == i * MR + m) v = acc[i][m];
    if (has_out) {
      if constexpr (kFold) {
        if (ep.ln_stats) v = ln_rstd * (v - ln_mean * fold_c) + fold_d;
      }
      if constexpr (kPre) xn = epilogue_pre<TP>(ep, om, on, v, pre);
      else xn = epilogue<TP>(ep, om, on, v);
    }
  }
  if constexpr (kFold) {
    if (ep.fold_stats) fold_stats_add(ep, xn);
  }
}

// ---------------------------------------------------------------------------
// one-row decode GEMV with the preceding LayerNorm as its prologue
// ---------------------------------------------------------------------------
// For the linears that consume a LayerNorm (QKV after the input LN, MLP-up after the
// post-attention LN), the pages fuse the LN into the GeMM ("DeepSpeed Inference ...",
// Section III.D).  At one activation row this kernel does so without a separate pass,
// and spends the LayerNorm's latency while the weights are in flight.  Vector memory
// loads of a wave complete in issue order, so the order of issue is what matters:
//   1. the float32 residual row x, then gamma and beta, into registers (NV float4 /
//      4-element pieces per thread);
//   2. the first UA of the wave's U non-temporal 1 KB weight-row loads;
//   3. the statistics (mean, then the biased variance of the centred registers: two
//      passes, float32, fixed order, so every block gets the same bits), which wait
//      only for x; then gamma * (x - mean) * rstd + beta, rounded to bf16, into LDS;
//   4. the rest of the weight row (issued once x, gamma and beta have freed their
//      registers), then the dot products with the activations read from LDS.
// The block's barriers wait for LDS operations only: a barrier with a memory fence
// would also wait for the weight loads in flight.
// Used for rows of up to kGemvLnMaxK elements.  There every block's extra reads (the
// float32 row, gamma and beta: 8 bytes per element) are small next to its weight rows,
// and the two launches it saves per layer are most of a short layer's time: measured
// on MI355X, BLOOM-560m (hidden 1024) at batch 1, 0.840 -> 0.683 ms per step eager and
// 0.802 -> 0.666 ms with the graph loop, identical tokens.  At hidden 14336 the same
// kernel was slower than LayerNorm + GEMV (QKV 40.2 against 28.3 + 4.6 us), so long rows
// keep the separate LayerNorm.
constexpr int kGemvLnMaxK = 4096;

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt unconstrained), then s_barrier
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// sum over the block's 4 waves, through `sh` (4 floats used by this call only)
__device__ __forceinline__ float gemv_block_sum(float v, float *sh) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  lds_barrier();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

template <typename TW, typename TX, int NV>
__global__ __launch_bounds__(256) void k_gemv_ln(const float *__restrict__ x,
                                                 const bf16_t *__restrict__ g,
                                                 const bf16_t *__restrict__ b, float eps,
                                                 const TW *__restrict__ W, int N, int K,
                                                 EpiParams ep) {
  using VO = VOps<TW>;
  constexpr int E = VO::kPerLane;
  constexpr int step = 64 * E;                   // elements per wave load
  constexpr int U = NV * 1024 / step;            // loads per weight row
  constexpr int UA = U < 20 ? U : 20;            // issued before the LayerNorm
  __shared__ __align__(16) TX a_s[NV * 1024];
  __shared__ float red[2][4];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wid;
  const TW *wr = W + (size_t)min(row, N - 1) * K;

  // Every load is issued unconditionally (addresses past the row clamped to its last
  // piece, values past it never used): loads under a branch would make the compiler
  // assume the worst about which ones are outstanding and wait for all of them.
  float4 v[NV];
  Param4<bf16_t> gv[NV], bv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int col = min(4 * (threadIdx.x + i * 256), K - 4);
    v[i] = *(const float4 *)(x + col);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int col = min(4 * (threadIdx.x + i * 256), K - 4);
    gv[i].load(g + col);
    bv[i].load(b + col);
  }
  u32x4 cw[U];
#pragma unroll
  for (int u = 0; u < UA; ++u)
    cw[u] = __builtin_nontemporal_load((const u32x4 *)(wr + min(u * step + lane * E, K - E)));
  // keep the scheduler from starting the statistics (and their wait for x) before every
  // load above is issued
  __builtin_amdgcn_sched_barrier(0);

  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (4 * (threadIdx.x + i * 256) < K) s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float mean = gemv_block_sum(s, red[0]) / (float)K;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (4 * (threadIdx.x + i * 256) < K) {
      const float p0 = v[i].x - mean, p1 = v[i].y - mean, p2 = v[i].z - mean, p3 = v[i].w - mean;
      ss += (p0 * p0 + p1 * p1) + (p2 * p2 + p3 * p3);
    }
  const float rstd = 1.0f / sqrtf(gemv_block_sum(ss, red[1]) / (float)K + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int col = 4 * (threadIdx.x + i * 256);
    if (col < K) {
      const float4 y = ln_apply<bf16_t>(v[i], mean, rstd, gv[i], bv[i]);
      if constexpr (sizeof(TX) == 4) {
        *(float4 *)(a_s + col) = y;
      } else if constexpr (std::is_same<TX, f16_t>::value) {
        uint2 t;
        t.x = (uint32_t)f2h_bits(y.x) | ((uint32_t)f2h_bits(y.y) << 16);
        t.y = (uint32_t)f2h_bits(y.z) | ((uint32_t)f2h_bits(y.w) << 16);
        *(uint2 *)(a_s + col) = t;
      } else {
        uint2 t;
        t.x = (uint32_t)f2bf(y.x) | ((uint32_t)f2bf(y.y) << 16);
        t.y = (uint32_t)f2bf(y.z) | ((uint32_t)f2bf(y.w) << 16);
        *(uint2 *)(a_s + col) = t;
      }
    }
  }
#pragma unroll
  for (int u = UA; u < U; ++u)
    cw[u] = __builtin_nontemporal_load((const u32x4 *)(wr + min(u * step + lane * E, K - E)));
  lds_barrier();

  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int k = u * step + lane * E;
    if (k < K) {
      float wf[E];
      VO::widen(cw[u], wf);
      constexpr int PX = XOps<TX>::kPer16;
#pragma unroll
      for (int p = 0; p < E / PX; ++p) {
        float af[PX];
        XOps<TX>::widen(*(const u32x4 *)(a_s + k + PX * p), af);
#pragma unroll
        for (int t = 0; t < PX; ++t) acc = fmaf(wf[PX * p + t], af[t], acc);
      }
    }
  }
  acc = wave_sum(acc);
  if (lane == 0 && row < N) epilogue<bf16_t>(ep, 0, row, acc);
}

bool gemv_ln_supported(int wdtype, int M, int K) {
  return M == 1 && (wdtype == WT_BF16 || wdtype == WT_INT8) && K >= 16 && K % 16 == 0 &&
         K <= kGemvLnMaxK;
}

template <typename TW, typename TX>
static void launch_gemv_ln_t(int N, int K, const float *x, const void *g, const void *b,
                             float eps, const void *W, const EpiParams &ep, hipStream_t st) {
  const dim3 grid((N + 3) / 4), block(256);
  const bf16_t *gg = (const bf16_t *)g, *bb = (const bf16_t *)b;
  const TW *w = (const TW *)W;
  const int nv = (K + 1023) / 1024;
  if (nv <= 1)
    BL_LAUNCH((k_gemv_ln<TW, TX, 1>), grid, block, 0, st, x, gg, bb, eps, w, N, K, ep);
  else
    BL_LAUNCH((k_gemv_ln<TW, TX, 4>), grid, block, 0, st, x, gg, bb, eps, w, N, K, ep);
}

template <typename TW>
static void launch_gemv_ln_w(int x_fmt, int N, int K, const float *x, const void *g,
                             const void *b, float eps, const void *W, const EpiParams &ep,
                             hipStream_t st) {
  if (x_fmt == AF_F32) launch_gemv_ln_t<TW, float>(N, K, x, g, b, eps, W, ep, st);
  else if (x_fmt == AF_F16) launch_gemv_ln_t<TW, f16_t>(N, K, x, g, b, eps, W, ep, st);
  else launch_gemv_ln_t<TW, bf16_t>(N, K, x, g, b, eps, W, ep, st);
}

hipError_t launch_gemv_ln(int wdtype, int x_fmt, int N, int K, const float *x, const void *g,
                          const void *b, float eps, const void *W, const EpiParams &ep,
                          hipStream_t st) {
  if (N <= 0) return hipSuccess;
  if (!gemv_ln_supported(wdtype, 1, K)) return hipErrorInvalidValue;
  if (wdtype == WT_BF16) launch_gemv_ln_w<bf16_t>(x_fmt, N, K, x, g, b, eps, W, ep, st);
  else launch_gemv_ln_w<int8_t>(x_fmt, N, K, x, g, b, eps, W, ep, st);
  return hipGetLastError();
}

LinearPlan plan_valu(int wdtype, int M, int N, int K) {
  LinearPlan p{};
  p.M = M; p.N = N; p.K = K;
  p.kind = LIN_VALU;
  p.mt = M <= 1 ? 1 : (M <= 2 ? 2 : 4);
  // Default: 2 rows per wave, 4 pieces per row double-buffered (8 KB in flight per
  // wave); enough when the grid fills every wave slot (LM head) or rows are short.
  // Batch-1 bf16 linears with long rows and grids that leave wave slots empty issue
  // a wave's whole row at once instead (14-28 KB in flight per wave): measured on
  // MI355X, QKV 5376 x 14336 5.15 -> 5.88 TB/s, up 7168 x 14336 5.75 -> 6.47,
  // down 14336 x 7168 6.39 -> 6.60.
  p.vr = 2;
  p.vu = p.mt == 4 ? 2 : 4;
  p.vdb = true;
  p.ks = 1;
  const int pieces = (K + 511) / 512;  // 1 KB wave loads of bf16
  if (p.mt == 1 && wdtype == WT_BF16 && N < 65536 && pieces > 4 && pieces <= 28) {
    p.vr = 1;
    p.vu = pieces <= 16 ? 16 : 28;
    p.vdb = false;
    // rows of 17-28 pieces (QKV and MLP-up of the 176B share, K = 14336): each row in
    // two halves of at most 14 pieces, on the two waves of a pair
    if (pieces > 16) { p.vu = 14; p.ks = 2; }
  }
  // Batch-1 bf16 linears with short rows (up to 2048) and many of them (the attention
  // output projection of the 176B share, 14336 x 1792): 4 whole rows per wave, so the
  // grid fits the chip's wave slots in one round; measured on MI355X 12.6 -> 11.4 us.
  if (p.mt == 1 && wdtype == WT_BF16 && N >= 8192 && pieces <= 4 && K >= 1024) {
    p.vr = 4;
    p.vu = 4;
    p.vdb = false;
  }
  const int rows_per_block = 4 * p.vr / p.ks;
  p.grid_x = (N + rows_per_block - 1) / rows_per_block;
  p.splits = 1;
  return p;
}


template <typename TW, typename TP, typename TX>
static void launch_valu_t(const LinearPlan &p, const void *X, const void *W, const EpiParams &ep,
                          hipStream_t st) {
  const dim3 grid(p.grid_x), block(256);
  const TX *x = (const TX *)X;
  const TW *w = (const TW *)W;
  if constexpr (std::is_same<TW, bf16_t>::value) {
    if (p.vr == 1 && p.mt == 1 && !p.vdb) {
      if (p.ks == 2)
        BL_LAUNCH((k_gemv_valu<TW, TP, TX, 1, 1, 14, false, 2>), grid, block, 0, st, x, w, p.M, p.N, p.K, ep);
      else if (p.vu == 16)
        BL_LAUNCH((k_gemv_valu<TW, TP, TX, 1, 1, 16, false>), grid, block, 0, st, x, w, p.M, p.N, p.K, ep);
      else
        BL_LAUNCH((k_gemv_valu<TW, TP, TX, 1, 1, 28, false>), grid, block, 0, st, x, w, p.M, p.N, p.K, ep);
      return;
    }
    if (p.vr == 4 && p.mt == 1 && !p.vdb) {
      BL_LAUNCH((k_gemv_valu<TW, TP, TX, 1, 4, 4, false>), grid, block, 0, st, x, w, p.M, p.N, p.K, ep);
      return;
    }
  }
  switch (p.mt) {
    case 1: BL_LAUNCH((k_gemv_valu<TW, TP, TX, 1, 2, 4, true>), grid, block, 0, st, x, w, p.M, p.N, p.K, ep); break;
    case 2: BL_LAUNCH((k_gemv_valu<TW, TP, TX, 2, 2, 4, true>), grid, block, 0, st, x, w, p.M, p.N, p.K, ep); break;
    default: BL_LAUNCH((k_gemv_valu<TW, TP, TX, 4, 2, 2, true>), grid, block, 0, st, x, w, p.M, p.N, p.K, ep); break;
  }
}

template <typename TW>
static void launch_valu_w(const LinearPlan &p, const void *X, const void *W, const EpiParams &ep,
                          hipStream_t st) {
  if (p.x_fmt == AF_F32) launch_valu_t<TW, bf16_t, float>(p, X, W, ep, st);
  else if (p.x_fmt == AF_F16) launch_valu_t<TW, bf16_t, f16_t>(p, X, W, ep, st);
  else if (p.x_fmt == AF_I8) {
    if constexpr (sizeof(TW) == 1) launch_valu_t<TW, bf16_t, int8_t>(p, X, W, ep, st);
  }
  else launch_valu_t<TW, bf16_t, bf16_t>(p, X, W, ep, st);
}

// A folded LayerNorm runs on one-row vector-ALU GEMVs against bf16 weights: its
// consumer (ln_stats and ln_cd set; not the LM head) and the residual projection before
// it (fold_g, fold_u and fold_stats set, EPI_RESID).
bool ln_fold_supported(int wdtype, const LinearPlan &p, const EpiParams &ep) {
  if (wdtype != WT_BF16 || p.kind != LIN_VALU || p.M != 1 || p.mt != 1 || p.splits != 1)
    return false;
  if (ep.ln_stats && (!ep.ln_cd || ep.mode == EPI_ARGMAX)) return false;
  if ((ep.fold_g || ep.fold_stats) && (ep.mode != EPI_RESID || !ep.fold_g || !ep.fold_u ||
                                       !ep.fold_stats))
    return false;
  return true;
}

hipError_t launch_valu(int wdtype, const LinearPlan &p, const void *X, const void *W,
                       const EpiParams &ep, hipStream_t st) {
  if (p.x_fmt == AF_I8 && (wdtype != WT_INT8 || !ep.xscale)) return hipErrorInvalidValue;
  if ((ep.ln_stats || ep.fold_g || ep.fold_stats) && !ln_fold_supported(wdtype, p, ep))
    return hipErrorInvalidValue;
  if (wdtype == WT_BF16) launch_valu_w<bf16_t>(p, X, W, ep, st);
  else launch_valu_w<int8_t>(p, X, W, ep, st);
  return hipGetLastError();
}

// c_n = sum_k W[n][k] g_k and d_n = sum_k W[n][k] b_k + bias_n for one linear (one
// wave per row; float64 sums in a fixed order, rounded once to float32).
__global__ __launch_bounds__(256) void k_ln_fold(const bf16_t *__restrict__ W,
                                                 const bf16_t *__restrict__ g,
                                                 const bf16_t *__restrict__ b,
                                                 const bf16_t *__restrict__ bias, int N, int K,
                                                 float *__restrict__ c, float *__restrict__ d) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const bf16_t *wr = W + (size_t)n * K;
  double sc = 0.0, sd = 0.0;
  for (int k = lane; k < K; k += 64) {
    const double w = (double)bf2f(wr[k]);
    sc += w * (double)bf2f(g[k]);
    sd += w * (double)bf2f(b[k]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sc += __shfl_xor(sc, o, 64);
    sd += __shfl_xor(sd, o, 64);
  }
  if (lane == 0) {
    c[n] = (float)sc;
    d[n] = (float)(sd + (bias ? (double)bf2f(bias[n]) : 0.0));
  }
}

hipError_t launch_ln_fold(const void *W, const void *g, const void *b, const void *bias, int N,
                          int K, float *c, float *d, hipStream_t st) {
  if (N <= 0) return hipSuccess;
  BL_LAUNCH(k_ln_fold, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, st, (const bf16_t *)W,
            (const bf16_t *)g, (const bf16_t *)b, (const bf16_t *)bias, N, K, c, d);
  return hipGetLastError();
}

}  // namespace bl
