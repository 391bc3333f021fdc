// Per-row sampling of the next token from float32 logits, and the float32 -> bf16 row
// conversion that feeds the LM head from a caller's hidden states.
//
// The pages' serving loop applies its own sampling parameters (temperature, top-p) to
// each member of a batch ("Hugging Face BLOOM Inference Optimization", Webserver
// Architecture and Request Handling); the definitions are the textbook ones (nucleus
// sampling: Holtzman et al., "The Curious Case of Neural Text Degeneration", Section
// 3.1).  Each row is cut into NB slices of whole 256-id segments, one 256-thread block
// per (slice, row), and the work runs as a chain of launches that pass partial results
// through a caller workspace:
//   1. max      T <= 0 rows: the slice's greedy candidate (largest logit, lowest id);
//               others: the slice maximum.
//   2. mass     m = max over the slices; p_v = exp((l_v - m) / T) in float32 (__expf),
//               taken as a fixed-point integer P_v = round(p_v * 2^40) (p_v <= 1, so a
//               row's total fits 64 bits for up to 2^23 tokens); the slice's total mass
//               and its mass in 256 buckets of the top 8 bits of the token's key (an
//               order-preserving map of the logit to 32 bits).
//   3. levels   nucleus threshold by radix selection, 8 key bits per launch: every block
//      1..3     sums the slices' bucket masses and takes the highest bucket whose mass,
//               plus the mass above it, still reaches top_p times the total (all blocks
//               compute the same choice; block 0 records it), then buckets the next 8
//               bits of the tokens matching the chosen prefix.  The threshold t is the
//               largest key whose kept mass (the P_v of tokens with key >= t) reaches
//               top_p times the total; tokens tied with the boundary token share its key
//               and are kept.  top_p >= 1 keeps every token, top_p <= 0 the largest
//               logits only (those rows skip the levels).
//   4. segments the kept mass of every 256-id segment of the slice.
//   5. draw     one block per row: r = floor(u * M) for the kept mass M, an integer scan
//               of the segment masses, and one wave walks the segment holding r (an
//               integer scan of its 256 ids): the first id whose running mass exceeds r.
// Every mass is an exact integer sum, so no result depends on the order of additions:
// the LDS bucket atomics and the slice split leave the tokens bitwise reproducible.
#include <algorithm>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

typedef unsigned long long u64;

constexpr int kSmpThreads = 256;
constexpr int kSmpWaves = kSmpThreads / 64;
constexpr int kSmpSub = 4;          // bucket histograms per wave (lane % kSmpSub)

// order-preserving map of a (non-NaN) float to an unsigned key
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workspace layout for B rows of V tokens, NB slices of SL ids (a multiple of 256).
struct SmpLayout {
  int NB, SL, nseg;
  size_t pmax, pidx, pS, hist, state, seg, total;
};

SmpLayout sample_layout(int B, int V) {
  SmpLayout L{};
  const int nseg = (V + 255) / 256;
  // up to 64 slices per row while the grid is small, at least 16 (while B <= 128) so
  // that large batches still fill the chip; measured at batch 128: 4 slices 209 us, 16
  // slices 190 us per call
  const int Bc = std::max(B, 1);
  int nb = std::max(1, std::max(std::min(64, 512 / Bc), std::min(16, 2048 / Bc)));
  nb = std::min(nb, nseg);
  const int segs_per_slice = (nseg + nb - 1) / nb;
  L.SL = 256 * segs_per_slice;
  L.NB = (V + L.SL - 1) / L.SL;
  L.nseg = nseg;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += (bytes + 255) & ~(size_t)255; return o; };
  L.pmax = take((size_t)B * L.NB * 4);
  L.pidx = take((size_t)B * L.NB * 4);
  L.pS = take((size_t)B * L.NB * 8);
  L.hist = take((size_t)2 * B * L.NB * 256 * 8);
  L.state = take((size_t)B * 2 * 4 * 8);      // [B][2 buffers][prefix, above, thr, -]
  L.seg = take((size_t)B * nseg * 8);
  L.total = off;
  return L;
}

struct SmpArgs {
  const float *logits;
  int V, NB, SL, nseg;
  const float *temperature, *top_p, *uniform;
  const int *step_dev;
  int *out;
  float *pmax;
  int *pidx;
  u64 *pS, *hist, *state, *seg;
};

// One pass over ids [v0, v1) of a row: f(value, id), 16-byte loads (8 in flight per
// thread) when the row is 16-byte aligned (v0 is a multiple of 256), else 4-byte loads.
template <typename F>
__device__ __forceinline__ void slice_pass(const float *__restrict__ l, int v0, int v1, F &&f) {
  const int tid = threadIdx.x;
  if ((((uintptr_t)l) & 15) == 0) {
    const int n4 = (v1 - v0) >> 2;
    const float4 *l4 = (const float4 *)(l + v0);
    for (int i0 = 0; i0 < n4; i0 += kSmpThreads * 8) {
      float4 x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = l4[min(i0 + k * kSmpThreads + tid, n4 - 1)];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k * kSmpThreads + tid;
        if (i < n4) {
          const int v = v0 + 4 * i;
          f(x[k].x, v); f(x[k].y, v + 1); f(x[k].z, v + 2); f(x[k].w, v + 3);
        }
      }
    }
    for (int v = v0 + 4 * n4 + tid; v < v1; v += kSmpThreads) f(l[v], v);
  } else {
    for (int v = v0 + tid; v < v1; v += kSmpThreads) f(l[v], v);
  }
}

__device__ __forceinline__ u64 wave_sum_u64(u64 v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// P = round(p * 2^40): p * 2^40 is exact in float32; its integer part split at 2^32
__device__ __forceinline__ u64 fix40(float p) {
  const float f = p * 1099511627776.0f;
  const uint32_t hi = (uint32_t)(f * 2.3283064365386963e-10f);   // floor(f / 2^32) <= 256
  const float rem = f - (float)hi * 4294967296.0f;                  // exact, in [0, 2^32)
  return ((u64)hi << 32) + (u64)(uint32_t)rintf(rem);
}

struct RowParams {
  float T, P, m, invT;
  bool greedy, radix;
};

// Block-wide reductions of the NB per-slice partials of row b (NB <= 64: one value per
// thread of the first wave).  Every thread of the block must call them.
__device__ __forceinline__ float row_max(const SmpArgs &a, int b) {
  __shared__ float rm;
  if (threadIdx.x < 64) {
    float v = (int)threadIdx.x < a.NB ? a.pmax[(size_t)b * a.NB + threadIdx.x] : -INFINITY;
    v = wave_max(v);
    if (threadIdx.x == 0) rm = v;
  }
  __syncthreads();
  return rm;
}

__device__ __forceinline__ u64 row_total(const SmpArgs &a, int b) {
  __shared__ u64 rt;
  if (threadIdx.x < 64) {
    u64 v = (int)threadIdx.x < a.NB ? a.pS[(size_t)b * a.NB + threadIdx.x] : 0ull;
    v = wave_sum_u64(v);
    if (threadIdx.x == 0) rt = v;
  }
  __syncthreads();
  return rt;
}

__device__ __forceinline__ RowParams row_params(const SmpArgs &a, int b, bool with_max) {
  RowParams r;
  r.T = a.temperature[b];
  r.P = a.top_p[b];
  r.invT = 1.0f / r.T;
  // a positive temperature whose reciprocal overflows float32 (T below ~2.9e-39) samples
  // from the limit of softmax(logits / T), the largest logits: it is taken as greedy
  r.greedy = !(r.T > 0.f) || !(r.invT <= 3.402823466e38f);
  r.radix = r.P > 0.f && r.P < 1.f;
  r.m = with_max ? row_max(a, b) : -INFINITY;
  return r;
}

__device__ __forceinline__ u64 pfix(const RowParams &rp, float x) {
  return fix40(__expf((x - rp.m) * rp.invT));
}

// 1. slice maximum (greedy rows: with the lowest id among the maxima)
__global__ __launch_bounds__(kSmpThreads) void k_smp_max(SmpArgs a) {
  __shared__ float sv[kSmpWaves];
  __shared__ int si[kSmpWaves];
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const float *l = a.logits + (size_t)b * a.V;
  const int v0 = j * a.SL, v1 = min(a.V, v0 + a.SL);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  slice_pass(l, v0, v1, [&](float x, int v) { argmax_take(bv, bi, x, v); });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    argmax_take(bv, bi, ov, oi);
  }
  if (lane == 0) { sv[wid] = bv; si[wid] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kSmpWaves; ++w) argmax_take(bv, bi, sv[w], si[w]);
    a.pmax[(size_t)b * a.NB + j] = bv;
    a.pidx[(size_t)b * a.NB + j] = bi;
  }
}

// Bucket masses of one slice: tokens whose key matches `prefix` in the bits above
// `shift + 8` add P into bucket (key >> shift) & 255.  Writes the block's 256 sums.
template <bool TOTAL>
__device__ __forceinline__ void slice_hist(const SmpArgs &a, const RowParams &rp, int b, int j,
                                           uint32_t prefix, int shift, u64 *dst, u64 *total) {
  __shared__ u64 h[kSmpWaves * kSmpSub][256];
  __shared__ u64 red[kSmpWaves];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i < kSmpWaves * kSmpSub * 256; i += kSmpThreads) (&h[0][0])[i] = 0ull;
  __syncthreads();
  const float *l = a.logits + (size_t)b * a.V;
  const int v0 = j * a.SL, v1 = min(a.V, v0 + a.SL);
  const uint32_t hi_mask = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
  const int hrow = wid * kSmpSub + (lane & (kSmpSub - 1));
  u64 s = 0;
  slice_pass(l, v0, v1, [&](float x, int) {
    const uint32_t k = order_key(x);
    if (TOTAL) {
      const u64 q = pfix(rp, x);
      s += q;
      if (rp.radix && q) atomicAdd(&h[hrow][k >> 24], q);
    } else if ((k & hi_mask) == prefix) {
      const u64 q = pfix(rp, x);
      if (q) atomicAdd(&h[hrow][(k >> shift) & 255u], q);
    }
  });
  if (TOTAL) {
    s = wave_sum_u64(s);
    if (lane == 0) red[wid] = s;
  }
  __syncthreads();
  if (TOTAL && tid == 0) {
    u64 t = 0;
    for (int w = 0; w < kSmpWaves; ++w) t += red[w];
    *total = t;
  }
  if (TOTAL && !rp.radix) return;
  {
    const int bk = tid;   // kSmpThreads == 256 buckets
    u64 t = 0;
#pragma unroll
    for (int w = 0; w < kSmpWaves * kSmpSub; ++w) t += h[w][bk];
    dst[bk] = t;
  }
}

// 2. total mass and the first radix level
__global__ __launch_bounds__(kSmpThreads) void k_smp_mass(SmpArgs a) {
  const int j = blockIdx.x, b = blockIdx.y;
  const RowParams rp = row_params(a, b, true);
  if (rp.greedy) return;
  slice_hist<true>(a, rp, b, j, 0u, 24, a.hist + ((size_t)b * a.NB + j) * 256,
                   a.pS + (size_t)b * a.NB + j);
}

// Selection of one radix level from the slices' bucket masses src[NB][256]: the highest
// bucket whose mass (plus `above`) reaches `target`.  All threads return the choice.
__device__ __forceinline__ void select_bucket(const SmpArgs &a, const u64 *src, u64 target,
                                              u64 above, int &bucket, u64 &above_out) {
  __shared__ u64 tot[256];
  __shared__ int sb;
  __shared__ u64 sa;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  {
    u64 t = 0;
#pragma unroll 8
    for (int jj = 0; jj < a.NB; ++jj) t += src[(size_t)jj * 256 + tid];
    tot[tid] = t;
  }
  __syncthreads();
  if (wid == 0) {
    const u64 c0 = tot[4 * lane], c1 = tot[4 * lane + 1], c2 = tot[4 * lane + 2],
              c3 = tot[4 * lane + 3];
    const u64 mine = c0 + c1 + c2 + c3;
    u64 suf = mine;                                // over lanes >= this one
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const u64 t = __shfl_down(suf, o, 64);
      if (lane + o < 64) suf += t;
    }
    const unsigned long long ok = __ballot(above + suf >= target);
    // lane 0's suffix is the whole prefix group, which reaches the target
    const int jl = ok ? 63 - __clzll((long long)ok) : 0;
    if (lane == jl) {
      u64 run = above + (suf - mine);
      int bk = 4 * lane;
      u64 ab = run;
      const u64 cs[4] = {c0, c1, c2, c3};
      for (int e = 3; e >= 0; --e) {
        if (run + cs[e] >= target) { bk = 4 * lane + e; ab = run; break; }
        run += cs[e];
      }
      sb = bk;
      sa = ab;
    }
  }
  __syncthreads();
  bucket = sb;
  above_out = sa;
}


__device__ __forceinline__ u64 row_target(const RowParams &rp, u64 S) {
  return (u64)ceil((double)rp.P * (double)S);
}

// 3. radix level `level` (1..3): choose the bucket of level - 1, bucket the next bits
__global__ __launch_bounds__(kSmpThreads) void k_smp_level(SmpArgs a, int level) {
  const int j = blockIdx.x, b = blockIdx.y;
  const RowParams rp = row_params(a, b, true);
  if (rp.greedy || !rp.radix) return;
  const u64 target = row_target(rp, row_total(a, b));
  // state of the previous level (its prefix and the mass above it): none for level 1
  const u64 *st_in = a.state + ((size_t)b * 2 + (level & 1)) * 4;
  u64 *st_out = a.state + ((size_t)b * 2 + ((level + 1) & 1)) * 4;
  uint32_t prefix = level == 1 ? 0u : (uint32_t)st_in[0];
  const u64 above = level == 1 ? 0ull : st_in[1];
  const u64 *src = a.hist + ((size_t)((level - 1) & 1) * gridDim.y + b) * a.NB * 256;
  int bucket;
  u64 above2;
  select_bucket(a, src, target, above, bucket, above2);
  const int shift_prev = 24 - 8 * (level - 1);
  prefix |= (uint32_t)bucket << shift_prev;
  if (j == 0 && threadIdx.x == 0) { st_out[0] = prefix; st_out[1] = above2; }
  u64 *dst = a.hist + (((size_t)(level & 1) * gridDim.y + b) * a.NB + j) * 256;
  slice_hist<false>(a, rp, b, j, prefix, 24 - 8 * level, dst, nullptr);
}

// Threshold key of the row (after the last level's choice)
__device__ __forceinline__ uint32_t row_threshold(const SmpArgs &a, const RowParams &rp, int b,
                                                  int nrows) {
  if (!(rp.P > 0.f)) return order_key(rp.m);
  if (!rp.radix) return 0u;
  const u64 target = row_target(rp, row_total(a, b));
  const u64 *st_in = a.state + ((size_t)b * 2 + (4 & 1)) * 4;    // written by level 3
  const uint32_t prefix = (uint32_t)st_in[0];
  const u64 *src = a.hist + ((size_t)(3 & 1) * nrows + b) * a.NB * 256;
  int bucket;
  u64 above2;
  select_bucket(a, src, target, st_in[1], bucket, above2);
  return prefix | (uint32_t)bucket;
}

// 4. kept mass of each 256-id segment of the slice
__global__ __launch_bounds__(kSmpThreads) void k_smp_seg(SmpArgs a) {
  const int j = blockIdx.x, b = blockIdx.y, lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const RowParams rp = row_params(a, b, true);
  if (rp.greedy) return;
  const uint32_t thr = row_threshold(a, rp, b, gridDim.y);
  if (j == 0 && threadIdx.x == 0) a.state[(size_t)b * 2 * 4 + 2] = thr;
  const float *l = a.logits + (size_t)b * a.V;
  const int s0 = j * (a.SL / 256), s1 = min(a.nseg, s0 + a.SL / 256);
  for (int sg0 = s0 + wid; sg0 < s1; sg0 += kSmpWaves * 4) {
    float x[4][4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[k][e] = l[min(a.V - 1, (sg0 + k * kSmpWaves) * 256 + 4 * lane + e)];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int sg = sg0 + k * kSmpWaves;
      u64 acc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = sg * 256 + 4 * lane + e;
        if (v < a.V && order_key(x[k][e]) >= thr) acc += pfix(rp, x[k][e]);
      }
      acc = wave_sum_u64(acc);
      if (lane == 0 && sg < s1) a.seg[(size_t)b * a.nseg + sg] = acc;
    }
  }
}

// 5. draw (one block per row); greedy rows merge the slices' candidates
__global__ __launch_bounds__(kSmpThreads) void k_smp_draw(SmpArgs a) {
  __shared__ u64 wsum[kSmpWaves];
  __shared__ int owner;
  __shared__ u64 own_lo;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const RowParams rp = row_params(a, b, true);
  if (rp.greedy) {
    if (tid == 0) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
      for (int j = 0; j < a.NB; ++j)
        argmax_take(bv, bi, a.pmax[(size_t)b * a.NB + j], a.pidx[(size_t)b * a.NB + j]);
      a.out[b] = bi == 0x7fffffff ? 0 : bi;
    }
    return;
  }
  const uint32_t thr = (uint32_t)a.state[(size_t)b * 2 * 4 + 2];
  const u64 *seg = a.seg + (size_t)b * a.nseg;
  // each thread takes a run of consecutive segments; exclusive integer scan
  const int per = (a.nseg + kSmpThreads - 1) / kSmpThreads;
  const int g0 = min(a.nseg, tid * per), g1 = min(a.nseg, g0 + per);
  u64 mine = 0;
  for (int g = g0; g < g1; ++g) mine += seg[g];
  u64 incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wid] = incl;
  if (tid == 0) owner = -1;
  __syncthreads();
  u64 base = 0, M = 0;
  for (int w = 0; w < kSmpWaves; ++w) {
    if (w < wid) base += wsum[w];
    M += wsum[w];
  }
  const int step = a.step_dev ? *a.step_dev : 0;
  const float uu = fminf(fmaxf(a.uniform[(size_t)step * gridDim.x + b], 0.f), 0x1.fffffep-1f);
  const u64 r = (u64)((double)uu * (double)M);   // < M
  u64 lo = base + incl - mine;
  for (int g = g0; g < g1; ++g) {
    const u64 hi = lo + seg[g];
    if (lo <= r && r < hi) { owner = g; own_lo = lo; }
    lo = hi;
  }
  __syncthreads();
  if (wid != 0) return;
  const int og = owner;
  int chosen = -1;
  if (og >= 0) {
    const float *l = a.logits + (size_t)b * a.V;
    const int v0 = og * 256 + 4 * lane;
    u64 q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = v0 + e;
      q[e] = 0;
      if (v < a.V) {
        const float x = l[v];
        if (order_key(x) >= thr) q[e] = pfix(rp, x);
      }
    }
    const u64 c1 = q[0], c2 = c1 + q[1], c3 = c2 + q[2], c4 = c3 + q[3];
    u64 inc = c4;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const u64 t = __shfl_up(inc, o, 64);
      if (lane >= o) inc += t;
    }
    const u64 ex = own_lo + (inc - c4);
    int first = 4;
    if (ex + c4 > r) first = (ex + c1 > r) ? 0 : (ex + c2 > r) ? 1 : (ex + c3 > r) ? 2 : 3;
    const unsigned long long hit = __ballot(first < 4);
    if (hit) {
      const int fl = __ffsll((long long)hit) - 1;
      chosen = og * 256 + 4 * fl + __shfl(first, fl, 64);
    }
  }
  if (lane == 0) a.out[b] = chosen >= 0 ? chosen : 0;
}

size_t sample_workspace_bytes(int batch, int vocab) {
  return sample_layout(batch, vocab).total;
}

hipError_t launch_sample_rows(const float *logits, int batch, int V, const float *temperature,
                              const float *top_p, const float *uniform, int *out, void *ws,
                              hipStream_t st, const int *step_dev) {
  if (batch <= 0) return hipSuccess;
  const SmpLayout L = sample_layout(batch, V);
  char *w = (char *)ws;
  SmpArgs a{logits, V, L.NB, L.SL, L.nseg, temperature, top_p, uniform, step_dev, out,
            (float *)(w + L.pmax), (int *)(w + L.pidx), (u64 *)(w + L.pS),
            (u64 *)(w + L.hist), (u64 *)(w + L.state), (u64 *)(w + L.seg)};
  const dim3 grid(L.NB, batch), block(kSmpThreads);
  hipLaunchKernelGGL(k_smp_max, grid, block, 0, st, a);
  hipLaunchKernelGGL(k_smp_mass, grid, block, 0, st, a);
  for (int level = 1; level <= 3; ++level)
    hipLaunchKernelGGL(k_smp_level, grid, block, 0, st, a, level);
  hipLaunchKernelGGL(k_smp_seg, grid, block, 0, st, a);
  hipLaunchKernelGGL(k_smp_draw, dim3(batch), block, 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// the same sampling with a library-held scratch buffer (no workspace argument)
// ---------------------------------------------------------------------------
// For callers that cannot allocate device memory (code under graph capture, tight
// serving loops).  The partial results live in a file-scope device array; each GPU
// holds its own copy, whose device address is looked up once per device (with that
// device current) and kept.  Kernels receive that address, never the array's name
// (which is a host-side stand-in in host code).  Calls on one GPU share the array:
// calls that overlap in time on one GPU race.  Nothing in it needs to start at zero
// (every partial is written before it is read within a call).
static __device__ __align__(256) unsigned char scratch[kSampleScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t sample_scratch_ptr(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_sample_rows_static(const float *logits, int batch, int V,
                                     const float *temperature, const float *top_p,
                                     const float *uniform, int *out, hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  if (sample_workspace_bytes(batch, V) > (size_t)kSampleScratchBytes) return hipErrorInvalidValue;
  void *ws = nullptr;
  const hipError_t e = sample_scratch_ptr(&ws);
  if (e != hipSuccess) return e;
  return launch_sample_rows(logits, batch, V, temperature, top_p, uniform, out, ws, st);
}

// y = x (n float32 values) in activation format fmt: bf16 (round to nearest even),
// float32, or two bf16 planes hi, lo (lo plane n elements after hi).
__global__ void k_f32_to_act(const float *__restrict__ x, void *__restrict__ y, int fmt,
                             size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    act_store(y, fmt, i, n, x[i]);
}

hipError_t launch_f32_to_act(const float *x, void *y, int fmt, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_f32_to_act, dim3(blocks), dim3(256), 0, st, x, y, fmt, n);
  return hipGetLastError();
}

}  // namespace bl
