// Per-row sampling of the next token from float32 logits, and the float32 -> bf16 row
// conversion that feeds the LM head from a caller's hidden states.
//
// The pages' serving loop applies its own sampling parameters (temperature, top-p) to
// each member of a batch ("Hugging Face BLOOM Inference Optimization", Webserver
// Architecture and Request Handling); the definitions are the textbook ones (nucleus
// sampling: Holtzman et al., "The Curious Case of Neural Text Degeneration", Section
// 3.1).  One 1024-thread block per row:
//   1. T <= 0: greedy (lowest id among the largest logits).
//   2. m = max logit; p_v = exp((l_v - m) / T) in float32 (__expf), taken as a fixed-point
//      integer P_v = round(p_v * 2^40) (p_v <= 1, so a row's total fits 64 bits for up
//      to 2^23 tokens).  Every mass below is an exact integer sum of these P_v, so it
//      does not depend on the order of the additions: bucket sums can use LDS atomics
//      and the result is still bitwise reproducible.
//   3. Nucleus: the largest threshold key t (keys: an order-preserving map of the
//      logits to 32-bit integers) whose kept mass, the sum of P_v over key(l_v) >= t,
//      reaches top_p times the total.  Found by radix selection, 8 key bits per level:
//      a level adds P into 256 buckets (4 histograms per wave) by the next 8 key bits
//      among the tokens matching the bits chosen so far, and takes the highest bucket
//      whose mass, plus the mass above it, still reaches the target.  The first level
//      is fused with the total-mass pass; later levels evaluate exp only for the tokens
//      of the chosen bucket.  Tokens tied with the boundary token share its key and are
//      kept.  top_p >= 1 keeps every token; top_p <= 0 the largest logits only.
//   4. Draw: r = floor(u * M) for the kept mass M; the kept tokens in id order are cut
//      into segments of 256 ids, the segments' masses are scanned, the segment holding
//      r is walked by one wave (an integer scan of its 256 ids), and the first id whose
//      running mass exceeds r is taken.
// The logits are re-read from memory (L2) in each pass (max, mass + first level, three
// more levels, the segment masses), with 16-byte loads, several in flight per thread.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kSmpThreads = 1024;
constexpr int kSmpWaves = kSmpThreads / 64;
constexpr int kSmpUnroll = 8;       // float4 loads in flight per thread in a pass
constexpr int kSmpMaxSeg = 4096;    // segments of the draw (LDS entries)
constexpr int kSmpSub = 4;          // bucket histograms per wave (lane % kSmpSub)

// order-preserving map of a (non-NaN) float to an unsigned key
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One pass over a row of V floats: f(value, id) for every element, each thread taking
// the same elements in every pass.  The 16-byte-aligned body is read as float4,
// kSmpUnroll loads issued before any is used; the few elements before and after it
// one by one.
template <typename F>
__device__ __forceinline__ void row_pass(const float *__restrict__ l, int V, F &&f) {
  const int head = min(V, (int)((-(int)(((uintptr_t)l) >> 2)) & 3));
  const int n4 = (V - head) >> 2;
  const float4 *l4 = (const float4 *)(l + head);
  const int tid = threadIdx.x;
  for (int i0 = 0; i0 < n4; i0 += kSmpThreads * kSmpUnroll) {
    float4 x[kSmpUnroll];
#pragma unroll
    for (int k = 0; k < kSmpUnroll; ++k)
      x[k] = l4[min(i0 + k * kSmpThreads + tid, n4 - 1)];
#pragma unroll
    for (int k = 0; k < kSmpUnroll; ++k) {
      const int i = i0 + k * kSmpThreads + tid;
      if (i < n4) {
        const int v = head + 4 * i;
        f(x[k].x, v); f(x[k].y, v + 1); f(x[k].z, v + 2); f(x[k].w, v + 3);
      }
    }
  }
  const int tail0 = head + 4 * n4;
  if (tid < head) f(l[tid], tid);
  if (tid < V - tail0) f(l[tail0 + tid], tail0 + tid);
}

typedef unsigned long long u64;

__global__ __launch_bounds__(kSmpThreads) void k_sample_rows(const float *__restrict__ logits,
                                                             int V,
                                                             const float *__restrict__ temperature,
                                                             const float *__restrict__ top_p,
                                                             const float *__restrict__ uniform,
                                                             int *__restrict__ out) {
  __shared__ float sh[kSmpWaves];
  __shared__ int ish[kSmpWaves];
  __shared__ u64 hist[kSmpWaves * kSmpSub][256];   // bucket masses; reused as segments
  __shared__ u64 tot[256];
  __shared__ u64 ush[kSmpWaves];
  __shared__ u64 sel_above;
  __shared__ int sel_bucket;
  __shared__ int owner;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const float *l = logits + (size_t)b * V;
  const float T = temperature[b];
  const float Pp = top_p[b];

  if (!(T > 0.f)) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    row_pass(l, V, [&](float x, int v) { argmax_take(bv, bi, x, v); });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      argmax_take(bv, bi, ov, oi);
    }
    if (lane == 0) { sh[wid] = bv; ish[wid] = bi; }
    __syncthreads();
    if (tid == 0) {
      float v0 = sh[0];
      int i0 = ish[0];
      for (int w = 1; w < kSmpWaves; ++w) argmax_take(v0, i0, sh[w], ish[w]);
      out[b] = i0 == 0x7fffffff ? 0 : i0;
    }
    return;
  }

  // block sum of a 64-bit integer (exact, any order)
  auto block_sum_u64 = [&](u64 v) -> u64 {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) ush[wid] = v;
    __syncthreads();
    u64 t = 0;
#pragma unroll
    for (int w = 0; w < kSmpWaves; ++w) t += ush[w];
    __syncthreads();
    return t;
  };
  auto clear_hist = [&]() {
    for (int i = tid; i < kSmpWaves * kSmpSub * 256; i += kSmpThreads) (&hist[0][0])[i] = 0ull;
  };
  const int hrow = wid * kSmpSub + (lane & (kSmpSub - 1));

  // 2. maximum
  float m = -INFINITY;
  row_pass(l, V, [&](float x, int) { m = fmaxf(m, x); });
  m = block_max<kSmpWaves>(m, sh);
  const float invT = 1.0f / T;
  // P = round(p * 2^40): p * 2^40 is exact in float32; its integer part is split at 2^32
  auto pfix = [&](float x) -> u64 {
    const float f = __expf((x - m) * invT) * 1099511627776.0f;
    const uint32_t hi = (uint32_t)(f * 2.3283064365386963e-10f);   // floor(f / 2^32) < 256
    const float rem = f - (float)hi * 4294967296.0f;                  // exact, in [0, 2^32)
    return ((u64)hi << 32) + (u64)(uint32_t)rintf(rem);
  };

  // 3. total mass and the nucleus threshold (level 0 fused with the total)
  const bool radix = Pp > 0.f && Pp < 1.f;
  clear_hist();
  __syncthreads();
  u64 s = 0;
  row_pass(l, V, [&](float x, int) {
    const u64 q = pfix(x);
    s += q;
    if (radix && q) atomicAdd(&hist[hrow][order_key(x) >> 24], q);
  });
  const u64 S = block_sum_u64(s);      // its barriers also order the histogram adds
  uint32_t thr = 0u;                   // keeps every token
  if (!(Pp > 0.f)) {
    thr = order_key(m);
  } else if (radix) {
    const u64 target = (u64)ceil((double)Pp * (double)S);
    uint32_t prefix = 0u;
    u64 above = 0;
    for (int level = 0; level < 4; ++level) {
      const int shift = 24 - 8 * level;
      if (level > 0) {
        const uint32_t hi_mask = 0xffffffffu << (shift + 8);
        clear_hist();
        __syncthreads();
        row_pass(l, V, [&](float x, int) {
          const uint32_t k = order_key(x);
          if ((k & hi_mask) == prefix) {
            const u64 q = pfix(x);
            if (q) atomicAdd(&hist[hrow][(k >> shift) & 255u], q);
          }
        });
        __syncthreads();
      }
      if (tid < 256) {
        u64 t = 0;
#pragma unroll
        for (int w = 0; w < kSmpWaves * kSmpSub; ++w) t += hist[w][tid];
        tot[tid] = t;
      }
      __syncthreads();
      if (wid == 0) {
        // lane j holds buckets 4j .. 4j + 3; suffix sums from the top bucket down
        const u64 c0 = tot[4 * lane], c1 = tot[4 * lane + 1], c2 = tot[4 * lane + 2],
                  c3 = tot[4 * lane + 3];
        const u64 mine = c0 + c1 + c2 + c3;
        u64 suf = mine;                            // sum over lanes >= this one
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const u64 t = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += t;
        }
        const u64 after = suf - mine;              // buckets above this lane's four
        const unsigned long long ok = __ballot(above + suf >= target);
        // the highest lane whose suffix (with everything above the prefix) reaches the
        // target; it exists, since lane 0's suffix is the whole prefix group
        const int jl = 63 - __clzll((long long)ok);
        if (lane == jl) {
          u64 run = above + after;
          int bk = 4 * lane;
          u64 ab = run;
          const u64 cs[4] = {c0, c1, c2, c3};
          for (int e = 3; e >= 0; --e) {
            if (run + cs[e] >= target) { bk = 4 * lane + e; ab = run; break; }
            run += cs[e];
          }
          sel_bucket = bk;
          sel_above = ab;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sel_bucket << shift;
      above = sel_above;
      __syncthreads();
    }
    thr = prefix;
  }

  // 4. draw in id order over segments of 256 ids (G = 256 * subs ids when the row has
  // more than kSmpMaxSeg * 256 tokens)
  const int subs = (V + 256 * kSmpMaxSeg - 1) / (256 * kSmpMaxSeg);
  const int G = 256 * subs;
  const int nseg = (V + G - 1) / G;
  u64 *seg = &hist[0][0];                      // kSmpMaxSeg entries
  constexpr int kSegBatch = 4;                 // segments per wave whose loads go together
  for (int sg0 = wid; sg0 < nseg; sg0 += kSmpWaves * kSegBatch) {
    u64 acc[kSegBatch];
#pragma unroll
    for (int k = 0; k < kSegBatch; ++k) acc[k] = 0;
    for (int sb = 0; sb < subs; ++sb) {
      float x[kSegBatch][4];
#pragma unroll
      for (int k = 0; k < kSegBatch; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[k][e] = l[min(V - 1, (sg0 + k * kSmpWaves) * G + sb * 256 + 4 * lane + e)];
#pragma unroll
      for (int k = 0; k < kSegBatch; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = (sg0 + k * kSmpWaves) * G + sb * 256 + 4 * lane + e;
          if (v < V && order_key(x[k][e]) >= thr) acc[k] += pfix(x[k][e]);
        }
    }
#pragma unroll
    for (int k = 0; k < kSegBatch; ++k) {
      u64 t = acc[k];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
      if (lane == 0 && sg0 + k * kSmpWaves < nseg) seg[sg0 + k * kSmpWaves] = t;
    }
  }
  __syncthreads();
  // inclusive scan of the segment masses: each thread owns 4 consecutive segments
  u64 loc[4];
  u64 run = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int sg = 4 * tid + e;
    run += sg < nseg ? seg[sg] : 0ull;
    loc[e] = run;
  }
  u64 incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) ush[wid] = incl;
  __syncthreads();
  u64 wbase = 0;
  for (int w = 0; w < wid; ++w) wbase += ush[w];
  u64 M = 0;
#pragma unroll
  for (int w = 0; w < kSmpWaves; ++w) M += ush[w];
  const u64 tbase = wbase + incl - run;        // mass before this thread's segments
  const float uu = fminf(fmaxf(uniform[b], 0.f), 0x1.fffffep-1f);
  const u64 r = (u64)((double)uu * (double)M);   // < M
  if (tid == 0) owner = -1;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int sg = 4 * tid + e;
    const u64 lo = tbase + (e ? loc[e - 1] : 0ull), hi = tbase + loc[e];
    if (sg < nseg && lo <= r && r < hi) {
      owner = sg;
      sel_above = lo;
    }
  }
  __syncthreads();
  const int own = owner;
  if (wid == 0) {
    int chosen = -1;
    if (own >= 0) {
      u64 base = sel_above;
      for (int sb = 0; sb < subs && chosen < 0; ++sb) {
        const int v0 = own * G + sb * 256 + 4 * lane;
        u64 q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int v = v0 + e;
          q[e] = 0;
          if (v < V) {
            const float x = l[v];
            if (order_key(x) >= thr) q[e] = pfix(x);
          }
        }
        const u64 c1 = q[0], c2 = c1 + q[1], c3 = c2 + q[2], c4 = c3 + q[3];
        u64 inc = c4;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const u64 t = __shfl_up(inc, o, 64);
          if (lane >= o) inc += t;
        }
        const u64 ex = base + (inc - c4);
        int first = 4;
        if (ex + c4 > r) first = (ex + c1 > r) ? 0 : (ex + c2 > r) ? 1 : (ex + c3 > r) ? 2 : 3;
        const unsigned long long hit = __ballot(first < 4);
        if (hit) {
          const int fl = __ffsll((long long)hit) - 1;
          const int fe = __shfl(first, fl, 64);
          chosen = own * G + sb * 256 + 4 * fl + fe;
        }
        base += __shfl(inc, 63, 64);
      }
    }
    if (lane == 0) out[b] = chosen >= 0 ? chosen : 0;
  }
}

__global__ void k_f32_to_bf16(const float *__restrict__ x, bf16_t *__restrict__ y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = f2bf(x[i]);
}

hipError_t launch_sample_rows(const float *logits, int batch, int V, const float *temperature,
                              const float *top_p, const float *uniform, int *out,
                              hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sample_rows, dim3(batch), dim3(kSmpThreads), 0, st, logits, V,
                     temperature, top_p, uniform, out);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float *x, void *y, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_f32_to_bf16, dim3(blocks), dim3(256), 0, st, x, (bf16_t *)y, n);
  return hipGetLastError();
}

}  // namespace bl
