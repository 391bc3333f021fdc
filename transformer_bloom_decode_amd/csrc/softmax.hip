// Fused ALiBi bias + left-pad / causal masking + float32 softmax over one score row
// per wavefront.  ("Hugging Face BLOOM Inference Optimization": Custom CUDA Kernels
// and Hardware Acceleration -- masked_fill then a float32 softmax with only the
// reductions upcast; Efficient PyTorch Implementation -- ALiBi computed in one place.)
//
// Each 64-lane wave owns one (b, h, i) row.  Lanes hold 4 consecutive keys per
// 256-key chunk, so loads and stores are contiguous per wave.  For rows of up to
// kRegChunks*256 keys the biased scores stay in registers between the max, exp-sum
// and normalise passes; longer rows re-read the scores.  The ALiBi bias is taken
// relative to the query position, slope * (j - qpos) <= 0, which differs from the
// pad-relative form by a per-row constant and so gives the same softmax while
// keeping the biased scores small.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kRegChunks = 8;  // 8 * 256 = 2048 keys held in registers

template <typename TIn> struct Vec4In;
template <> struct Vec4In<float> {
  static __device__ __forceinline__ void load(const float *p, float v[4]) {
    const float4 t = *(const float4 *)p;
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
  }
};
template <> struct Vec4In<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t *p, float v[4]) {
    const uint2 t = *(const uint2 *)p;
    v[0] = lo_bf(t.x); v[1] = hi_bf(t.x); v[2] = lo_bf(t.y); v[3] = hi_bf(t.y);
  }
};

template <typename TOut> struct Vec4Out;
template <> struct Vec4Out<float> {
  static __device__ __forceinline__ void store(float *p, const float v[4]) {
    *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Vec4Out<bf16_t> {
  static __device__ __forceinline__ void store(bf16_t *p, const float v[4]) {
    uint2 t;
    t.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    t.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *(uint2 *)p = t;
  }
};

struct RowInfo {
  long row;
  int first, last, qpos;
  float slope;
};

__device__ __forceinline__ RowInfo row_info(long row, const int *valid_len, int H, int Q, int K,
                                            int n_total, int head_off) {
  RowInfo r;
  r.row = row;
  const int i = (int)(row % Q);
  const int h = (int)((row / Q) % H);
  const int b = (int)(row / ((long)Q * H));
  int vl = valid_len[b];
  vl = vl < 0 ? 0 : (vl > K ? K : vl);
  r.first = K - vl;
  r.qpos = K - Q + i;
  r.last = r.qpos;
  r.slope = alibi_slope(n_total, head_off + h);
  return r;
}

// Rows whose length is a multiple of 4 and at most kRegChunks * 256.
template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void k_alibi_softmax_reg(const TIn *__restrict__ scores,
                                                           const int *__restrict__ valid_len,
                                                           TOut *__restrict__ probs, int B, int H,
                                                           int Q, int K, int n_total, int head_off) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)B * H * Q) return;
  const RowInfo r = row_info(row, valid_len, H, Q, K, n_total, head_off);
  const TIn *s = scores + row * (long)K;
  TOut *p = probs + row * (long)K;

  float v[kRegChunks][4];
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int j0 = c * 256 + lane * 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) v[c][t] = -INFINITY;
    if (j0 < K && j0 + 3 >= r.first && j0 <= r.last) {
      float raw[4];
      Vec4In<TIn>::load(s + j0, raw);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = j0 + t;
        if (j >= r.first && j <= r.last) {
          v[c][t] = raw[t] + r.slope * (float)(j - r.qpos);
          mx = fmaxf(mx, v[c][t]);
        }
      }
    }
  }
  mx = wave_max(mx);
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float e = (v[c][t] == -INFINITY) ? 0.f : __expf(v[c][t] - mx);
      v[c][t] = e;
      sum += e;
    }
  sum = wave_sum(sum);
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
#pragma unroll
  for (int c = 0; c < kRegChunks; ++c) {
    const int j0 = c * 256 + lane * 4;
    if (j0 < K) {
      float o[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = v[c][t] * inv;
      Vec4Out<TOut>::store(p + j0, o);
    }
  }
}

// Any row length: three passes over the scores (max, sum, write).
template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void k_alibi_softmax_any(const TIn *__restrict__ scores,
                                                           const int *__restrict__ valid_len,
                                                           TOut *__restrict__ probs, int B, int H,
                                                           int Q, int K, int n_total, int head_off) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)B * H * Q) return;
  const RowInfo r = row_info(row, valid_len, H, Q, K, n_total, head_off);
  const TIn *s = scores + row * (long)K;
  TOut *p = probs + row * (long)K;
  float mx = -INFINITY;
  for (int j = r.first + lane; j <= r.last; j += 64)
    mx = fmaxf(mx, to_f<TIn>(s[j]) + r.slope * (float)(j - r.qpos));
  mx = wave_max(mx);
  float sum = 0.f;
  for (int j = r.first + lane; j <= r.last; j += 64)
    sum += __expf(to_f<TIn>(s[j]) + r.slope * (float)(j - r.qpos) - mx);
  sum = wave_sum(sum);
  const float inv = sum > 0.f ? 1.0f / sum : 0.f;
  for (int j = lane; j < K; j += 64) {
    float o = 0.f;
    if (j >= r.first && j <= r.last)
      o = __expf(to_f<TIn>(s[j]) + r.slope * (float)(j - r.qpos) - mx) * inv;
    p[j] = from_f<TOut>(o);
  }
}

template <typename TIn, typename TOut>
static hipError_t launch_softmax_t(const void *scores, const int *valid_len, void *probs, int B,
                                   int H, int Q, int K, int n_total, int head_off,
                                   hipStream_t stream) {
  const long rows = (long)B * H * Q;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  const bool aligned = ((uintptr_t)scores % 16 == 0) && ((uintptr_t)probs % 16 == 0);
  if (aligned && K % 4 == 0 && K <= kRegChunks * 256) {
    hipLaunchKernelGGL((k_alibi_softmax_reg<TIn, TOut>), grid, block, 0, stream,
                       (const TIn *)scores, valid_len, (TOut *)probs, B, H, Q, K, n_total,
                       head_off);
  } else {
    hipLaunchKernelGGL((k_alibi_softmax_any<TIn, TOut>), grid, block, 0, stream,
                       (const TIn *)scores, valid_len, (TOut *)probs, B, H, Q, K, n_total,
                       head_off);
  }
  return hipGetLastError();
}

hipError_t launch_alibi_softmax(const void *scores, bool in_bf16, const int *valid_len,
                                void *probs, bool out_bf16, int B, int H, int Q, int K,
                                int n_total, int head_off, hipStream_t stream) {
  if (in_bf16 && out_bf16)
    return launch_softmax_t<bf16_t, bf16_t>(scores, valid_len, probs, B, H, Q, K, n_total, head_off, stream);
  if (in_bf16)
    return launch_softmax_t<bf16_t, float>(scores, valid_len, probs, B, H, Q, K, n_total, head_off, stream);
  if (out_bf16)
    return launch_softmax_t<float, bf16_t>(scores, valid_len, probs, B, H, Q, K, n_total, head_off, stream);
  return launch_softmax_t<float, float>(scores, valid_len, probs, B, H, Q, K, n_total, head_off, stream);
}

}  // namespace bl
