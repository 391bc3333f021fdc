// Embedding gather and row LayerNorm.
//
// One 256-thread block per row.  LayerNorm statistics are float32 and two-pass
// (mean, then the biased variance of the centred values), matching the definition
// gamma * (x - mean) / sqrt(var + eps) + beta.  The residual stream is float32.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

// x[row] = E[token[row]] as float32, then optionally LayerNorm'd in place.
template <typename TP>
__global__ __launch_bounds__(256) void k_embed(const int *__restrict__ tokens,
                                               const TP *__restrict__ embed,
                                               const TP *__restrict__ g, const TP *__restrict__ b,
                                               float *__restrict__ x, int h, int vocab, int do_ln,
                                               float eps) {
  __shared__ float sh[4];
  const int row = blockIdx.x;
  int tok = tokens[row];
  tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);  // ids outside the vocabulary clamp
  const TP *e = embed + (size_t)tok * h;
  float *xr = x + (size_t)row * h;
  if (!do_ln) {
    for (int i = threadIdx.x; i < h; i += 256) xr[i] = to_f<TP>(e[i]);
    return;
  }
  float s = 0.f;
  for (int i = threadIdx.x; i < h; i += 256) s += to_f<TP>(e[i]);
  const float mean = block_sum<4>(s, sh) / (float)h;
  float ss = 0.f;
  for (int i = threadIdx.x; i < h; i += 256) {
    const float dlt = to_f<TP>(e[i]) - mean;
    ss += dlt * dlt;
  }
  const float var = block_sum<4>(ss, sh) / (float)h;
  const float rstd = 1.0f / sqrtf(var + eps);
  for (int i = threadIdx.x; i < h; i += 256)
    xr[i] = (to_f<TP>(e[i]) - mean) * rstd * to_f<TP>(g[i]) + to_f<TP>(b[i]);
}

// out[row] = LN(x[row * in_step + in_off]) in the activation type; out_f32 (nullable)
// receives the same values before rounding.
template <typename TP, typename TA>
__global__ __launch_bounds__(256) void k_layernorm(const float *__restrict__ x, int in_step,
                                                   int in_off, const TP *__restrict__ g,
                                                   const TP *__restrict__ b, TA *__restrict__ out,
                                                   float *__restrict__ out_f32, int h, float eps) {
  __shared__ float sh[4];
  const int row = blockIdx.x;
  const float *xr = x + ((size_t)row * in_step + in_off) * h;
  float s = 0.f;
  for (int i = threadIdx.x; i < h; i += 256) s += xr[i];
  const float mean = block_sum<4>(s, sh) / (float)h;
  float ss = 0.f;
  for (int i = threadIdx.x; i < h; i += 256) {
    const float dlt = xr[i] - mean;
    ss += dlt * dlt;
  }
  const float var = block_sum<4>(ss, sh) / (float)h;
  const float rstd = 1.0f / sqrtf(var + eps);
  TA *o = out + (size_t)row * h;
  float *of = out_f32 ? out_f32 + (size_t)row * h : nullptr;
  for (int i = threadIdx.x; i < h; i += 256) {
    const float y = (xr[i] - mean) * rstd * to_f<TP>(g[i]) + to_f<TP>(b[i]);
    o[i] = from_f<TA>(y);
    if (of) of[i] = y;
  }
}

hipError_t launch_embed(bool f32, const int *tokens, const void *embed, const void *g,
                        const void *b, float *x, int rows, int h, int vocab, int do_ln, float eps,
                        hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (f32)
    hipLaunchKernelGGL(k_embed<float>, dim3(rows), dim3(256), 0, stream, tokens,
                       (const float *)embed, (const float *)g, (const float *)b, x, h, vocab,
                       do_ln, eps);
  else
    hipLaunchKernelGGL(k_embed<bf16_t>, dim3(rows), dim3(256), 0, stream, tokens,
                       (const bf16_t *)embed, (const bf16_t *)g, (const bf16_t *)b, x, h, vocab,
                       do_ln, eps);
  return hipGetLastError();
}

hipError_t launch_layernorm(bool f32, const float *x, int in_step, int in_off, const void *g,
                            const void *b, void *out, float *out_f32, int rows, int h, float eps,
                            hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (f32)
    hipLaunchKernelGGL((k_layernorm<float, float>), dim3(rows), dim3(256), 0, stream, x, in_step,
                       in_off, (const float *)g, (const float *)b, (float *)out, out_f32, h, eps);
  else
    hipLaunchKernelGGL((k_layernorm<bf16_t, bf16_t>), dim3(rows), dim3(256), 0, stream, x,
                       in_step, in_off, (const bf16_t *)g, (const bf16_t *)b, (bf16_t *)out,
                       out_f32, h, eps);
  return hipGetLastError();
}

}  // namespace bl
