// Embedding gather and row LayerNorm.
//
// One block per row.  A row of up to kLnThreads * 4 * kLnVec floats is held in
// registers (float4 pieces), so the row is read from memory once: the mean is a
// block sum of the registers, the biased variance a second block sum of the centred
// registers (two-pass, float32), then gamma * (x - mean) / sqrt(var + eps) + beta is
// written.  Longer rows fall back to re-reading the row.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

constexpr int kLnThreads = 1024;
constexpr int kLnWaves = kLnThreads / 64;
constexpr int kLnVec = 4;   // float4 pieces per thread: rows up to 16384

template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ float4 load(const float *p) { return *(const float4 *)p; }
  static __device__ __forceinline__ void store(float *p, float4 v) { *(float4 *)p = v; }
};
template <> struct Vec4<bf16_t> {
  static __device__ __forceinline__ float4 load(const bf16_t *p) {
    const uint2 t = *(const uint2 *)p;
    return make_float4(lo_bf(t.x), hi_bf(t.x), lo_bf(t.y), hi_bf(t.y));
  }
  static __device__ __forceinline__ void store(bf16_t *p, float4 v) {
    uint2 t;
    t.x = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
    t.y = (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16);
    *(uint2 *)p = t;
  }
};

__device__ __forceinline__ float sum4(float4 v) { return (v.x + v.y) + (v.z + v.w); }

// Normalise the register-held row piece v[] (columns 4*(threadIdx.x + i*kLnThreads)).
// Returns mean and rstd; `h` is the row length (a multiple of 4).
__device__ __forceinline__ void ln_stats(const float4 (&v)[kLnVec], int h, float eps, float *sh,
                                         float &mean, float &rstd) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kLnVec; ++i)
    if (4 * (threadIdx.x + i * kLnThreads) < h) s += sum4(v[i]);
  mean = block_sum<kLnWaves>(s, sh) / (float)h;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kLnVec; ++i)
    if (4 * (threadIdx.x + i * kLnThreads) < h) {
      const float a = v[i].x - mean, b = v[i].y - mean, c = v[i].z - mean, d = v[i].w - mean;
      ss += (a * a + b * b) + (c * c + d * d);
    }
  const float var = block_sum<kLnWaves>(ss, sh) / (float)h;
  rstd = 1.0f / sqrtf(var + eps);
}

// Write the register-held row y[] (columns 4 (threadIdx.x + i kLnThreads) < h) in
// format fmt.  The int8 formats quantise the whole row with one scale (row_quant of the
// row's largest magnitude, a block reduction in `sh`); AF_I8 stores that scale `plane`
// bytes after the first code.
__device__ __forceinline__ void ln_store_row(const float4 (&y)[kLnVec], void *out, int fmt,
                                             size_t plane, int row, int h, float *sh) {
  if (fmt == AF_I8) {
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < kLnVec; ++i)
      if (4 * (threadIdx.x + i * kLnThreads) < h) am = fmaxf(am, fabs4max(y[i]));
    const RowQuant rq = row_quant(block_max<kLnWaves>(am, sh));
#pragma unroll
    for (int i = 0; i < kLnVec; ++i) {
      const int col = 4 * (threadIdx.x + i * kLnThreads);
      if (col < h) q8_store4(out, (size_t)row * h + col, y[i], rq);
    }
    if (threadIdx.x == 0) q8_scale_ptr(out, plane)[row] = rq.scale;
    return;
  }
#pragma unroll
  for (int i = 0; i < kLnVec; ++i) {
    const int col = 4 * (threadIdx.x + i * kLnThreads);
    if (col < h) act_store4(out, fmt, (size_t)row * h + col, plane, y[i]);
  }
}

// Block z of the clearing blocks zeroes words [z kZeroBlockWords, (z + 1) kZeroBlockWords)
// of zero[nzero] with 16-byte stores (nzero even, zero 16-byte aligned).
constexpr int kZeroBlockWords = 8192;
__device__ __forceinline__ void zero_words(unsigned long long *zero, int nzero, int z,
                                           int nthreads) {
  const int end = min(nzero, (z + 1) * kZeroBlockWords);
  for (int i = z * kZeroBlockWords + 2 * (int)threadIdx.x; i < end; i += 2 * nthreads)
    *(uint4 *)(zero + i) = make_uint4(0u, 0u, 0u, 0u);
}

// x[row] = E[token[row]] as float32, then optionally LayerNorm'd.  With nzero > 0 the
// grid has ceil(nzero / kZeroBlockWords) more blocks, which only clear zero[].
template <typename TP>
__global__ __launch_bounds__(kLnThreads) void k_embed(const int *__restrict__ tokens,
                                                      const TP *__restrict__ embed,
                                                      const TP *__restrict__ g,
                                                      const TP *__restrict__ b,
                                                      float *__restrict__ x, int h, int vocab,
                                                      int do_ln, float eps,
                                                      int rows,
                                                      unsigned long long *__restrict__ zero,
                                                      int nzero) {
  __shared__ float sh[kLnWaves];
  const int row = blockIdx.x;
  if (row >= rows) {   // the blocks past the rows clear the folded-LayerNorm accumulators
    zero_words(zero, nzero, row - rows, kLnThreads);
    return;
  }
  int tok = tokens[row];
  tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);  // ids outside the vocabulary clamp
  const TP *e = embed + (size_t)tok * h;
  float *xr = x + (size_t)row * h;
  float4 v[kLnVec];
  Param4<TP> gv[kLnVec], bv[kLnVec];
#pragma unroll
  for (int i = 0; i < kLnVec; ++i) {
    const int col = 4 * (threadIdx.x + i * kLnThreads);
    v[i] = col < h ? Vec4<TP>::load(e + col) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (do_ln) {
#pragma unroll
    for (int i = 0; i < kLnVec; ++i) {
      const int col = min(4 * (threadIdx.x + i * kLnThreads), h - 4);
      gv[i].load(g + col);
      bv[i].load(b + col);
    }
  }
  float mean = 0.f, rstd = 1.f;
  if (do_ln) ln_stats(v, h, eps, sh, mean, rstd);
#pragma unroll
  for (int i = 0; i < kLnVec; ++i) {
    const int col = 4 * (threadIdx.x + i * kLnThreads);
    if (col < h) Vec4<float>::store(xr + col, do_ln ? ln_apply<TP>(v[i], mean, rstd, gv[i], bv[i]) : v[i]);
  }
}

// out[row] = LN(x[row * in_step + in_off]) in the activation format `fmt` (ActFmt; a
// second bf16 plane `plane` elements later for AF_BF16X2); out_f32 (nullable) receives
// the same values before rounding.
template <typename TP>
__global__ __launch_bounds__(kLnThreads) void k_layernorm(const float *__restrict__ x,
                                                          int in_step, int in_off,
                                                          const TP *__restrict__ g,
                                                          const TP *__restrict__ b,
                                                          void *__restrict__ out, int fmt,
                                                          size_t plane,
                                                          float *__restrict__ out_f32, int h,
                                                          float eps) {
  __shared__ float sh[kLnWaves];
  const int row = blockIdx.x;
  const float *xr = x + ((size_t)row * in_step + in_off) * h;
  float4 v[kLnVec];
  Param4<TP> gv[kLnVec], bv[kLnVec];
#pragma unroll
  for (int i = 0; i < kLnVec; ++i) {
    const int col = 4 * (threadIdx.x + i * kLnThreads);
    v[i] = col < h ? Vec4<float>::load(xr + col) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < kLnVec; ++i) {
    const int col = min(4 * (threadIdx.x + i * kLnThreads), h - 4);  // in bounds; unused past h
    gv[i].load(g + col);
    bv[i].load(b + col);
  }
  float mean, rstd;
  ln_stats(v, h, eps, sh, mean, rstd);
  float *of = out_f32 ? out_f32 + (size_t)row * h : nullptr;
#pragma unroll
  for (int i = 0; i < kLnVec; ++i) {
    const int col = 4 * (threadIdx.x + i * kLnThreads);
    if (col < h) {
      v[i] = ln_apply<TP>(v[i], mean, rstd, gv[i], bv[i]);
      if (of) Vec4<float>::store(of + col, v[i]);
    }
  }
  ln_store_row(v, out, fmt, plane, row, h, sh);
}

// Residual + LayerNorm epilogue of a K-split linear ("DeepSpeed Inference ...", Section
// III.D: bias with residual addition, then the next layer-norm): for each column n of
// the row, y = (sum over the S partials in split order) * scale[n] + bias[n] and x += y
// -- the same float32 operations, in the same order, as k_splitk_epilogue in residual
// mode -- then out = LN(x) of the updated row, as k_layernorm.  All S partial pieces of a
// column group are loaded before the first add.
template <typename TP, int S>
__global__ __launch_bounds__(kLnThreads) void k_splitk_resid_ln(
    const float *__restrict__ partial, int M, const float *__restrict__ xscale,
    const uint16_t *__restrict__ scale, const TP *__restrict__ bias, float *__restrict__ x,
    const TP *__restrict__ g, const TP *__restrict__ b, void *__restrict__ out, int fmt,
    size_t plane, int h, float eps) {
  __shared__ float sh[kLnWaves];
  const int row = blockIdx.x;
  const size_t MN = (size_t)M * h;
  float *xr = x + (size_t)row * h;
  const float *pr = partial + (size_t)row * h;
  const float xs = xscale ? xscale[row] : 1.f;   // int8 activations: the row's scale
  float4 v[kLnVec];
  Param4<TP> gv[kLnVec], bv[kLnVec];
#pragma unroll
  for (int i = 0; i < kLnVec; ++i) {
    const int col = 4 * (threadIdx.x + i * kLnThreads);
    if (col >= h) {
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      continue;
    }
    float4 pz[S];
#pragma unroll
    for (int z = 0; z < S; ++z) pz[z] = *(const float4 *)(pr + z * MN + col);
    const float4 x0 = *(const float4 *)(xr + col);
    float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int z = 0; z < S; ++z) {
      y.x += pz[z].x; y.y += pz[z].y; y.z += pz[z].z; y.w += pz[z].w;
    }
    if (xscale) {
      y.x *= xs; y.y *= xs; y.z *= xs; y.w *= xs;
    }
    if (scale) {
      y.x *= h2f(scale[col]); y.y *= h2f(scale[col + 1]);
      y.z *= h2f(scale[col + 2]); y.w *= h2f(scale[col + 3]);
    }
    if (bias) {
      y.x += to_f<TP>(bias[col]); y.y += to_f<TP>(bias[col + 1]);
      y.z += to_f<TP>(bias[col + 2]); y.w += to_f<TP>(bias[col + 3]);
    }
    v[i] = make_float4(x0.x + y.x, x0.y + y.y, x0.z + y.z, x0.w + y.w);
    Vec4<float>::store(xr + col, v[i]);
  }
#pragma unroll
  for (int i = 0; i < kLnVec; ++i) {
    const int col = min(4 * (threadIdx.x + i * kLnThreads), h - 4);
    gv[i].load(g + col);
    bv[i].load(b + col);
  }
  float mean, rstd;
  ln_stats(v, h, eps, sh, mean, rstd);
#pragma unroll
  for (int i = 0; i < kLnVec; ++i)
    if (4 * (threadIdx.x + i * kLnThreads) < h) v[i] = ln_apply<TP>(v[i], mean, rstd, gv[i], bv[i]);
  ln_store_row(v, out, fmt, plane, row, h, sh);
}

// Per-row int8 quantisation of float32 rows in[rows][K] (K a multiple of 4) into AF_I8
// (codes, then the rows' scales `plane` bytes after the first code): the attention and
// GeLU outputs of the W8A8 mode, whose rows several blocks produce.  One block per row: the row's largest magnitude, then a
// second pass (from cache) writes the codes.
constexpr int kQuantThreads = 1024;
__global__ __launch_bounds__(kQuantThreads) void k_quant_rows(const float *__restrict__ in, int K,
                                                              void *__restrict__ out,
                                                              size_t plane) {
  __shared__ float sh[kQuantThreads / 64];
  const int row = blockIdx.x;
  const float *r = in + (size_t)row * K;
  float am = 0.f;
  for (int c = 4 * threadIdx.x; c < K; c += 4 * kQuantThreads)
    am = fmaxf(am, fabs4max(*(const float4 *)(r + c)));
  const RowQuant rq = row_quant(block_max<kQuantThreads / 64>(am, sh));
  for (int c = 4 * threadIdx.x; c < K; c += 4 * kQuantThreads)
    q8_store4(out, (size_t)row * K + c, *(const float4 *)(r + c), rq);
  if (threadIdx.x == 0) q8_scale_ptr(out, plane)[row] = rq.scale;
}

hipError_t launch_quant_rows(const float *in, int rows, int K, void *out, int fmt,
                             hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (fmt != AF_I8 || K % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_quant_rows, dim3(rows), dim3(kQuantThreads), 0, stream, in, K, out,
                     (size_t)rows * K);
  return hipGetLastError();
}

// Rows longer than the register tile, or not a multiple of 4: re-read the row.
template <typename TP>
__global__ __launch_bounds__(256) void k_layernorm_any(const float *__restrict__ x, int in_step,
                                                       int in_off, const TP *__restrict__ g,
                                                       const TP *__restrict__ b,
                                                       void *__restrict__ out, int fmt,
                                                       size_t plane,
                                                       float *__restrict__ out_f32, int h,
                                                       float eps) {
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
  float *of = out_f32 ? out_f32 + (size_t)row * h : nullptr;
  for (int i = threadIdx.x; i < h; i += 256) {
    const float y = (xr[i] - mean) * rstd * to_f<TP>(g[i]) + to_f<TP>(b[i]);
    act_store(out, fmt, (size_t)row * h + i, plane, y);
    if (of) of[i] = y;
  }
}

template <typename TP>
__global__ __launch_bounds__(256) void k_embed_any(const int *__restrict__ tokens,
                                                   const TP *__restrict__ embed,
                                                   const TP *__restrict__ g,
                                                   const TP *__restrict__ b,
                                                   float *__restrict__ x, int h, int vocab,
                                                   int do_ln, float eps,
                                                   int rows,
                                                   unsigned long long *__restrict__ zero,
                                                   int nzero) {
  __shared__ float sh[4];
  const int row = blockIdx.x;
  if (row >= rows) {   // the blocks past the rows clear the folded-LayerNorm accumulators
    zero_words(zero, nzero, row - rows, 256);
    return;
  }
  int tok = tokens[row];
  tok = tok < 0 ? 0 : (tok >= vocab ? vocab - 1 : tok);
  const TP *e = embed + (size_t)tok * h;
  float *xr = x + (size_t)row * h;
  float mean = 0.f, rstd = 1.f;
  if (do_ln) {
    float s = 0.f;
    for (int i = threadIdx.x; i < h; i += 256) s += to_f<TP>(e[i]);
    mean = block_sum<4>(s, sh) / (float)h;
    float ss = 0.f;
    for (int i = threadIdx.x; i < h; i += 256) {
      const float dlt = to_f<TP>(e[i]) - mean;
      ss += dlt * dlt;
    }
    rstd = 1.0f / sqrtf(block_sum<4>(ss, sh) / (float)h + eps);
  }
  for (int i = threadIdx.x; i < h; i += 256) {
    const float v = to_f<TP>(e[i]);
    xr[i] = do_ln ? (v - mean) * rstd * to_f<TP>(g[i]) + to_f<TP>(b[i]) : v;
  }
}

static bool fits_regs(int h) { return h % 4 == 0 && h <= kLnThreads * 4 * kLnVec; }

hipError_t launch_embed(bool f32, const int *tokens, const void *embed, const void *g,
                        const void *b, float *x, int rows, int h, int vocab, int do_ln, float eps,
                        unsigned long long *zero, int nzero, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (nzero < 0 || nzero % 2 || ((uintptr_t)zero & 15)) return hipErrorInvalidValue;
  const bool reg = fits_regs(h);
  const unsigned grid =
      (unsigned)rows + (unsigned)((nzero + kZeroBlockWords - 1) / kZeroBlockWords);
  if (f32) {
    if (reg)
      hipLaunchKernelGGL(k_embed<float>, dim3(grid), dim3(kLnThreads), 0, stream, tokens,
                         (const float *)embed, (const float *)g, (const float *)b, x, h, vocab,
                         do_ln, eps, rows, zero, nzero);
    else
      hipLaunchKernelGGL(k_embed_any<float>, dim3(grid), dim3(256), 0, stream, tokens,
                         (const float *)embed, (const float *)g, (const float *)b, x, h, vocab,
                         do_ln, eps, rows, zero, nzero);
  } else {
    if (reg)
      hipLaunchKernelGGL(k_embed<bf16_t>, dim3(grid), dim3(kLnThreads), 0, stream, tokens,
                         (const bf16_t *)embed, (const bf16_t *)g, (const bf16_t *)b, x, h,
                         vocab, do_ln, eps, rows, zero, nzero);
    else
      hipLaunchKernelGGL(k_embed_any<bf16_t>, dim3(grid), dim3(256), 0, stream, tokens,
                         (const bf16_t *)embed, (const bf16_t *)g, (const bf16_t *)b, x, h,
                         vocab, do_ln, eps, rows, zero, nzero);
  }
  return hipGetLastError();
}

bool splitk_resid_ln_supported(int h, int splits) {
  return fits_regs(h) && splits >= 2 && splits <= 8;
}

hipError_t launch_splitk_resid_ln(const float *partial, int splits, int rows, const float *xscale,
                                  const void *scale, const void *bias, float *x, const void *g,
                                  const void *b, void *out, int fmt, int h, float eps,
                                  hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (!splitk_resid_ln_supported(h, splits)) return hipErrorInvalidValue;
  const dim3 grid(rows), block(kLnThreads);
  const uint16_t *sc = (const uint16_t *)scale;
  const bf16_t *bi = (const bf16_t *)bias, *gg = (const bf16_t *)g, *bb = (const bf16_t *)b;
  const size_t plane = (size_t)rows * h;
#define BL_SRL(S)                                                                          \
  case S:                                                                                  \
    hipLaunchKernelGGL((k_splitk_resid_ln<bf16_t, S>), grid, block, 0, stream, partial,   \
                       rows, xscale, sc, bi, x, gg, bb, out, fmt, plane, h, eps);           \
    break;
  switch (splits) {
    BL_SRL(2) BL_SRL(3) BL_SRL(4) BL_SRL(5) BL_SRL(6) BL_SRL(7) BL_SRL(8)
    default: return hipErrorInvalidValue;
  }
#undef BL_SRL
  return hipGetLastError();
}

hipError_t launch_layernorm(bool f32, const float *x, int in_step, int in_off, const void *g,
                            const void *b, void *out, int fmt, float *out_f32, int rows, int h,
                            float eps, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const bool reg = fits_regs(h);
  const size_t plane = (size_t)rows * h;
  if (fmt == AF_I8 && !reg) return hipErrorInvalidValue;
  if (f32) {
    if (reg)
      hipLaunchKernelGGL((k_layernorm<float>), dim3(rows), dim3(kLnThreads), 0, stream, x,
                         in_step, in_off, (const float *)g, (const float *)b, out, fmt, plane,
                         out_f32, h, eps);
    else
      hipLaunchKernelGGL((k_layernorm_any<float>), dim3(rows), dim3(256), 0, stream, x,
                         in_step, in_off, (const float *)g, (const float *)b, out, fmt, plane,
                         out_f32, h, eps);
  } else {
    if (reg)
      hipLaunchKernelGGL((k_layernorm<bf16_t>), dim3(rows), dim3(kLnThreads), 0, stream, x,
                         in_step, in_off, (const bf16_t *)g, (const bf16_t *)b, out, fmt, plane,
                         out_f32, h, eps);
    else
      hipLaunchKernelGGL((k_layernorm_any<bf16_t>), dim3(rows), dim3(256), 0, stream, x,
                         in_step, in_off, (const bf16_t *)g, (const bf16_t *)b, out, fmt, plane,
                         out_f32, h, eps);
  }
  return hipGetLastError();
}

}  // namespace bl
