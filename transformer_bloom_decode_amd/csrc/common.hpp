// Device helpers shared by the gfx950 kernels: storage-type conversions, wave and
// block reductions, the ALiBi slope, the tanh GeLU, and the epilogue description
// used by every linear-layer kernel.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef _Float16 f16_t;   // IEEE binary16 (activations and KV cache in the fp16 mode)

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// fp16 <-> float32 (round to nearest even); lo / hi half of a dword
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16_t, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16_t, (uint16_t)(w >> 16));
}
__device__ __forceinline__ uint16_t f2h_bits(float f) {
  return __builtin_bit_cast(uint16_t, (f16_t)f);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }
template <> __device__ __forceinline__ float to_f<f16_t>(f16_t v) { return (float)v; }
template <> __device__ __forceinline__ float to_f<int8_t>(int8_t v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }
template <> __device__ __forceinline__ f16_t from_f<f16_t>(float v) { return (f16_t)v; }

// two bf16 packed in a dword -> floats
__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// reductions (fixed order: results are bitwise reproducible)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sum over a block of NW waves; `sh` holds NW floats.  All threads get the result.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float *sh) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += sh[i];
  __syncthreads();
  return t;
}

template <int NW>
__device__ __forceinline__ float block_max(float v, float *sh) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = v;
  __syncthreads();
  float t = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) t = fmaxf(t, sh[i]);
  __syncthreads();
  return t;
}

// ---------------------------------------------------------------------------
// model pieces
// ---------------------------------------------------------------------------

// ALiBi slope of global head g in an n_total-head model (ALiBi paper, Section 3):
// c = largest power of two <= n_total; heads g < c use 2^(-8(g+1)/c), the others the
// odd terms 2^(-4(2(g-c)+1)/c) of the 2c-head sequence.  The exponent is exact in
// fp32 (c is a power of two), so only exp2 rounds.
// Greedy choice: larger value wins, equal values go to the lower index.
__device__ __forceinline__ void argmax_take(float &bv, int &bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__device__ __forceinline__ float alibi_slope(int n_total, int g) {
  const int c = 1 << (31 - __clz(n_total));
  const float e = (g < c) ? (-8.0f * (float)(g + 1)) / (float)c
                          : (-4.0f * (float)(2 * (g - c) + 1)) / (float)c;
  return exp2f(e);
}

// tanh form of GeLU: 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3)))
__device__ __forceinline__ float gelu_tanh(float y) {
  const float k0 = 0.7978845608028654f;
  const float k1 = 0.044715f;
  return 0.5f * y * (1.0f + tanhf(k0 * (y + k1 * y * y * y)));
}

// Four parameters (gamma or beta) as loaded, unpacked only when used, so that their
// loads can be issued together with the row's and retire while the statistics run.
template <typename TP> struct Param4;
template <> struct Param4<float> {
  float4 v;
  __device__ __forceinline__ void load(const float *p) { v = *(const float4 *)p; }
  __device__ __forceinline__ float4 get() const { return v; }
};
template <> struct Param4<bf16_t> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16_t *p) { v = *(const uint2 *)p; }
  __device__ __forceinline__ float4 get() const {
    return make_float4(lo_bf(v.x), hi_bf(v.x), lo_bf(v.y), hi_bf(v.y));
  }
};

template <typename TP>
__device__ __forceinline__ float4 ln_apply(float4 x, float mean, float rstd, const Param4<TP> &g,
                                           const Param4<TP> &b) {
  const float4 gg = g.get(), bb = b.get();
  return make_float4((x.x - mean) * rstd * gg.x + bb.x, (x.y - mean) * rstd * gg.y + bb.y,
                     (x.z - mean) * rstd * gg.z + bb.z, (x.w - mean) * rstd * gg.w + bb.w);
}

// ---------------------------------------------------------------------------
// activation storage formats
// ---------------------------------------------------------------------------
// Activations (LayerNorm outputs, attention output, GeLU output) are stored in the
// form their consumer reads: bf16; float32 or fp16 (read by the vector-ALU GEMV); or a
// pair of bf16 planes hi = bf16(v), lo = bf16(v - hi) (read by the MFMA GEMM as two bf16
// operands; hi + lo carries v to within 2^-17 of its value).  The lo plane starts
// `plane` elements after the hi plane.
// The int8 activations of the W8A8 mode are quantised per row (row_quant): AF_I8 holds
// the int8 codes [rows][n] followed, `plane` bytes after the first code, by one float32
// scale per row, which the consuming linear's epilogue applies (EpiParams::xscale).
// Only kernels that own whole rows write them (the LayerNorms, k_quant_rows).
enum ActFmt : int { AF_BF16 = 0, AF_F32 = 1, AF_BF16X2 = 2, AF_F16 = 3, AF_I8 = 4 };

// Symmetric int8 quantisation of a slice whose largest magnitude is amax: scale =
// amax / 127, and the code of v is the nearest integer (ties to even) to v * (127 /
// amax), clamped to [-127, 127]; a slice of zeros has scale 0 and codes 0.  Both
// divisions are IEEE float32 divisions and the product is one float32 multiply (DeepSpeed's
// INT8 inference, "DeepSpeed Inference ...", Section VII.B, is named without its scheme;
// this is the plain symmetric per-slice form).
struct RowQuant {
  float inv, scale;
};
__device__ __forceinline__ RowQuant row_quant(float amax) {
  RowQuant q;
  q.inv = amax > 0.f ? 127.0f / amax : 0.f;
  q.scale = amax / 127.0f;
  return q;
}
__device__ __forceinline__ int quant_code(float v, float inv) {
  return (int)fminf(fmaxf(rintf(v * inv), -127.f), 127.f);
}
__device__ __forceinline__ float fabs4max(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}
// codes of elements i .. i+3 of a row quantised with q (AF_I8)
__device__ __forceinline__ void q8_store4(void *p, size_t i, float4 v, RowQuant q) {
  const int a = quant_code(v.x, q.inv), b = quant_code(v.y, q.inv);
  const int c = quant_code(v.z, q.inv), d = quant_code(v.w, q.inv);
  *(uint32_t *)((int8_t *)p + i) = (uint32_t)(a & 255) | ((uint32_t)(b & 255) << 8) |
                                   ((uint32_t)(c & 255) << 16) | ((uint32_t)(d & 255) << 24);
}
// scale of row `row` of an AF_I8 buffer whose codes take `plane` bytes
__device__ __forceinline__ float *q8_scale_ptr(void *p, size_t plane) {
  return (float *)((char *)p + plane);
}

__device__ __forceinline__ void act_store(void *p, int fmt, size_t i, size_t plane, float v) {
  if (fmt == AF_F32) {
    ((float *)p)[i] = v;
  } else if (fmt == AF_F16) {
    ((uint16_t *)p)[i] = f2h_bits(v);
  } else {
    const bf16_t hi = f2bf(v);
    ((bf16_t *)p)[i] = hi;
    if (fmt == AF_BF16X2) ((bf16_t *)p)[i + plane] = f2bf(v - bf2f(hi));
  }
}

// four consecutive elements i .. i+3 (i a multiple of 4)
__device__ __forceinline__ void act_store4(void *p, int fmt, size_t i, size_t plane, float4 v) {
  if (fmt == AF_F32) {
    *(float4 *)((float *)p + i) = v;
    return;
  }
  if (fmt == AF_F16) {
    uint2 t;
    t.x = (uint32_t)f2h_bits(v.x) | ((uint32_t)f2h_bits(v.y) << 16);
    t.y = (uint32_t)f2h_bits(v.z) | ((uint32_t)f2h_bits(v.w) << 16);
    *(uint2 *)((uint16_t *)p + i) = t;
    return;
  }
  const bf16_t h0 = f2bf(v.x), h1 = f2bf(v.y), h2 = f2bf(v.z), h3 = f2bf(v.w);
  uint2 t;
  t.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
  t.y = (uint32_t)h2 | ((uint32_t)h3 << 16);
  *(uint2 *)((bf16_t *)p + i) = t;
  if (fmt == AF_BF16X2) {
    uint2 l;
    l.x = (uint32_t)f2bf(v.x - bf2f(h0)) | ((uint32_t)f2bf(v.y - bf2f(h1)) << 16);
    l.y = (uint32_t)f2bf(v.z - bf2f(h2)) | ((uint32_t)f2bf(v.w - bf2f(h3)) << 16);
    *(uint2 *)((bf16_t *)p + i + plane) = l;
  }
}

// ---------------------------------------------------------------------------
// linear-layer epilogues
// ---------------------------------------------------------------------------
enum EpiMode : int {
  EPI_QKV = 0,     // split fused q|k|v rows: q (fp32, scaled) to a buffer, k/v to the cache
  EPI_RESID = 1,   // residual stream x[m][n] += y
  EPI_GELU = 2,    // u[m][n] = act(gelu(y))
  EPI_ARGMAX = 3,  // per-tile (max, lowest index) over n, for the LM head
  EPI_STORE = 4,   // out[m][n] = y as fp32 (used by tests of the raw product)
};

struct EpiParams {
  int mode;
  const void *bias;        // [N] parameter type, nullable
  const uint16_t *scale;   // [N] fp16 per-row scales (int8 weights), nullable
  const float *xscale;     // [M] float32 per-row scales of int8 activations, nullable
  // EPI_QKV
  float *q;                // [M][H][d]
  void *kc, *vc;           // cache of this layer: [max_batch][H][max_len][d]
  int kv_fmt;              // AF_BF16, AF_F16 or AF_F32 cache elements
  int H, d, max_len;
  int pos_base;            // absolute position of row m is pos_base + m % rows_per_seq
  const int *pos_dev;      // if set, *pos_dev replaces pos_base (replayed decode step);
                           // a slot at or past max_len is then not written
  int rows_per_seq;        // 1 (decode) or the prompt length (prefill)
  float q_scale;           // 1/sqrt(d)
  float *kv_stage;         // if set, k and v go to kv_stage[m][H][2][d] (float32) instead
                           // of the cache, for the int8 cache's quantisation kernel
  // EPI_RESID / EPI_GELU / EPI_STORE
  void *out;               // [M][ld]
  int ld;
  int out_fmt;             // EPI_GELU: ActFmt of out (AF_BF16X2: lo plane `plane` later)
  size_t plane;
  // EPI_ARGMAX
  float *am_val;           // [M][am_stride]
  int *am_idx;
  int am_stride;
  // EPI_RESID of one row with the next LayerNorm folded into its consumer: also stores
  // fold_g[n] * x[n] (ActFmt fold_fmt) to fold_u, and the kernel adds the block's sums
  // of x[n] and x[n]^2 to the accumulators fold_stats (LnStats below)
  const void *fold_g;      // [ld] the next LayerNorm's gamma (parameter type), nullable
  void *fold_u;            // [ld]
  int fold_fmt;
  unsigned long long *fold_stats;
  // consumer of a folded LayerNorm (one-row GEMV): the activations are gamma * x; mean
  // and rstd of x come from ln_stats, and the epilogue applies rstd (acc - mean c) + d
  const unsigned long long *ln_stats;   // nullable
  const float *ln_cd;      // [2][N]: c then d
  float ln_eps;
};

// Sums of a row's x and x^2 for a folded LayerNorm, added by the blocks of the GEMV that
// writes the row and read by the one that consumes it.  A block's sum goes in as one
// 64-bit fixed-point integer (the sum of x in 2^-32 units, the sum of x^2 in 2^-24
// units, each rounded once per block) with an atomic that returns nothing: integer
// additions commute, so the totals -- and every result that depends on them -- do not
// depend on the order in which the blocks arrive.  Range: |sum of x| < 2^31 and sum of
// x^2 < 2^38 per row (an RMS of 4000 over 14336 values); a block's scaled sum is
// clamped to 2^62.  Measured on MI355X, the atomics set the cost (four per block took
// twice the time of two), and the atomics of one address are served one after another
// (with 8 slots the 3584-block down projection took three times as long), so kStatSlots
// slots spread them.  Layout per LayerNorm: [kStatSlots][sum of x, sum of x^2], 1 KB.
constexpr int kStatSlots = 64;
constexpr int kStatWords = kStatSlots * 2;
constexpr int kStatFrac1 = 32, kStatFrac2 = 24;

// adds v * 2^frac, rounded to an integer, to the accumulator *a
__device__ __forceinline__ void stat_add(unsigned long long *a, double v, int frac) {
  const double t = ldexp(v, frac);
  const double c = t < 0x1p62 ? (t > -0x1p62 ? t : -0x1p62) : 0x1p62;   // (NaN -> bound)
  atomicAdd(a, (unsigned long long)(long long)rint(c));
}

// the two totals (sum of x, sum of x^2) of one LayerNorm's accumulators, a copy of which
// is in LDS: lane l takes slot l, then a wave reduction (all 64 lanes get the totals)
__device__ __forceinline__ void stat_totals_wave(const unsigned long long *lds, double &s1,
                                                 double &s2) {
  static_assert(kStatSlots == 64, "one slot per lane");
  const int lane = threadIdx.x & 63;
  long long v1 = (long long)lds[2 * lane], v2 = (long long)lds[2 * lane + 1];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    v1 += __shfl_xor(v1, o, 64);
    v2 += __shfl_xor(v2, o, 64);
  }
  s1 = ldexp((double)v1, -kStatFrac1);
  s2 = ldexp((double)v2, -kStatFrac2);
}

// The operands an epilogue loads for output (m, n): bias[n], scale[n], xscale[m], the
// residual x[m][n] (EPI_RESID) and fold_g[n] (EPI_RESID with a folded LayerNorm after
// it).  A kernel that loads them before its dot product keeps those loads off the end
// of the wave, where they would otherwise be waited for one after another.
struct EpiPre {
  float bias, scale, xscale, x, g;
};

template <typename TP>
__device__ __forceinline__ EpiPre epi_prefetch(const EpiParams &e, int m, int n) {
  EpiPre p;
  p.xscale = e.xscale ? e.xscale[m] : 1.f;
  p.scale = e.scale ? h2f(e.scale[n]) : 1.f;
  p.bias = e.bias ? to_f<TP>(((const TP *)e.bias)[n]) : 0.f;
  const bool resid = e.mode == EPI_RESID;
  p.x = resid ? ((const float *)e.out)[(size_t)m * e.ld + n] : 0.f;
  p.g = resid && e.fold_g ? to_f<TP>(((const TP *)e.fold_g)[n]) : 0.f;
  return p;
}

// y = acc * scale[n] + bias[n], then the mode's action.  TP = parameter type.  PRE: the
// operands come from epi_prefetch (p); otherwise they are loaded here, where they are
// used.  Returns the updated x[m][n] for EPI_RESID, else y.
template <typename TP, bool PRE>
__device__ __forceinline__ float epilogue_impl(const EpiParams &e, int m, int n, float acc,
                                               const EpiPre &p) {
  float y = acc;
  if (e.xscale) y *= PRE ? p.xscale : e.xscale[m];
  if (e.scale) y *= PRE ? p.scale : h2f(e.scale[n]);
  if (e.bias) y += PRE ? p.bias : to_f<TP>(((const TP *)e.bias)[n]);
  switch (e.mode) {
    case EPI_QKV: {
      const int d = e.d, H = e.H;
      const int hd = n / (3 * d);
      const int r = n - hd * 3 * d;
      const int t = r / d;
      const int c = r - t * d;
      if (t == 0) {
        e.q[((size_t)m * H + hd) * d + c] = y * e.q_scale;
      } else if (e.kv_stage) {
        e.kv_stage[(((size_t)m * H + hd) * 2 + (t - 1)) * d + c] = y;
      } else {
        const int b = m / e.rows_per_seq;
        const int pos = (e.pos_dev ? *e.pos_dev : e.pos_base) + (m - b * e.rows_per_seq);
        if (pos < e.max_len) {
          const size_t i = (((size_t)b * H + hd) * e.max_len + pos) * d + c;
          void *cache = t == 1 ? e.kc : e.vc;
          if (e.kv_fmt == AF_F32) ((float *)cache)[i] = y;
          else if (e.kv_fmt == AF_F16) ((uint16_t *)cache)[i] = f2h_bits(y);
          else ((bf16_t *)cache)[i] = f2bf(y);
        }
      }
      break;
    }
    case EPI_RESID: {
      float *x = (float *)e.out + (size_t)m * e.ld + n;
      const float xn = (PRE ? p.x : *x) + y;
      *x = xn;
      if (e.fold_g)
        act_store(e.fold_u, e.fold_fmt, (size_t)m * e.ld + n, 0,
                  (PRE ? p.g : to_f<TP>(((const TP *)e.fold_g)[n])) * xn);
      return xn;
    }
    case EPI_GELU:
      act_store(e.out, e.out_fmt, (size_t)m * e.ld + n, e.plane, gelu_tanh(y));
      break;
    case EPI_STORE:
      ((float *)e.out)[(size_t)m * e.ld + n] = y;
      break;
    default:
      break;
  }
  return y;
}

template <typename TP>
__device__ __forceinline__ float epilogue_pre(const EpiParams &e, int m, int n, float acc,
                                              const EpiPre &p) {
  return epilogue_impl<TP, true>(e, m, n, acc, p);
}

// the epilogue with its operands loaded where it runs.  TP = parameter type.
template <typename TP>
__device__ __forceinline__ float epilogue(const EpiParams &e, int m, int n, float acc) {
  return epilogue_impl<TP, false>(e, m, n, acc, EpiPre{});
}

}  // namespace bl
