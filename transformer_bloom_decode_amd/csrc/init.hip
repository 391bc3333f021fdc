// Seeded synthetic weights written on the GPU: the counter-hash generator of the
// library's weight specification (bloom.h, bloom_init_weights), so a model of any size
// is filled in place without a host copy.  Every value is a pure function of (seed,
// tensor id, flat index):
//   hash    r = SplitMix64 finaliser of (key + index), key = SplitMix64 finaliser of
//           (seed << 32 xor tensor id) (Steele, Lea and Flood, "Fast splittable
//           pseudorandom number generators", OOPSLA 2014);
//   normal  z = (sum of the four 16-bit fields of r) - 131070, exact; value =
//           mean + float32(z) * scale, each step one IEEE float32 round-to-nearest-even
//           operation (no fused multiply-add), then rounded to bf16 (nearest even) for
//           bf16 storage;
//   int8    r mod 255 - 127;
//   scale   fp16 of scale * (0.5 + (r >> 40) * 2^-24), float32 arithmetic, rounded to
//           the nearest fp16 (ties to even, subnormals kept).
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

__device__ __forceinline__ uint64_t splitmix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// IEEE binary16 bits of f, round to nearest even, subnormals kept, overflow to inf.
__device__ __forceinline__ uint16_t f16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);
  if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);
  if (a < 0x38800000u) {
    if (a < 0x33000000u) return (uint16_t)sign;
    const uint32_t mant = (a & 0x7fffffu) | 0x800000u;
    const int shift = 126 - (int)(a >> 23);
    uint32_t half = mant >> shift;
    const uint32_t rem = mant & ((1u << shift) - 1u), mid = 1u << (shift - 1);
    if (rem > mid || (rem == mid && (half & 1u))) half++;
    return (uint16_t)(sign | half);
  }
  const uint32_t r = a + 0x0fffu + ((a >> 13) & 1u) - 0x38000000u;
  return (uint16_t)(sign | (r >> 13));
}

__global__ __launch_bounds__(256) void k_init_tensor(InitTensor t) {
  // each product and sum below is one IEEE float32 operation: no fused multiply-add
#pragma clang fp contract(off)
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < t.n; i += (size_t)gridDim.x * 256) {
    const uint64_t r = splitmix64(t.key + i);
    if (t.op == 0) {
      const int32_t s = (int32_t)(r & 0xffffu) + (int32_t)((r >> 16) & 0xffffu) +
                        (int32_t)((r >> 32) & 0xffffu) + (int32_t)(r >> 48);
      float v = (float)(s - 131070) * t.scale;
      if (t.mean != 0.f) v = t.mean + v;
      if (t.kind == 0) ((float *)t.out)[i] = v;
      else ((bf16_t *)t.out)[i] = f2bf(v);
    } else if (t.op == 1) {
      // r mod 255 from the byte sum (2^8 = 1 mod 255)
      uint32_t bsum = 0;
#pragma unroll
      for (int b = 0; b < 8; ++b) bsum += (uint32_t)((r >> (8 * b)) & 0xffu);
      ((int8_t *)t.out)[i] = (int8_t)((int)(bsum % 255u) - 127);
    } else {
      const float u = (float)(r >> 40) * 5.9604644775390625e-8f;
      const float half_plus = 0.5f + u;
      ((uint16_t *)t.out)[i] = f16_bits(t.scale * half_plus);
    }
  }
}

hipError_t launch_init_tensor(const InitTensor &t, hipStream_t st) {
  if (t.n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((t.n + 255) / 256, 16384);
  hipLaunchKernelGGL(k_init_tensor, dim3(blocks), dim3(256), 0, st, t);
  return hipGetLastError();
}

}  // namespace bl
