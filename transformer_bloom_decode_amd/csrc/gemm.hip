// Linear layers y = x W^T (+ scale, bias, epilogue) for the decoder layer and the
// LM head.
//
// The pages' analysis ("DeepSpeed Inference ...", Section III.A) is that small-batch
// inference is bound by reading the weights, so the decode kernel is built around
// streaming W once at full bandwidth; Section III.C (SBI-GeMM) tiles the output
// dimension across blocks and splits the input dimension when there are too few
// output tiles; Section III.D fuses bias, GeLU, residual and the QKV split into the
// GEMM.  Here, on gfx950:
//
//  * k_gemv_valu (up to 4 activation rows, the batch-1..4 decode step), in gemv.hip.
//  * k_gemm_lg (5+ rows: decode batches, LM heads, prompt passes): MFMA 32x32x16 with
//    both operands copied straight from global memory into LDS (global_load_lds), tile
//    sizes and K splits chosen per shape (plan_linear); int8 weights widened from LDS,
//    or, with int8 activations (W8A8), both operands int8 on the 32x32x32 int8 MFMA.
//  * k_gemm_f32: a plain float32 path for the fp32 model.
//
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

thread_local LaunchEvents g_launch_events;

// two signed bytes of w (selected by the byte offset) -> two bf16 in one dword (exact)
__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int byte0) {
  const float f0 = (float)(int)(int8_t)(w >> (8 * byte0));
  const float f1 = (float)(int)(int8_t)(w >> (8 * byte0 + 8));
  return (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
}

__device__ __forceinline__ u32x4 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return u32x4{i8x2_to_bf16x2(lo, 0), i8x2_to_bf16x2(lo, 2), i8x2_to_bf16x2(hi, 0),
               i8x2_to_bf16x2(hi, 2)};
}

// fp16 operands (fp16 activations): two floats -> two fp16 in one dword, a in the low
// half (nearest even, one packed conversion instruction)
__device__ __forceinline__ uint32_t f2x_f16(float a, float b) {
  typedef f16_t h2v __attribute__((ext_vector_type(2)));
  typedef float f2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, h2v));
}
// eight int8 -> fp16 (exact)
__device__ __forceinline__ u32x4 i8x8_to_f16x8(uint32_t lo, uint32_t hi) {
  u32x4 r;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t w = t < 2 ? lo : hi;
    const int b0 = 16 * (t & 1);
    r[t] = f2x_f16((float)(int)(int8_t)(w >> b0), (float)(int)(int8_t)(w >> (b0 + 8)));
  }
  return r;
}
// eight bf16 -> fp16: exact for magnitudes from 2^-14 to 65504 (bf16's 8-bit significand
// fits fp16's 11 bits); smaller ones round to fp16's subnormal grid of 2^-24
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
  return u32x4{f2x_f16(lo_bf(w[0]), hi_bf(w[0])), f2x_f16(lo_bf(w[1]), hi_bf(w[1])),
               f2x_f16(lo_bf(w[2]), hi_bf(w[2])), f2x_f16(lo_bf(w[3]), hi_bf(w[3]))};
}


// ---------------------------------------------------------------------------
// Prompt-pass GEMM on MFMA 32x32x16 with LDS staged by direct-to-LDS loads
// ---------------------------------------------------------------------------
// Y = X . W^T for 5+ rows, bf16 or int8 weights.  A block owns a BM x BN output tile and
// WGM x WGN waves, each a (BM/WGM) x (BN/WGN) tile of 32x32 MFMA blocks with float32
// accumulators.  K advances in 64-wide tiles through two LDS stages: each wave copies
// 1 KB pieces (8 rows x 128 bytes; int8 W: 16 rows x 64 bytes) of the X and W tiles
// straight from global memory into LDS (global_load_lds_dwordx4, no register staging),
// S - 1 tiles ahead of the MFMAs.  int8 weights are widened to bf16 (exactly) as they
// are read from LDS and scaled per row in the epilogue.
// Inside a row the eight 16-byte k-pieces sit at slot piece ^ ((row >> 1) & 7), which
// makes the MFMA operand reads (32 rows x 16 bytes per half-wave) free of LDS bank
// conflicts (measured with the LDS bank-conflict counter on MI355X).  Blocks are
// numbered so that the blocks one XCD runs take consecutive tiles (M fastest): the W
// tile they share stays in that XCD's L2.  With split-K the block writes float32
// partials and k_splitk_epilogue sums them in a fixed order.
constexpr int kLg = 64;          // K tile

// s_waitcnt vmcnt(V), expcnt and lgkmcnt left unconstrained
template <int V> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(V >= 0 && V < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((V & 15) | ((V >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most J * CPW loads of this wave are outstanding, for the largest J <=
// `after` (J <= JMAX): the copies of every K tile issued before the last `after` have
// landed.
template <int CPW, int JMAX> __device__ __forceinline__ void lg_wait(int after) {
  if constexpr (JMAX <= 0) {
    wait_vmcnt<0>();
  } else {
    if (after >= JMAX) wait_vmcnt<JMAX * CPW>();
    else lg_wait<CPW, JMAX - 1>(after);
  }
}

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// the same block shape on fp16 operands
__device__ __forceinline__ f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 32x32 block, k = 32, int8 x int8 -> int32 (exact): lane l holds A row l % 32 and B
// row l % 32, k 16 (l / 32) .. +16, as 16 bytes; D as in the bf16 form (checked on
// MI355X against a CPU product).
__device__ __forceinline__ i32x16 mfma32_i8(u32x4 a, u32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// XS = 1: bf16 activations; XS = 2: activations held as two bf16 planes (hi, lo) whose
// sum carries a float32 value to 2^-17: both planes are staged and each is multiplied
// with the same weights (two MFMAs per block), so the product keeps that precision.
// TX = int8_t: int8 activation codes against int8 weights (W8A8), int32 accumulators;
// the epilogue applies the row's activation scale and the weight row's scale.
// TX = f16_t: fp16 activations on the fp16 MFMA; the weights are turned into fp16 as
// they are read from LDS (int8 exactly; bf16 exactly down to 2^-14 in magnitude).
template <typename TW, int BM, int BN, int WGM, int WGN, int S, int BK, int XS,
          typename TX = bf16_t>
struct LgCfg {
  static constexpr int kWaves = WGM * WGN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int WTM = BM / WGM, WTN = BN / WGN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int XRB = BK * (int)sizeof(TX);          // X bytes per row per K tile
  static constexpr int WRB = BK * (int)sizeof(TW);          // W bytes per row per K tile
  static constexpr int CXP = BM * XRB / 1024;               // 1 KB X pieces per plane
  static constexpr int CX = XS * CXP, CW = BN * WRB / 1024; // 1 KB pieces per K tile
  static constexpr int CPW = (CX + CW) / kWaves;           // pieces per wave per K tile
  static constexpr int kStage = XS * BM * XRB + BN * WRB;   // bytes per stage
  static constexpr int kLds = S * kStage;
  static_assert((CX + CW) % kWaves == 0 && CPW * (S - 1) < 64, "piece split");
  static_assert(S >= 2 && S <= 6, "stages");
  static_assert(TM >= 1 && TN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(BK == 64 || (BK == 32 && sizeof(TW) == 2) || (BK == 128 && sizeof(TX) == 1),
                "K tile");
  static_assert(XS == 1 || XS == 2, "activation planes");
  static_assert(sizeof(TX) == 2 || (sizeof(TW) == 1 && XS == 1), "W8A8 tiles");
  static_assert(!std::is_same<TX, f16_t>::value || XS == 1, "fp16 activations: one plane");
  static_assert(kLds <= 160 * 1024, "LDS");
};

// LDS slot of 16-byte piece q of row r for rows of RB bytes (128 or 64): pieces are
// XOR-swizzled by the row's position in the 256-byte bank period, which keeps 16
// consecutive rows' reads of one piece on distinct banks.
template <int RB> __device__ __forceinline__ int lg_slot(int r, int q) {
  return RB == 128 ? (q ^ ((r >> 1) & 7)) : (q ^ ((r >> 2) & 3));
}

// The 16 outputs one lane holds of a 32x32 block: column n, rows m0 + 8 (v / 4) +
// v % 4 (m0 includes the lane's 4 (lane / 32)).  Kept out of line: inlined for every
// block of a wave, the epilogue made the compiler leave the accumulator loops rolled,
// which turned the accumulators into a scratch-memory array stored on every K step.
// The residual mode issues all 16 loads of x before any store.
template <typename TP>
__device__ __attribute__((noinline)) void lg_out16(const EpiParams &ep, float *partial, int z,
                                                   int M, int N, int m0, int n, f32x16 acc) {
  if (n >= N) return;
  if (partial) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + 8 * (v >> 2) + (v & 3);
      if (m < M) partial[((size_t)z * M + m) * N + n] = acc[v];
    }
    return;
  }
  if (ep.mode == EPI_RESID) {
    const float sc = ep.scale ? h2f(ep.scale[n]) : 1.f;
    const float bi = ep.bias ? to_f<TP>(((const TP *)ep.bias)[n]) : 0.f;
    float *x = (float *)ep.out + n;
    float xv[16], xs[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = min(m0 + 8 * (v >> 2) + (v & 3), M - 1);
      xv[v] = x[(size_t)m * ep.ld];
      xs[v] = ep.xscale ? ep.xscale[m] : 1.f;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + 8 * (v >> 2) + (v & 3);
      float y = acc[v];
      if (ep.xscale) y *= xs[v];
      if (ep.scale) y *= sc;
      if (ep.bias) y += bi;
      if (m < M) x[(size_t)m * ep.ld] = xv[v] + y;
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = m0 + 8 * (v >> 2) + (v & 3);
    if (m < M) epilogue<TP>(ep, m, n, acc[v]);
  }
}

// Argmax epilogue of one 32x32 block (LM head): for each of the lane's 16 rows, the
// best (value, lowest index) over the 32 columns its half-wave holds, written by the
// half's first lane to red_v / red_i [local row][col_slot].
template <typename TP>
__device__ __attribute__((noinline)) void lg_argmax16(const EpiParams &ep, int N, int lrow0,
                                                      int n, int col_slot, int nslots,
                                                      float *red_v, int *red_i, f32x16 acc) {
  const float sc = (ep.scale && n < N) ? h2f(ep.scale[n]) : 1.f;
  const float bi0 = (ep.bias && n < N) ? to_f<TP>(((const TP *)ep.bias)[n]) : 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    float bv = n < N ? acc[v] * sc + bi0 : -INFINITY;
    int bi = n < N ? n : 0x7fffffff;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      argmax_take(bv, bi, ov, oi);
    }
    if ((threadIdx.x & 31) == 0) {
      const int lr = lrow0 + 8 * (v >> 2) + (v & 3);
      red_v[lr * nslots + col_slot] = bv;
      red_i[lr * nslots + col_slot] = bi;
    }
  }
}

template <typename TW, typename TP, int BM, int BN, int WGM, int WGN, int S, int BK,
          bool SCHED = false, int XS = 1, typename TX = bf16_t>
__global__ __launch_bounds__(WGM * WGN * 64) void k_gemm_lg(
    const TX *__restrict__ X, const TW *__restrict__ W, int M, int N, int K,
    int tiles_m, int tiles_n, int splits, float *__restrict__ partial, EpiParams ep) {
  using C = LgCfg<TW, BM, BN, WGM, WGN, S, BK, XS, TX>;
  constexpr bool kI8 = sizeof(TW) == 1;
  constexpr bool kX8 = sizeof(TX) == 1;   // W8A8: int8 x int8 on the int32 MFMA
  constexpr bool kXH = std::is_same<TX, f16_t>::value;   // fp16 activations, fp16 MFMA
  using Acc = std::conditional_t<kX8, i32x16, f32x16>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char lg_lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid % WGM, wn = wid / WGM;
  const int nb = gridDim.x, b = blockIdx.x, xcd = b & 7, slot = b >> 3;
  const int L = xcd * (nb >> 3) + min(xcd, nb & 7) + slot;     // bijective renumbering
  const int mt = L % tiles_m, nt = (L / tiles_m) % tiles_n, z = L / (tiles_m * tiles_n);
  const int m0 = mt * BM, n0 = nt * BN;
  const int KT = K / BK;
  const int kt0 = (int)(((long)KT * z) / splits), kt1 = (int)(((long)KT * (z + 1)) / splits);

  // Source of each of this wave's pieces: a 1 KB piece holds 1024 / RB rows of RB
  // bytes; lane -> row lane / (RB / 16), LDS slot lane % (RB / 16), which holds the
  // row's 16-byte piece lg_slot(row, slot) (the swizzle is an involution).
  const unsigned char *src[C::CPW];
#pragma unroll
  for (int c = 0; c < C::CPW; ++c) {
    const int pc = wid * C::CPW + c;
    if (pc < C::CX) {
      constexpr int LPR = C::XRB / 16;
      const int pl = pc / C::CXP;                     // activation plane (hi, lo)
      const int rr = (pc - pl * C::CXP) * (1024 / C::XRB) + lane / LPR;
      const int q = lg_slot<C::XRB>(rr, lane % LPR);
      src[c] = (const unsigned char *)(X + (size_t)pl * M * K + (size_t)min(m0 + rr, M - 1) * K) +
               q * 16;
    } else {
      constexpr int LPR = C::WRB / 16;
      const int rr = (pc - C::CX) * (1024 / C::WRB) + lane / LPR;
      const int q = lg_slot<C::WRB>(rr, lane % LPR);
      src[c] = (const unsigned char *)(W + (size_t)min(n0 + rr, N - 1) * K) + q * 16;
    }
  }
  auto issue = [&](int kt) {
    unsigned char *st = lg_lds + (kt % S) * C::kStage;
#pragma unroll
    for (int c = 0; c < C::CPW; ++c) {
      const int pc = wid * C::CPW + c;
      const size_t adv = (size_t)kt * (pc < C::CX ? C::XRB : C::WRB);   // bytes per K tile
      __builtin_amdgcn_global_load_lds((const void *)(src[c] + adv),
                                       (__attribute__((address_space(3))) void *)(
                                           st + pc * 1024),
                                       16, 0, 0);
    }
  };

  Acc acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[i][j] = Acc{};

#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (kt0 + p < kt1) issue(kt0 + p);
  for (int kt = kt0; kt < kt1; ++kt) {
    // This wave's copies of tile kt have landed once at most (tiles issued after it) x
    // CPW of its loads are outstanding; the barrier (deliberately without a memory
    // fence, which would make the compiler wait for every outstanding load) then makes
    // every wave's copies visible, and also orders every wave's reads of the stage
    // refilled below, which the previous step read.
    lg_wait<C::CPW, S - 2>(min(S - 2, kt1 - 1 - kt));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (kt + S - 1 < kt1) issue(kt + S - 1);
    const unsigned char *xb = lg_lds + (kt % S) * C::kStage;
    const unsigned char *wb = xb + C::CX * 1024;
    if constexpr (kX8) {
      // 32-wide substeps; both operands are 16-byte pieces of the K tile's rows, read for
      // every substep of the tile before its MFMAs
      constexpr int NSUB = BK / 32;
      u32x4 a[NSUB][C::TM], bv[NSUB][C::TN];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const int piece = 2 * s + (lane >> 5);
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
          const int r = wm * C::WTM + 32 * i + (lane & 31);
          a[s][i] = *(const u32x4 *)(xb + r * C::XRB + 16 * lg_slot<C::XRB>(r, piece));
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          const int r = wn * C::WTN + 32 * j + (lane & 31);
          bv[s][j] = *(const u32x4 *)(wb + r * C::WRB + 16 * lg_slot<C::WRB>(r, piece));
        }
      }
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma32_i8(a[s][i], bv[s][j], acc[i][j]);
    } else {
      // operands of 16-wide substep s + 1 are read while the MFMAs of substep s run
      u32x4 a[2][XS][C::TM], bv[2][C::TN];
      auto rd = [&](int s, int q) {
        const int piece = 2 * s + (lane >> 5);   // 8-element k-piece within the K tile
#pragma unroll
        for (int pl = 0; pl < XS; ++pl)
#pragma unroll
          for (int i = 0; i < C::TM; ++i) {
            const int r = wm * C::WTM + 32 * i + (lane & 31);
            a[q][pl][i] = *(const u32x4 *)(xb + pl * C::CXP * 1024 + r * C::XRB +
                                           16 * lg_slot<C::XRB>(r, piece));
          }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          const int r = wn * C::WTN + 32 * j + (lane & 31);
          if constexpr (kI8) {
            // 8 int8 of k-piece `piece` (half of a 16-byte slot), widened to bf16 (exact)
            const uint2 t = *(const uint2 *)(wb + r * C::WRB +
                                             16 * lg_slot<C::WRB>(r, piece >> 1) +
                                             8 * (piece & 1));
            bv[q][j] = kXH ? i8x8_to_f16x8(t.x, t.y) : i8x8_to_bf16x8(t.x, t.y);
          } else {
            const u32x4 t = *(const u32x4 *)(wb + r * C::WRB + 16 * lg_slot<C::WRB>(r, piece));
            bv[q][j] = kXH ? bf16x8_to_f16x8(t) : t;
          }
        }
      };
      rd(0, 0);
#pragma unroll
      for (int s = 0; s < BK / 16; ++s) {
        if (s + 1 < BK / 16) rd(s + 1, (s + 1) & 1);
#pragma unroll
        for (int pl = 0; pl < XS; ++pl)
#pragma unroll
          for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
              acc[i][j] = kXH ? mfma32_f16(a[s & 1][pl][i], bv[s & 1][j], acc[i][j])
                              : mfma32(a[s & 1][pl][i], bv[s & 1][j], acc[i][j]);
        if constexpr (SCHED) {
          // interleave: one MFMA, then one of the next substep's LDS reads, ...
          if (s + 1 < BK / 16) {
#pragma unroll
            for (int q = 0; q < C::TM + C::TN; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, C::TM * C::TN - (C::TM + C::TN), 0);
          }
        }
      }
    }
  }

  // D layout of a 32x32 block: lane holds column lane % 32, value v row
  // 8 (v / 4) + 4 (lane / 32) + v % 4
  if constexpr (kX8) {
    // int32 sums (exact) -> float32; the scales come in the epilogue
    float *part = splits > 1 ? partial : nullptr;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        lg_out16<TP>(ep, part, z, M, N, m0 + wm * C::WTM + 32 * i + 4 * (lane >> 5),
                     n0 + wn * C::WTN + 32 * j + (lane & 31),
                     __builtin_convertvector(acc[i][j], f32x16));
    return;
  } else {
    if (ep.mode == EPI_ARGMAX) {
      // one (max, index) partial per row per N tile (the plan never splits K here)
      constexpr int NS = WGN * C::TN;
      float *red_v = (float *)lg_lds;
      int *red_i = (int *)(lg_lds + BM * NS * sizeof(float));
      __syncthreads();  // every wave is done reading the LDS stages
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          lg_argmax16<TP>(ep, N, wm * C::WTM + 32 * i + 4 * (lane >> 5),
                          n0 + wn * C::WTN + 32 * j + (lane & 31), wn * C::TN + j, NS, red_v,
                          red_i, acc[i][j]);
      __syncthreads();
      for (int lr = tid; lr < BM; lr += C::kThreads) {
        const int m = m0 + lr;
        if (m >= M) continue;
        float bv = red_v[lr * NS];
        int bi = red_i[lr * NS];
        for (int c = 1; c < NS; ++c) argmax_take(bv, bi, red_v[lr * NS + c], red_i[lr * NS + c]);
        ep.am_val[(size_t)m * ep.am_stride + nt] = bv;
        ep.am_idx[(size_t)m * ep.am_stride + nt] = bi;
      }
      return;
    }
    float *part = splits > 1 ? partial : nullptr;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        lg_out16<TP>(ep, part, z, M, N, m0 + wm * C::WTM + 32 * i + 4 * (lane >> 5),
                     n0 + wn * C::WTN + 32 * j + (lane & 31), acc[i][j]);
  }
}

// ---------------------------------------------------------------------------
// generic float32 path: one thread per output, blocks of 256 consecutive n
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemm_f32(const float *__restrict__ X,
                                                  const float *__restrict__ W, int M, int N, int K,
                                                  EpiParams ep) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int m = blockIdx.y;
  const int n = blockIdx.x * 256 + threadIdx.x;
  float s = 0.f;
  if (n < N) {
    const float *x = X + (size_t)m * K;
    const float *w = W + (size_t)n * K;
    for (int k = 0; k < K; ++k) s = fmaf(x[k], w[k], s);
  }
  if (ep.mode != EPI_ARGMAX) {
    if (n < N) epilogue<float>(ep, m, n, s);
    return;
  }
  float bv = n < N ? s : -INFINITY;
  int bi = n < N ? n : 0x7fffffff;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    argmax_take(bv, bi, ov, oi);
  }
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) argmax_take(bv, bi, sv[w], si[w]);
    ep.am_val[(size_t)m * ep.am_stride + blockIdx.x] = bv;
    ep.am_idx[(size_t)m * ep.am_stride + blockIdx.x] = bi;
  }
}

// ---------------------------------------------------------------------------
// split-K reduction (fixed order over splits) + epilogue
// ---------------------------------------------------------------------------
// All S (<= kMaxSplits) partials of an output are loaded before the first add, so the
// loads overlap; the sum runs over z = 0, 1, ... in that fixed order.
constexpr int kMaxSplits = 8;

template <typename TP>
__global__ __launch_bounds__(256) void k_splitk_epilogue(const float *__restrict__ partial, int S,
                                                         int M, int N, EpiParams ep) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t MN = (size_t)M * N;
  if (idx >= MN) return;
  float v[kMaxSplits];
#pragma unroll
  for (int z = 0; z < kMaxSplits; ++z) v[z] = z < S ? partial[(size_t)z * MN + idx] : 0.f;
  float s = 0.f;
#pragma unroll
  for (int z = 0; z < kMaxSplits; ++z)
    if (z < S) s += v[z];
  epilogue<TP>(ep, (int)(idx / N), (int)(idx % N), s);
}

// Final greedy choice per row: lowest index among the per-tile maxima.  1024 threads,
// each folding a strided slice of the partials with independent loads.
constexpr int kMergeThreads = 1024;

__global__ __launch_bounds__(kMergeThreads) void k_argmax_merge(const float *__restrict__ val,
                                                                const int *__restrict__ idx,
                                                                int stride, int nblk,
                                                                int *__restrict__ out) {
  __shared__ float sv[kMergeThreads / 64];
  __shared__ int si[kMergeThreads / 64];
  const int m = blockIdx.x;
  const float *vr = val + (size_t)m * stride;
  const int *ir = idx + (size_t)m * stride;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  int b = threadIdx.x;
  for (; b + 3 * kMergeThreads < nblk; b += 4 * kMergeThreads) {
    float v[4];
    int i[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) { v[u] = vr[b + u * kMergeThreads]; i[u] = ir[b + u * kMergeThreads]; }
#pragma unroll
    for (int u = 0; u < 4; ++u) argmax_take(bv, bi, v[u], i[u]);
  }
  for (; b < nblk; b += kMergeThreads) argmax_take(bv, bi, vr[b], ir[b]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    argmax_take(bv, bi, ov, oi);
  }
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = bv; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kMergeThreads / 64; ++w) argmax_take(bv, bi, sv[w], si[w]);
    out[m] = bi == 0x7fffffff ? 0 : bi;
  }
}

// ---------------------------------------------------------------------------
// host-side planning and launch
// ---------------------------------------------------------------------------
// Tile configurations of the direct-to-LDS GEMM (LinearPlan::lg).
enum LgTile : int {
  LG_256 = 1,      // 256 x 256, 8 waves (4 x 2), 2 stages (prompt pass, 512+ rows)
  LG_128 = 0,      // 128 x 128, 4 waves, 2 stages (prompt pass, 256+ rows)
  LG_D32 = 2,      // 32 x 128, 4 waves, 4 stages (decode / short passes, <= 32 rows)
  LG_D64 = 3,      // 64 x 128, 4 waves, 3 stages (<= 64 rows)
  LG_D128 = 4,     // 128 x 128, 4 waves, 3 stages (<= 128 rows)
  LG_256x128 = 5,  // 256 x 128, 8 waves (4 x 2), 3 stages (prompt pass, 512-1023 rows)
  LG_D32W = 6,     // 32 x 256, 4 waves, 4 stages (int8 weights, <= 32 rows)
  LG_D64W = 7,     // 64 x 256, 4 waves (1 x 4), 3 stages (int8 weights, <= 64 rows, long N)
  LG_D128N = 8,    // 128 x 128, 4 waves (1 x 4), 3 stages (int8 weights, <= 128 rows)
  LG_P8 = 9,       // 128 x 256, 4 waves (1 x 4), 2 stages (int8 weights, prompt pass)
  LG_X8_128 = 10,  // W8A8: 128 x 256, 8 waves (2 x 4), 3 stages of 128-wide K tiles
  LG_X8_64 = 11,   // W8A8: 64 x 256, 4 waves (1 x 4), 3 stages of 128-wide K tiles
  LG_X8_32 = 12,   // W8A8: 32 x 256, 4 waves (1 x 4), 4 stages of 128-wide K tiles
  LG_D128P = 13,   // two bf16 planes: 128 x 256, 8 waves (2 x 4), 4 stages of 32-wide K tiles
  LG_256H = 14,    // fp16 activations: 256 x 256, 8 waves (2 x 4), 2 stages (1024+ rows)
  LG_256x128H = 15,  // fp16 activations: 256 x 128, 8 waves (2 x 4), 3 stages (512-1023 rows)
  LG_128H = 16,    // fp16 activations: 128 x 128, 4 waves (1 x 4), 2 stages (256-511 rows)
  LG_X8_P = 17,    // W8A8 prompt pass: 256 x 256, 8 waves (2 x 4), 2 stages of 128-wide K tiles
};

LinearPlan plan_linear(int wdtype, int M, int N, int K, bool argmax, int act) {
  LinearPlan p{};
  p.M = M; p.N = N; p.K = K;
  if (wdtype == WT_F32) {
    p.kind = LIN_F32;
    p.grid_x = (N + 255) / 256;
    p.splits = 1;
    return p;
  }
  const bool q8 = act == AF_I8;   // W8A8 (int8 weights only; the caller checks)
  if (M <= kValuMaxRows) {
    // int8 activations: the GEMV reads the codes (the epilogue applies the row scales)
    p = plan_valu(wdtype, M, N, K);
    if (argmax && p.ks != 1) {   // the argmax epilogue takes whole rows per wave
      p.ks = 1;
      p.vu = 28;
      p.grid_x = (N + 4 * p.vr - 1) / (4 * p.vr);
    }
    p.x_fmt = act;
    p.q8 = q8;
    return p;
  }
  // Direct-to-LDS MFMA GEMM for everything else (hidden sizes are multiples of 64).
  p.kind = LIN_LG;
  // fp16 activations: one fp16 plane on the fp16 MFMA; float32 ones: two bf16 planes
  p.xs = act == AF_F32 ? 2 : 1;
  p.xh = act == AF_F16;
  p.x8 = q8;
  p.q8 = q8;
  const int KT = K / kLg;
  if (!argmax && M >= 256) {
    // Prompt passes: tiles of 256 x 256 (8 waves of 64 x 128, one block per CU: 128 KB
    // of LDS) from 1024 rows, 256 x 128 with 3 stages (8 waves of 64 x 64, 144 KB) from
    // 512 rows, else 128 x 128 (two blocks per CU).  Split-K is chosen to minimise
    // (rounds of resident blocks) / splits, with a 10% charge for the reduction pass.
    // Measured on the 176B share (% of the bf16 MFMA peak): 512 rows, 256 x 128 against
    // 256 x 256: QKV 32.8 / 30.7, dense 23.3 / 18.2, down 34.9 / 33.9, up 33.6 / 34.7;
    // 2048 rows, dense 29.0 with 256 x 256 against 23.5 with 128 x 128.
    // int8 weights: 128 x 256 tiles with the four waves side by side (each wave all 128
    // rows and 64 columns, so every weight is widened to bf16 once per block), two
    // blocks per CU.  Measured (full 176B int8, 256 rows): QKV 506.6 -> 372.2 us, up
    // 621.7 -> 471.6, down 618.4 -> 486.8; 2048 rows: down 4675 -> 3442 us.
    // Two activation planes double the X tile: 128 x 128 tiles (96 KB of LDS) are the
    // largest bf16 prompt tiles that still fit.
    // W8A8: the same 128 x 256 tiles, int8 activation rows of 64 bytes per K tile.
    // fp16 activations against bf16 weights: each wave turns the weights it reads into
    // fp16, so the wave grids put fewer waves on each weight column (2 x 4 instead of
    // 4 x 2, 1 x 4 instead of 2 x 2).  Measured (176B share, the four linears, fp16
    // activations): 2048 rows 2190 -> 1838 us, 512 rows 637 -> 559 us, 256 rows 367 ->
    // 346 us.
    // W8A8 with K a multiple of 128: 256 x 256 tiles of 128-wide K tiles (128-byte rows of
    // both operands per copy, as the bf16 prompt tiles); measured on the full 176B int8
    // linears against the 128 x 256 tiles of 64-wide K tiles: 256 rows 1556 -> 971 us,
    // 1024 rows 5322 -> 3184 us, 2048 rows 10353 -> 5792 us (35% of the int8 peak).
    if (wdtype == WT_INT8) p.lg = (q8 && K % 128 == 0) ? LG_X8_P : LG_P8;
    else if (p.xs == 2) p.lg = LG_128;
    else if (p.xh) p.lg = M >= 1024 ? LG_256H : (M >= 512 ? LG_256x128H : LG_128H);
    else p.lg = M >= 1024 ? LG_256 : (M >= 512 ? LG_256x128 : LG_128);
    const bool bm128 = p.lg == LG_128 || p.lg == LG_P8 || p.lg == LG_128H;
    const int bm = bm128 ? 128 : 256;
    const int bn =
        (p.lg == LG_256 || p.lg == LG_P8 || p.lg == LG_256H || p.lg == LG_X8_P) ? 256 : 128;
    const int slots = bm128 ? 512 : 256;
    p.grid_x = (M + bm - 1) / bm;
    p.grid_y = (N + bn - 1) / bn;
    const long tiles = (long)p.grid_x * p.grid_y;
    int best = 1;
    double best_cost = 1e30;
    for (int sp = 1; sp <= 8 && sp <= KT; ++sp) {
      if (sp > 1 && (long)sp * M * N > kLgPartialCapFloats) break;
      const double cost = (double)((tiles * sp + slots - 1) / slots) / sp + (sp > 1 ? 0.1 : 0.0);
      if (cost < best_cost - 1e-9) { best_cost = cost; best = sp; }
    }
    p.splits = best;
    return p;
  }
  // Decode batches, LM heads and short passes: a 32/64/128-row activation tile against
  // 128 weight rows, 3-4 LDS stages in flight, and K split (each split keeping >= 8 K
  // tiles).  bf16 weights: the split gives about one block per CU.  Measured on MI355X
  // (176B share, 128 rows; per-shape best split in brackets): QKV 5376 x 14336 53.4 us
  // with 4 splits -> 45.5 us with 6 [6], up 4 splits [4], down and dense 2 [2].
  // int8 weights: the 64-byte K-tile rows leave little in flight per stage and the
  // widening to bf16 costs vector-ALU time, so the tiles take 256 weight rows where N
  // is long (one wave per 64 columns), the 128-row tile gives each wave all 128 rows
  // and 32 columns (every weight widened once), two blocks fit per CU, and the split
  // minimises rounds of 512 resident blocks per split (+10% for the reduction).
  // Measured (full 176B int8): 16 rows QKV 43008 x 14336 175.6 -> 146.0 us, up
  // 214.4 -> 193.3, down 247.0 -> 196.9; 64 rows QKV 197.3 -> 172.8, up 263.1 ->
  // 227.2; 128 rows QKV 295.0 -> 258.0, down 364.7 -> 345.0.  The argmax epilogue
  // needs whole dot products, so the LM head is never split.
  const bool i8 = wdtype == WT_INT8;
  int bm, bn;
  if (!i8) {
    p.lg = M <= 32 ? LG_D32 : (M <= 64 ? LG_D64 : LG_D128);
    bm = M <= 32 ? 32 : (M <= 64 ? 64 : 128);
    bn = 128;
    // two bf16 planes and 65-128 rows: 128 x 256 tiles of 32-wide K tiles (one block per
    // CU; the 176B share's four linears 254 -> 242 us at 128 rows)
    if (p.xs == 2 && M > 64) { p.lg = LG_D128P; bn = 256; }
  } else if (q8) {
    // W8A8: 256 weight rows per block and 128-wide K tiles (128-byte rows of both
    // operands per copy); one block per CU.  Measured on MI355X (full 176B int8 linears,
    // QKV + dense + up + down, against 64-wide K tiles 128 x 128 / 64 x 256): 128 rows
    // 879 -> 620 us, 64 rows 626 -> 548, 16 rows 540 -> 475.
    // (K not a multiple of 128: the 64-wide K tiles, 64 x 256 / 128 x 128)
    if (K % 128) {
      if (M <= 64) { p.lg = LG_D64W; bm = 64; bn = 256; }
      else { p.lg = LG_D128N; bm = 128; bn = 128; }
    } else {
      if (M <= 32) { p.lg = LG_X8_32; bm = 32; }
      else if (M <= 64) { p.lg = LG_X8_64; bm = 64; }
      else { p.lg = LG_X8_128; bm = 128; }
      bn = 256;
    }
  } else if (M <= 32) {
    p.lg = LG_D32W; bm = 32; bn = 256;
  } else if (M <= 64) {
    p.lg = N >= 32768 ? LG_D64W : LG_D64; bm = 64; bn = N >= 32768 ? 256 : 128;
  } else {
    p.lg = LG_D128N; bm = 128; bn = 128;
  }
  p.grid_x = (M + bm - 1) / bm;
  p.grid_y = (N + bn - 1) / bn;
  const long tiles = (long)p.grid_x * p.grid_y;
  int sp = 1;
  const int kt_plan = p.lg == LG_D128P ? K / 32 : (q8 && !(K % 128) ? K / 128 : KT);
  const bool x8_tile = p.lg == LG_X8_128 || p.lg == LG_X8_64 || p.lg == LG_X8_32;
  if (!i8 && p.lg != LG_D128P) {
    sp = (int)max(1l, min(8l, 256 / tiles));
  } else if (x8_tile) {
    // W8A8 tiles, one block per CU: the fewest splits that put 60% of the CUs to work
    // (measured on the 176B int8 linears: 168 or 224 blocks stream as fast unsplit as
    // split, and a split's float32 partials cost traffic -- MLP-up at 128 rows 200 us
    // unsplit, 282 us in two; 56 blocks want 3-4 splits)
    while (sp < 8 && tiles * sp < 154) ++sp;
  } else {
    // the split minimises rounds of resident blocks per split, +10% for the reduction
    // pass: two blocks per CU for the 64-wide int8 tiles, one for the two-plane 128 x 256
    const long slots = p.lg == LG_D128P ? 256 : 512;
    double best_cost = 1e30;
    for (int s2 = 1; s2 <= 8; ++s2) {
      const double cost = (double)((tiles * s2 + slots - 1) / slots) / s2 + (s2 > 1 ? 0.1 : 0.0);
      if (cost < best_cost - 1e-9) { best_cost = cost; sp = s2; }
    }
  }
  while (sp > 1 && kt_plan / sp < 8) --sp;
  while (sp > 1 && (long)sp * M * N > kLgPartialCapFloats) --sp;
  p.splits = argmax ? 1 : sp;
  return p;
}

int plan_x_fmt(const LinearPlan &p) {
  if (p.kind == LIN_F32) return AF_F32;
  if (p.kind == LIN_VALU) return p.x_fmt;
  if (p.x8) return AF_I8;
  if (p.xh) return AF_F16;
  return p.xs == 2 ? AF_BF16X2 : AF_BF16;
}

int argmax_partials_per_row(const LinearPlan &p) {
  return p.kind == LIN_LG ? p.grid_y : p.grid_x;
}

size_t linear_partial_bytes(const LinearPlan &p) {
  return p.splits > 1 ? (size_t)p.splits * p.M * p.N * sizeof(float) : 0;
}

// More than 64 KB of dynamic LDS must be allowed once per kernel and device; the flags
// are set under a lock so that concurrent callers (distinct caches and workspaces) are
// safe.
static std::mutex g_lds_attr_mu;

template <typename TW, int BM, int BN, int WGM, int WGN, int S, int BK = kLg, int XS = 1,
          typename TX = bf16_t>
static hipError_t launch_lg_t(const LinearPlan &p, const void *X, const void *W, float *partial,
                              const EpiParams &ep, hipStream_t st) {
  using C = LgCfg<TW, BM, BN, WGM, WGN, S, BK, XS, TX>;
  static std::atomic<uint64_t> attr_set{0};   // bit per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_set.load(std::memory_order_acquire) & bit)) {
    std::lock_guard<std::mutex> lock(g_lds_attr_mu);
    if (!(attr_set.load(std::memory_order_relaxed) & bit)) {
      e = hipFuncSetAttribute(
          (const void *)k_gemm_lg<TW, bf16_t, BM, BN, WGM, WGN, S, BK, false, XS, TX>,
          hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
      if (e != hipSuccess) return e;
      attr_set.fetch_or(bit, std::memory_order_release);
    }
  }
  BL_LAUNCH((k_gemm_lg<TW, bf16_t, BM, BN, WGM, WGN, S, BK, false, XS, TX>),
            dim3((unsigned)(p.grid_x * p.grid_y * p.splits)), dim3(C::kThreads), C::kLds, st,
            (const TX *)X, (const TW *)W, p.M, p.N, p.K, p.grid_x, p.grid_y, p.splits,
            partial, ep);
  return hipGetLastError();
}

template <typename TW, int XS, typename TX = bf16_t>
static hipError_t launch_lg(const LinearPlan &p, const void *X, const void *W, float *partial,
                            const EpiParams &ep, hipStream_t st) {
  switch (p.lg) {
    case LG_256:
      if constexpr (XS == 1) return launch_lg_t<TW, 256, 256, 4, 2, 2, kLg, 1, TX>(p, X, W, partial, ep, st);
      return hipErrorInvalidValue;
    case LG_128: return launch_lg_t<TW, 128, 128, 2, 2, 2, kLg, XS, TX>(p, X, W, partial, ep, st);
    case LG_D32: return launch_lg_t<TW, 32, 128, 1, 4, 4, kLg, XS, TX>(p, X, W, partial, ep, st);
    case LG_D64: return launch_lg_t<TW, 64, 128, 1, 4, 3, kLg, XS, TX>(p, X, W, partial, ep, st);
    case LG_256x128:
      if constexpr (XS == 1) return launch_lg_t<TW, 256, 128, 4, 2, 3, kLg, 1, TX>(p, X, W, partial, ep, st);
      return hipErrorInvalidValue;
    case LG_D32W:
      if constexpr (sizeof(TW) == 1)
        return launch_lg_t<TW, 32, 256, 1, 4, 4, kLg, XS, TX>(p, X, W, partial, ep, st);
      return hipErrorInvalidValue;
    case LG_D64W:
      if constexpr (sizeof(TW) == 1)
        return launch_lg_t<TW, 64, 256, 1, 4, 3, kLg, XS, TX>(p, X, W, partial, ep, st);
      return hipErrorInvalidValue;
    case LG_D128N:
      if constexpr (sizeof(TW) == 1)
        return launch_lg_t<TW, 128, 128, 1, 4, 3, kLg, XS, TX>(p, X, W, partial, ep, st);
      return hipErrorInvalidValue;
    case LG_P8:
      if constexpr (sizeof(TW) == 1)
        return launch_lg_t<TW, 128, 256, 1, 4, 2, kLg, XS, TX>(p, X, W, partial, ep, st);
      return hipErrorInvalidValue;
    case LG_256H:
      if constexpr (XS == 1) return launch_lg_t<TW, 256, 256, 2, 4, 2, kLg, 1, TX>(p, X, W, partial, ep, st);
      return hipErrorInvalidValue;
    case LG_256x128H:
      if constexpr (XS == 1) return launch_lg_t<TW, 256, 128, 2, 4, 3, kLg, 1, TX>(p, X, W, partial, ep, st);
      return hipErrorInvalidValue;
    case LG_128H: return launch_lg_t<TW, 128, 128, 1, 4, 2, kLg, XS, TX>(p, X, W, partial, ep, st);
    case LG_D128P:
      if constexpr (sizeof(TW) == 2 && XS == 2)
        return launch_lg_t<TW, 128, 256, 2, 4, 4, 32, XS, TX>(p, X, W, partial, ep, st);
      return hipErrorInvalidValue;
    default: return launch_lg_t<TW, 128, 128, 2, 2, 3, kLg, XS, TX>(p, X, W, partial, ep, st);
  }
}

// W8A8 tiles (int8 activation codes against int8 weights)
static hipError_t launch_lg_x8(const LinearPlan &p, const void *X, const void *W, float *partial,
                               const EpiParams &ep, hipStream_t st) {
  switch (p.lg) {
    case LG_X8_128:
      return launch_lg_t<int8_t, 128, 256, 2, 4, 3, 128, 1, int8_t>(p, X, W, partial, ep, st);
    case LG_X8_64: return launch_lg_t<int8_t, 64, 256, 1, 4, 3, 128, 1, int8_t>(p, X, W, partial, ep, st);
    case LG_X8_32: return launch_lg_t<int8_t, 32, 256, 1, 4, 4, 128, 1, int8_t>(p, X, W, partial, ep, st);
    case LG_D64W: return launch_lg_t<int8_t, 64, 256, 1, 4, 3, kLg, 1, int8_t>(p, X, W, partial, ep, st);
    case LG_D128N: return launch_lg_t<int8_t, 128, 128, 1, 4, 3, kLg, 1, int8_t>(p, X, W, partial, ep, st);
    case LG_P8: return launch_lg_t<int8_t, 128, 256, 1, 4, 2, kLg, 1, int8_t>(p, X, W, partial, ep, st);
    case LG_X8_P: return launch_lg_t<int8_t, 256, 256, 2, 4, 2, 128, 1, int8_t>(p, X, W, partial, ep, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_linear(int wdtype, const LinearPlan &p, const void *X, const void *W,
                         float *partial, const EpiParams &ep, hipStream_t st,
                         bool splitk_epilogue) {
  if (p.M <= 0) return hipSuccess;
  // a folded LayerNorm's statistics exist on the one-row vector-ALU GEMV only
  if ((ep.ln_stats || ep.fold_stats) && p.kind != LIN_VALU) return hipErrorInvalidValue;
  if (p.kind == LIN_F32) {
    BL_LAUNCH(k_gemm_f32, dim3(p.grid_x, p.M), dim3(256), 0, st, (const float *)X,
                       (const float *)W, p.M, p.N, p.K, ep);
    return hipGetLastError();
  }
  if (p.kind == LIN_VALU) return launch_valu(wdtype, p, X, W, ep, st);
  if (p.kind != LIN_LG || p.splits > kMaxSplits || (p.xs != 1 && p.xs != 2))
    return hipErrorInvalidValue;
  if (p.x8 && (wdtype != WT_INT8 || !ep.xscale || ep.mode == EPI_ARGMAX))
    return hipErrorInvalidValue;
  if ((p.lg == LG_X8_128 || p.lg == LG_X8_64 || p.lg == LG_X8_32 || p.lg == LG_X8_P) && p.K % 128)
    return hipErrorInvalidValue;
  hipError_t e;
  if (p.x8)
    e = launch_lg_x8(p, X, W, partial, ep, st);
  else if (p.xh)
    e = wdtype == WT_BF16 ? launch_lg<bf16_t, 1, f16_t>(p, X, W, partial, ep, st)
                          : launch_lg<int8_t, 1, f16_t>(p, X, W, partial, ep, st);
  else if (wdtype == WT_BF16)
    e = p.xs == 2 ? launch_lg<bf16_t, 2>(p, X, W, partial, ep, st)
                  : launch_lg<bf16_t, 1>(p, X, W, partial, ep, st);
  else
    e = p.xs == 2 ? launch_lg<int8_t, 2>(p, X, W, partial, ep, st)
                  : launch_lg<int8_t, 1>(p, X, W, partial, ep, st);
  if (e != hipSuccess) return e;
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.splits <= 1 || !splitk_epilogue) return err;
  const size_t MN = (size_t)p.M * p.N;
  BL_LAUNCH((k_splitk_epilogue<bf16_t>), dim3((unsigned)((MN + 255) / 256)),
                     dim3(256), 0, st, partial, p.splits, p.M, p.N, ep);
  return hipGetLastError();
}

hipError_t launch_argmax_merge(const float *val, const int *idx, int stride, int nblk, int rows,
                               int *out, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_argmax_merge, dim3(rows), dim3(kMergeThreads), 0, st, val, idx, stride,
                     nblk, out);
  return hipGetLastError();
}

}  // namespace bl
