// ALiBi attention of one query row over the KV cache, and the standalone KV append.
//
// One 256-thread block per (query row m, head h).  Query row m belongs to sequence
// b = m / rows_per_seq at absolute position qpos = pos_base + m % rows_per_seq (the
// decode step: rows_per_seq = 1, pos_base = current length; the prompt pass:
// rows_per_seq = prompt length, pos_base = 0).  Keys j in [pad_b, qpos] are visible,
// pad_b = prompt_len - valid_len[b] (left padding).  Steps, all in float32:
//   1. s_j = q . k_j + slope_h * (j - qpos)   (q already carries 1/sqrt(d); keys and
//      values read as 16-byte pieces, d/8 lanes per key, partial dots summed across
//      those lanes; all K and V loads of a batch of slots are issued together, before
//      the row's valid length is known; slots before pad_b are masked)
//   2. softmax over the visible keys only -- masked keys are never touched, i.e. they
//      get probability exactly 0.  Within a batch: block max, exp, running sum; across
//      batches (rows longer than one batch) the running sum and the P.V accumulators
//      are rescaled by exp(old max - new max), the usual online form of the same
//      softmax.
//   3. o = (sum_j p_j v_j) / sum_j p_j, per lane group over its keys, then summed over
//      the groups in LDS in a fixed order.
// A query with no visible key (a left-pad position of the prompt) gets o = 0.
// An int8 cache holds codes and one float32 scale per (row, head, slot) for keys and for
// values: the key's scale multiplies its dot product, the value's scale its probability
// weight in P.V (the same products as with the dequantised vectors, rounded once more).
// ("Hugging Face BLOOM Inference Optimization", Custom CUDA Kernels and Hardware
// Acceleration, for the fused mask + float32 softmax; "DeepSpeed Inference ...",
// Section III.D, attention fused as one kernel.)
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace bl {

template <typename TA> struct KVLoad8;
template <> struct KVLoad8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t *p, float v[8]) {
    const u32x4 t = *(const u32x4 *)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = lo_bf(t[i]); v[2 * i + 1] = hi_bf(t[i]); }
  }
};
template <> struct KVLoad8<float> {
  static __device__ __forceinline__ void load(const float *p, float v[8]) {
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// Raw 8-element pieces of a key / value row as loaded (bf16: one 16-byte load).
template <typename TA> struct KVRaw;
template <> struct KVRaw<bf16_t> {
  u32x4 a;
  __device__ __forceinline__ void load(const bf16_t *p) { a = *(const u32x4 *)p; }
  __device__ __forceinline__ float get(int t) const {
    return (t & 1) ? hi_bf(a[t >> 1]) : lo_bf(a[t >> 1]);
  }
};
template <> struct KVRaw<f16_t> {
  u32x4 a;
  __device__ __forceinline__ void load(const f16_t *p) { a = *(const u32x4 *)p; }
  __device__ __forceinline__ float get(int t) const {
    return (t & 1) ? f16hi(a[t >> 1]) : f16lo(a[t >> 1]);
  }
};
template <> struct KVRaw<int8_t> {
  uint2 a;   // 8 int8 codes; the key's scale is applied to its dot product / probability
  __device__ __forceinline__ void load(const int8_t *p) { a = *(const uint2 *)p; }
  __device__ __forceinline__ float get(int t) const {
    return (float)(int8_t)((t < 4 ? a.x : a.y) >> (8 * (t & 3)));
  }
};
template <> struct KVRaw<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float *p) {
    a = *(const float4 *)p;
    b = *(const float4 *)(p + 4);
  }
  __device__ __forceinline__ float get(int t) const {
    const float4 &v = t < 4 ? a : b;
    switch (t & 3) { case 0: return v.x; case 1: return v.y; case 2: return v.z; default: return v.w; }
  }
};

// Keys per lane group per batch: all K and V loads of a batch are issued together.
template <typename TA> struct KeysPerBatch { static constexpr int value = 8; };
template <> struct KeysPerBatch<float> { static constexpr int value = 4; };

template <typename TA>
__global__ __launch_bounds__(256) void k_attention(const float *__restrict__ q,
                                                   const TA *__restrict__ kc,
                                                   const TA *__restrict__ vc,
                                                   const float *__restrict__ ksc,
                                                   const float *__restrict__ vsc,
                                                   const int *__restrict__ valid_len,
                                                   void *__restrict__ o, int o_fmt,
                                                   size_t o_plane, int H, int d, int max_len,
                                                   int n_total, int head_off, int rows_per_seq,
                                                   int pos_base, const int *__restrict__ pos_dev,
                                                   int prompt_len, int chunk,
                                                   float *__restrict__ part) {
  constexpr int KB = KeysPerBatch<TA>::value;
  constexpr bool kQ = sizeof(TA) == 1;   // int8 cache with per-slot scales
  __shared__ float pv[256 * 8];     // [G][d] per-group P.V partials
  __shared__ float red[4];
  const int m = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x;
  const int b = m / rows_per_seq;
  const size_t head_base = ((size_t)b * H + h) * (size_t)max_len * d;
  const TA *kb = kc + head_base;
  const TA *vb = vc + head_base;
  const size_t scale_base = ((size_t)b * H + h) * (size_t)max_len;

  // lane group g (L = d/8 lanes) handles slots j = g (mod G); lane `sub` owns dims
  // [8 sub, 8 sub + 8) of each of them
  const int L = d >> 3;
  const int G = 256 / L;
  const int g = tid / L, sub = tid - g * L;

  // The K/V loads address slots directly and wait neither for the position nor for
  // valid_len: the first batch goes out before the position is read (slots up to the
  // cache end, in bounds), later ones up to the block's last slot; slots past the last
  // visible one, and the left-pad slots [0, first) (the prompt pass wrote them), are
  // masked in the scores.
  KVRaw<TA> kr[KB], vr[KB];
  float ks[KB], vs[KB];
  auto load_batch = [&](int j0, int jcap) {
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int jj = min(j0 + u * G + g, jcap);
      kr[u].load(kb + (size_t)jj * d + 8 * sub);
      vr[u].load(vb + (size_t)jj * d + 8 * sub);
      if constexpr (kQ) {
        ks[u] = ksc[scale_base + jj];
        vs[u] = vsc[scale_base + jj];
      }
    }
  };
  const int z = blockIdx.z;
  const int jlo = part ? z * chunk : 0;
  load_batch(jlo, max_len - 1);

  // a position read from device memory is clamped to the cache (the host checks the
  // others): slots at or past max_len are never addressed
  const int qpos = min((pos_dev ? *pos_dev : pos_base) + (m - b * rows_per_seq), max_len - 1);
  const int vl_in = valid_len[b];
  const size_t out0 = ((size_t)m * H + h) * d;
  const int S = qpos + 1;
  const float slope = alibi_slope(n_total, head_off + h);
  const float *qr = q + ((size_t)m * H + h) * d;
  float qv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) qv[t] = qr[8 * sub + t];
  const int vl = vl_in < 1 ? 1 : (vl_in > prompt_len ? prompt_len : vl_in);
  const int first = prompt_len - vl;

  // Online softmax over batches of G*KB slots (one batch when qpos < G*KB): running
  // maximum mrun (block-uniform), per-thread running sum and P.V accumulators, all
  // rescaled by exp(mrun_old - mrun_new) when the maximum grows.
  // split over the keys (part set): block z takes slots [z chunk, (z + 1) chunk) and
  // leaves its unnormalised partial (running max, sum, P.V) for k_attention_merge
  const int jhi = part ? min(S, jlo + chunk) : S;
  float mrun = -INFINITY, lsum = 0.f;
  float acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.f;
  for (int j0 = jlo; j0 < jhi; j0 += G * KB) {
    if (j0 != jlo) load_batch(j0, jhi - 1);
    // scores s_j = q.k_j + slope * (j - qpos), summed across the group's L lanes;
    // slots before `first` are masked
    float sc[KB];
    float bmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int jj = j0 + u * G + g;
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) dot = fmaf(qv[t], kr[u].get(t), dot);
      for (int off = L >> 1; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
      if constexpr (kQ) dot *= ks[u];
      sc[u] = (jj < jhi && jj >= first) ? dot + slope * (float)(jj - qpos) : -INFINITY;
      bmax = fmaxf(bmax, sc[u]);
    }
    const float mnew = fmaxf(mrun, block_max<4>(bmax, red));
    // 0 while no slot has been visible (mrun = -inf): lsum and acc are still 0
    const float alpha = mrun == -INFINITY ? 0.f : __expf(mrun - mnew);
    lsum *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] *= alpha;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int jj = j0 + u * G + g;
      if (jj < jhi && jj >= first) {
        const float p = __expf(sc[u] - mnew);
        if (sub == 0) lsum += p;                  // each key counted once per group
        float pw = p;
        if constexpr (kQ) pw = p * vs[u];
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] = fmaf(pw, vr[u].get(t), acc[t]);
      }
    }
    mrun = mnew;
  }
  const float total = block_sum<4>(lsum, red);

#pragma unroll
  for (int t = 0; t < 8; ++t) pv[g * d + 8 * sub + t] = acc[t];
  __syncthreads();
  if (part) {
    // partial [m][h][z]: max, sum, then the d P.V sums (all relative to the max)
    float *pp = part + (((size_t)m * H + h) * gridDim.z + z) * (d + 2);
    if (tid == 0) { pp[0] = mrun; pp[1] = total; }
    for (int e = tid; e < d; e += 256) {
      float s = 0.f;
      for (int gg = 0; gg < G; ++gg) s += pv[gg * d + e];
      pp[2 + e] = s;
    }
    return;
  }
  // a query with no visible key (a left-pad position of the prompt) gets o = 0
  const float inv = qpos < first ? 0.f : 1.0f / total;
  for (int e = tid; e < d; e += 256) {
    float s = 0.f;
    for (int gg = 0; gg < G; ++gg) s += pv[gg * d + e];
    act_store(o, o_fmt, out0 + e, o_plane, s * inv);
  }
}

// Merge of the key-split partials of one (row, head) in split order: with M the largest
// partial max and w_z = exp(max_z - M) (0 for a split without visible keys), o =
// sum_z w_z PV_z / sum_z w_z sum_z -- the same softmax over all the keys; no visible
// key at all gives o = 0.
__global__ __launch_bounds__(128) void k_attention_merge(const float *__restrict__ part, int nsplit,
                                                         int H, int d, void *__restrict__ o,
                                                         int o_fmt, size_t o_plane) {
  const int mh = blockIdx.x;
  const float *pp = part + (size_t)mh * nsplit * (d + 2);
  float mx = -INFINITY;
  for (int z = 0; z < nsplit; ++z) mx = fmaxf(mx, pp[(size_t)z * (d + 2)]);
  float den = 0.f;
  for (int z = 0; z < nsplit; ++z) {
    const float mz = pp[(size_t)z * (d + 2)];
    if (mz != -INFINITY) den += __expf(mz - mx) * pp[(size_t)z * (d + 2) + 1];
  }
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  for (int e = threadIdx.x; e < d; e += 128) {
    float s = 0.f;
    for (int z = 0; z < nsplit; ++z) {
      const float mz = pp[(size_t)z * (d + 2)];
      if (mz != -INFINITY) s += __expf(mz - mx) * pp[(size_t)z * (d + 2) + 2 + e];
    }
    act_store(o, o_fmt, (size_t)mh * d + e, o_plane, s * inv);
  }
}

// Prompt pass: the same attention for the rows_per_seq query rows of each sequence,
// one 256-thread block per (sequence b, head h, chunk of 256 / (d/8) query rows).  Lane
// group g (d/8 lanes) owns query row r = chunk * rows_per_block + g at position
// qpos = pos_base + r; the block walks the keys from the sequence's first valid slot to
// its last row's position in tiles staged in LDS (each tile read once from the cache and
// shared by all the block's rows), 8 keys at a time per group: scores (masked above
// qpos: causal), their maximum, the rescale of the running sum and P.V accumulators,
// then exp and P.V -- the online form of the same float32 softmax.  A row with no
// visible key gets o = 0, as in k_attention.
constexpr int kPromptTileBytes = 16384;   // LDS per K (and per V) tile

template <typename TA>
__global__ __launch_bounds__(256) void k_attention_prompt(
    const float *__restrict__ q, const TA *__restrict__ kc, const TA *__restrict__ vc,
    const float *__restrict__ ksc, const float *__restrict__ vsc,
    const int *__restrict__ valid_len, void *__restrict__ o, int o_fmt, size_t o_plane, int H,
    int d, int max_len, int n_total, int head_off, int rows_per_seq, int pos_base,
    int prompt_len, int nchunk) {
  constexpr bool kQ = sizeof(TA) == 1;   // int8 cache with per-slot scales
  __shared__ __attribute__((aligned(16))) unsigned char ks_raw[kPromptTileBytes];
  __shared__ __attribute__((aligned(16))) unsigned char vs_raw[kPromptTileBytes];
  __shared__ float ks_tile[kQ ? 64 : 1], vs_tile[kQ ? 64 : 1];   // the tile's slot scales
  const TA *ks = (const TA *)ks_raw;
  const TA *vs = (const TA *)vs_raw;
  const int tid = threadIdx.x;
  const int b = blockIdx.x / nchunk, c = blockIdx.x - b * nchunk, h = blockIdx.y;
  const int L = d >> 3, QR = 256 / L;
  const int g = tid / L, sub = tid - g * L;
  const int r = c * QR + g;
  const bool active = r < rows_per_seq;
  const int qpos = pos_base + r;
  const int last = pos_base + min(rows_per_seq, c * QR + QR) - 1;   // block's last position
  const int vl_in = valid_len[b];
  const int vl = vl_in < 1 ? 1 : (vl_in > prompt_len ? prompt_len : vl_in);
  const int first = prompt_len - vl;
  const float slope = alibi_slope(n_total, head_off + h);
  const size_t head_base = ((size_t)b * H + h) * (size_t)max_len * d;
  const TA *kb = kc + head_base;
  const TA *vb = vc + head_base;
  const size_t scale_base = ((size_t)b * H + h) * (size_t)max_len;
  const size_t m = (size_t)b * rows_per_seq + (active ? r : 0);
  float qv[8];
  const float *qr = q + (m * H + h) * d + 8 * sub;
#pragma unroll
  for (int t = 0; t < 8; ++t) qv[t] = active ? qr[t] : 0.f;

  const int tile = min(64, kPromptTileBytes / (d * (int)sizeof(TA)));   // keys per tile
  const int piece_elems = 16 / (int)sizeof(TA);
  float mrun = -INFINITY, lsum = 0.f;
  float acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.f;
  for (int j0 = first; j0 <= last; j0 += tile) {
    const int cnt = min(tile, last + 1 - j0);
    __syncthreads();   // the previous tile has been read by every group
    const int pieces = cnt * d / piece_elems;
    for (int i = tid; i < pieces; i += 256) {
      ((u32x4 *)ks_raw)[i] = *(const u32x4 *)(kb + (size_t)j0 * d + (size_t)i * piece_elems);
      ((u32x4 *)vs_raw)[i] = *(const u32x4 *)(vb + (size_t)j0 * d + (size_t)i * piece_elems);
    }
    if constexpr (kQ) {
      if (tid < cnt) {
        ks_tile[tid] = ksc[scale_base + j0 + tid];
        vs_tile[tid] = vsc[scale_base + j0 + tid];
      }
    }
    __syncthreads();
    // every group runs every key of the tile (the shuffles stay convergent); keys
    // above the group's own position are masked
    for (int u0 = 0; u0 < cnt; u0 += 8) {
      float sc[8];
      float cmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int jj = u0 + u;
        float dot = 0.f;
        if (jj < cnt) {
          const TA *kp = ks + jj * d + 8 * sub;
#pragma unroll
          for (int t = 0; t < 8; ++t) dot = fmaf(qv[t], to_f<TA>(kp[t]), dot);
        }
        for (int off = L >> 1; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
        if constexpr (kQ) dot = jj < cnt ? dot * ks_tile[jj] : 0.f;
        const int j = j0 + jj;
        sc[u] = (jj < cnt && j <= qpos) ? dot + slope * (float)(j - qpos) : -INFINITY;
        cmax = fmaxf(cmax, sc[u]);
      }
      const float mnew = fmaxf(mrun, cmax);
      if (mnew == -INFINITY) continue;        // nothing visible to this row yet
      const float alpha = mrun == -INFINITY ? 0.f : __expf(mrun - mnew);
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] *= alpha;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (sc[u] == -INFINITY) continue;
        const float p = __expf(sc[u] - mnew);
        lsum += p;
        const TA *vp = vs + (u0 + u) * d + 8 * sub;
        float pw = p;
        if constexpr (kQ) pw = p * vs_tile[u0 + u];
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] = fmaf(pw, to_f<TA>(vp[t]), acc[t]);
      }
      mrun = mnew;
    }
  }
  if (!active) return;
  const float inv = (qpos < first || lsum == 0.f) ? 0.f : 1.0f / lsum;
  const size_t out0 = (m * H + h) * d + 8 * sub;
#pragma unroll
  for (int t = 0; t < 8; t += 4)
    act_store4(o, o_fmt, out0 + t, o_plane,
               make_float4(acc[t] * inv, acc[t + 1] * inv, acc[t + 2] * inv, acc[t + 3] * inv));
}

// Decode attention, one wave per (row, head) pair, for steps with many pairs (a large
// batch, or many heads): the same steps, in float32, as k_attention, with the lane
// groups of one wave taking the keys (G = 64 / (d / 8) keys per pass, KB passes per
// batch) and wave reductions only -- no block barrier, and four times as many pairs
// resident per CU as with one 256-thread block per pair.  Measured on MI355X with
// 14336 pairs of 17-115 slots (int8 cache, batch 128): the block kernel spent its time
// in each block's chain of dependent steps rather than in bandwidth.
// A lane's piece of a key / value row in k_attention_wave: EPL elements, and the keys
// per lane group per batch.  int8 codes: 16 per lane (one 16-byte load) for head dims
// of 16 and more.
struct KVRaw16I8 {
  u32x4 a;
  __device__ __forceinline__ void load(const int8_t *p) { a = *(const u32x4 *)p; }
  __device__ __forceinline__ float get(int t) const {
    return (float)(int8_t)(a[t >> 2] >> (8 * (t & 3)));
  }
};
template <typename TA, int EPL> struct WavePiece {
  using T = KVRaw<TA>;
  static constexpr int kKB = KeysPerBatch<TA>::value;
};
template <> struct WavePiece<int8_t, 16> {
  using T = KVRaw16I8;
  static constexpr int kKB = 8;
};

template <typename TA, int EPL>
__global__ __launch_bounds__(256) void k_attention_wave(
    const float *__restrict__ q, const TA *__restrict__ kc, const TA *__restrict__ vc,
    const float *__restrict__ ksc, const float *__restrict__ vsc,
    const int *__restrict__ valid_len, void *__restrict__ o, int o_fmt, size_t o_plane, int H,
    int d, int max_len, int n_total, int head_off, int pairs, int pos_base,
    const int *__restrict__ pos_dev, int prompt_len) {
  constexpr int KB = WavePiece<TA, EPL>::kKB;
  using Raw = typename WavePiece<TA, EPL>::T;
  constexpr bool kQ = sizeof(TA) == 1;   // int8 cache with per-slot scales
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (pair >= pairs) return;   // a whole wave; nothing below waits for other waves
  const int m = pair / H, h = pair - m * H;   // decode: row m is sequence m
  const int qpos = min(pos_dev ? *pos_dev : pos_base, max_len - 1);
  const int vl_in = valid_len[m];
  const int S = qpos + 1;
  const float slope = alibi_slope(n_total, head_off + h);
  const size_t head_base = ((size_t)m * H + h) * (size_t)max_len * d;
  const TA *kb = kc + head_base;
  const TA *vb = vc + head_base;
  const size_t scale_base = ((size_t)m * H + h) * (size_t)max_len;
  const float *qr = q + ((size_t)m * H + h) * d;

  // lane group g (L = d / EPL lanes) takes slots j = g (mod G) of each batch; lane `sub`
  // owns dims [EPL sub, EPL sub + EPL)
  const int L = d / EPL;
  const int G = 64 / L;
  const int g = lane / L, sub = lane - g * L;
  float qv[EPL];
#pragma unroll
  for (int t = 0; t < EPL; ++t) qv[t] = qr[EPL * sub + t];
  const int vl = vl_in < 1 ? 1 : (vl_in > prompt_len ? prompt_len : vl_in);
  const int first = prompt_len - vl;

  float mrun = -INFINITY, lsum = 0.f;
  float acc[EPL];
#pragma unroll
  for (int t = 0; t < EPL; ++t) acc[t] = 0.f;
  for (int j0 = 0; j0 < S; j0 += G * KB) {
    // slots past the end load slot S - 1 (written, masked below): no branch around loads
    Raw kr[KB], vr[KB];
    float ks[KB], vs[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int jj = min(j0 + u * G + g, S - 1);
      kr[u].load(kb + (size_t)jj * d + EPL * sub);
      vr[u].load(vb + (size_t)jj * d + EPL * sub);
      if constexpr (kQ) {
        ks[u] = ksc[scale_base + jj];
        vs[u] = vsc[scale_base + jj];
      }
    }
    float sc[KB];
    float bmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int jj = j0 + u * G + g;
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < EPL; ++t) dot = fmaf(qv[t], kr[u].get(t), dot);
      for (int off = L >> 1; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
      if constexpr (kQ) dot *= ks[u];
      sc[u] = (jj < S && jj >= first) ? dot + slope * (float)(jj - qpos) : -INFINITY;
      bmax = fmaxf(bmax, sc[u]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, off, 64));
    const float mnew = fmaxf(mrun, bmax);
    // 0 while no slot has been visible (mrun = -inf): lsum and acc are still 0
    const float alpha = mrun == -INFINITY ? 0.f : __expf(mrun - mnew);
    lsum *= alpha;
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[t] *= alpha;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int jj = j0 + u * G + g;
      if (jj < S && jj >= first) {
        const float p = __expf(sc[u] - mnew);
        if (sub == 0) lsum += p;                  // each key counted once per group
        float pw = p;
        if constexpr (kQ) pw = p * vs[u];
#pragma unroll
        for (int t = 0; t < EPL; ++t) acc[t] = fmaf(pw, vr[u].get(t), acc[t]);
      }
    }
    mrun = mnew;
  }
  // sum the groups' partial P.V (lanes with the same `sub`) and the key counts
#pragma unroll
  for (int off = L; off < 64; off <<= 1)
#pragma unroll
    for (int t = 0; t < EPL; ++t) acc[t] += __shfl_xor(acc[t], off, 64);
  const float total = wave_sum(lsum);
  if (g == 0) {
    // a query with no visible key gets o = 0
    const float inv = qpos < first ? 0.f : 1.0f / total;
    const size_t out0 = ((size_t)m * H + h) * d + EPL * sub;
#pragma unroll
    for (int t = 0; t < EPL; t += 4)
      act_store4(o, o_fmt, out0 + t, o_plane,
                 make_float4(acc[t] * inv, acc[t + 1] * inv, acc[t + 2] * inv, acc[t + 3] * inv));
  }
}

template <typename TA>
static void launch_attention_t(const float *q, const void *kc, const void *vc, const float *ksc,
                               const float *vsc, const int *valid_len, void *o, int o_fmt,
                               size_t o_plane, int rows,
                               int H, int d, int max_len, int n_total, int head_off,
                               int rows_per_seq, int pos_base, const int *pos_dev,
                               int prompt_len, bool prompt_kernel, int nchunk, int nsplit,
                               float *part, hipStream_t st) {
  if (prompt_kernel) {
    const dim3 grid((unsigned)(rows / rows_per_seq * nchunk), H), block(256);
    hipLaunchKernelGGL(k_attention_prompt<TA>, grid, block, 0, st, q, (const TA *)kc,
                       (const TA *)vc, ksc, vsc, valid_len, o, o_fmt, o_plane, H, d, max_len,
                       n_total,
                       head_off, rows_per_seq, pos_base, prompt_len, nchunk);
  } else if (nsplit == 1 && rows_per_seq == 1 && (long)rows * H >= kAttnWavePairs) {
    const int pairs = rows * H;
    const dim3 grid((unsigned)((pairs + 3) / 4)), block(256);
    bool wide = false;
    if constexpr (sizeof(TA) == 1) {
      wide = d >= 16;
      if (wide)
        hipLaunchKernelGGL((k_attention_wave<TA, 16>), grid, block, 0, st, q, (const TA *)kc,
                           (const TA *)vc, ksc, vsc, valid_len, o, o_fmt, o_plane, H, d,
                           max_len, n_total, head_off, pairs, pos_base, pos_dev, prompt_len);
    }
    if (!wide)
      hipLaunchKernelGGL((k_attention_wave<TA, 8>), grid, block, 0, st, q, (const TA *)kc,
                         (const TA *)vc, ksc, vsc, valid_len, o, o_fmt, o_plane, H, d, max_len,
                         n_total, head_off, pairs, pos_base, pos_dev, prompt_len);
  } else {
    const int chunk = (max_len + nsplit - 1) / nsplit;
    const dim3 grid(rows, H, nsplit), block(256);
    hipLaunchKernelGGL(k_attention<TA>, grid, block, 0, st, q, (const TA *)kc, (const TA *)vc,
                       ksc, vsc, valid_len, o, o_fmt, o_plane, H, d, max_len, n_total, head_off,
                       rows_per_seq, pos_base, pos_dev, prompt_len, chunk,
                       nsplit > 1 ? part : nullptr);
    if (nsplit > 1)
      hipLaunchKernelGGL(k_attention_merge, dim3(rows * H), dim3(128), 0, st, part, nsplit, H, d,
                         o, o_fmt, o_plane);
  }
}

// Key splits of the decode attention: enough (row, head, split) blocks to spread a long
// cache over the chip -- at most kAttnSplitBlocks blocks in all, at least 256 slots of
// the cache's capacity per split, at most kAttnMaxSplits splits (1: no split).  The
// capacity, not the current length, sets it, so a captured step replays unchanged.
int attention_splits(int rows, int H, int max_len, int rows_per_seq) {
  if (rows_per_seq != 1) return 1;
  const long heads = (long)rows * H;
  if (heads >= kAttnSplitBlocks) return 1;
  const long by_blocks = kAttnSplitBlocks / heads;
  const long by_len = (max_len + 255) / 256;
  return (int)std::max(1l, std::min({by_blocks, by_len, (long)kAttnMaxSplits}));
}

hipError_t launch_attention(int kv_fmt, const float *q, const void *kc, const void *vc,
                            const float *ksc, const float *vsc,
                            const int *valid_len, void *o, int o_fmt, int rows, int H, int d,
                            int max_len, int n_total, int head_off, int rows_per_seq,
                            int pos_base, const int *pos_dev, int prompt_len, float *part,
                            hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int nsplit = attention_splits(rows, H, max_len, rows_per_seq);
  if (nsplit > 1 && !part) return hipErrorInvalidValue;
  const size_t o_plane = (size_t)rows * H * d;
  // The prompt kernel when it still fills the chip (>= 256 blocks); a short prompt of
  // one or a few sequences keeps one block per (row, head), which spreads its few keys
  // over more CUs (measured, 176B share batch 1: 14 blocks took 9.7 us, 224 took 6.0).
  const int QR = 256 / (d >> 3);
  const int nchunk = (rows_per_seq + QR - 1) / QR;
  const long prompt_blocks = (long)(rows / max(rows_per_seq, 1)) * nchunk * H;
  // (its tiles are copied in 16-byte pieces: a key must be a whole number of them)
  const int elem = kv_fmt == AF_F32 ? 4 : (kv_fmt == AF_I8 ? 1 : 2);
  const bool prompt_kernel =
      rows_per_seq > 1 && !pos_dev && prompt_blocks >= 256 && (d * elem) % 16 == 0;
  if (kv_fmt == AF_I8 && (!ksc || !vsc)) return hipErrorInvalidValue;
#define BL_ATTN(TA)                                                                        \
  launch_attention_t<TA>(q, kc, vc, ksc, vsc, valid_len, o, o_fmt, o_plane, rows, H, d,     \
                         max_len, n_total, head_off, rows_per_seq, pos_base, pos_dev,       \
                         prompt_len, prompt_kernel, nchunk, nsplit, part, st)
  if (kv_fmt == AF_I8) BL_ATTN(int8_t);
  else if (kv_fmt == AF_F32) BL_ATTN(float);
  else if (kv_fmt == AF_F16) BL_ATTN(f16_t);
  else BL_ATTN(bf16_t);
#undef BL_ATTN
  return hipGetLastError();
}

// src [batch][H][n_new][d] -> cache [layer][max_batch][H][max_len][d] slots pos..pos+n_new-1
template <typename TA>
__global__ __launch_bounds__(256) void k_kv_append(const TA *__restrict__ sk,
                                                   const TA *__restrict__ sv,
                                                   TA *__restrict__ ck, TA *__restrict__ cv,
                                                   int batch, int H, int n_new, int d,
                                                   int max_len, int pos) {
  const size_t total = (size_t)batch * H * n_new * d;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (size_t)gridDim.x * 256) {
    const int e = (int)(i % d);
    size_t r = i / d;
    const int t = (int)(r % n_new);
    r /= n_new;  // r = b * H + h
    const size_t dst = (r * max_len + pos + t) * d + e;
    ck[dst] = sk[i];
    cv[dst] = sv[i];
  }
}

hipError_t launch_kv_append(bool f32, const void *k, const void *v, void *ck, void *cv,
                            int batch, int H, int n_new, int d, int max_len, int pos,
                            hipStream_t st) {
  const size_t total = (size_t)batch * H * n_new * d;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  if (f32)
    hipLaunchKernelGGL(k_kv_append<float>, dim3(blocks), dim3(256), 0, st, (const float *)k,
                       (const float *)v, (float *)ck, (float *)cv, batch, H, n_new, d, max_len,
                       pos);
  else
    hipLaunchKernelGGL(k_kv_append<bf16_t>, dim3(blocks), dim3(256), 0, st, (const bf16_t *)k,
                       (const bf16_t *)v, (bf16_t *)ck, (bf16_t *)cv, batch, H, n_new, d,
                       max_len, pos);
  return hipGetLastError();
}

// int8 KV cache: new keys and values (float32) -> codes in their slots plus one float32
// scale per (row, head, slot) each for keys and values (row_quant over the head's d
// values).  One wave per (row b, new token t, head h, key or value); token t of row b
// goes to slot pos + t (pos = *pos_dev when set, else pos_base); slots at or past
// max_len are not written.  The sources are read through strides, so that both the QKV
// epilogue's staging buffer [rows][H][2][d] and kv_cache_append's [batch][H][n_new][d]
// inputs serve.
__global__ __launch_bounds__(256) void k_kv_quant(KvQuantArgs a) {
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (w >= (long)a.batch * a.n * a.H * 2) return;   // uniform per wave
  const int kind = (int)(w & 1);
  long r = w >> 1;
  const int h = (int)(r % a.H);
  r /= a.H;
  const int t = (int)(r % a.n), b = (int)(r / a.n);
  const float *src = (kind ? a.v : a.k) + b * a.sb + t * a.st + h * a.sh;
  float v[4];
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < a.d ? src[c] : 0.f;
    am = fmaxf(am, fabsf(v[i]));
  }
  const RowQuant rq = row_quant(wave_max(am));
  const int pos = (a.pos_dev ? *a.pos_dev : a.pos_base) + t;
  if (pos >= a.max_len) return;
  const size_t slot = ((size_t)b * a.H + h) * a.max_len + pos;
  int8_t *dst = (kind ? a.vc : a.kc) + slot * a.d;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    if (c < a.d) dst[c] = (int8_t)quant_code(v[i], rq.inv);
  }
  if (lane == 0) (kind ? a.vs : a.ks)[slot] = rq.scale;
}

hipError_t launch_kv_quant(const KvQuantArgs &a, hipStream_t st) {
  const long waves = (long)a.batch * a.n * a.H * 2;
  if (waves == 0) return hipSuccess;
  if (a.d > 256 || a.d <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_kv_quant, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// In-place compaction of the KV cache ("Hugging Face BLOOM Inference Optimization",
// Webserver Architecture and Request Handling: finished requests are extracted from
// the running batch): destination row j0 + i takes source row rows[i] (rows strictly
// increasing, rows[i] >= j0 + i), slots [0, len), keys and values, every layer and head.
// One block per (layer, head) walks its destination rows in increasing order; every
// thread copies the same 16-byte offsets of each row, so a row is read (as a source)
// before the same thread overwrites it (as a later destination) and no barrier is
// needed; blocks touch disjoint (layer, head) ranges.
struct KvRows {
  int src[kKvCompactChunk];
};

__global__ __launch_bounds__(256) void k_kv_compact(unsigned char *__restrict__ kc,
                                                    unsigned char *__restrict__ vc,
                                                    size_t layer_stride, size_t row_stride,
                                                    size_t head_stride, size_t row_bytes,
                                                    KvRows rows, int n, int j0) {
  const size_t base = blockIdx.x * layer_stride + blockIdx.y * head_stride;
  const size_t pieces = row_bytes / 16;
  const size_t tail = (row_bytes - 16 * pieces) / 4;   // trailing dwords
  for (int i = 0; i < n; ++i) {
    const int src = rows.src[i], dst = j0 + i;
    if (src == dst) continue;
    const size_t so = base + (size_t)src * row_stride, dof = base + (size_t)dst * row_stride;
    for (size_t p = threadIdx.x; p < pieces; p += 256) {
      const u32x4 a = *(const u32x4 *)(kc + so + 16 * p);
      const u32x4 b = *(const u32x4 *)(vc + so + 16 * p);
      *(u32x4 *)(kc + dof + 16 * p) = a;
      *(u32x4 *)(vc + dof + 16 * p) = b;
    }
    if (threadIdx.x < tail) {
      const size_t o = 16 * pieces + 4 * threadIdx.x;
      const uint32_t a = *(const uint32_t *)(kc + so + o);
      const uint32_t b = *(const uint32_t *)(vc + so + o);
      *(uint32_t *)(kc + dof + o) = a;
      *(uint32_t *)(vc + dof + o) = b;
    }
  }
}

hipError_t launch_kv_compact(void *kc, void *vc, int n_layer, int H, int max_batch, int max_len,
                             int d, size_t act, int len, const int *rows, int n_keep,
                             hipStream_t st) {
  const size_t head_stride = (size_t)max_len * d * act;
  const size_t row_stride = (size_t)H * head_stride;
  const size_t layer_stride = (size_t)max_batch * row_stride;
  const size_t row_bytes = (size_t)len * d * act;
  if (row_bytes == 0 || n_keep <= 0) return hipSuccess;
  for (int j0 = 0; j0 < n_keep; j0 += kKvCompactChunk) {
    KvRows r{};
    const int n = std::min(kKvCompactChunk, n_keep - j0);
    for (int i = 0; i < n; ++i) r.src[i] = rows[j0 + i];
    hipLaunchKernelGGL(k_kv_compact, dim3(n_layer, H), dim3(256), 0, st, (unsigned char *)kc,
                       (unsigned char *)vc, layer_stride, row_stride, head_stride, row_bytes, r,
                       n, j0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bl
