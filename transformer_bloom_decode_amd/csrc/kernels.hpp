// Host-side launch entry points of the gfx950 kernels (used by the C ABI layer).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

// Events for the launch timer.  When set, the next BL_LAUNCH goes through
// hipExtLaunchKernelGGL, whose start/stop events are timestamped by the kernel's own
// dispatch packet (the same timestamps a kernel-trace profiler reads, with no extra
// marker packets in the stream), and the events are then cleared.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchEvents g_launch_events;

#define BL_LAUNCH(kernel, grid, block, shmem, stream, ...)                                    \
  do {                                                                                       \
    if (::bl::g_launch_events.start) {                                                       \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ::bl::g_launch_events.start, \
                            ::bl::g_launch_events.stop, 0, __VA_ARGS__);                     \
      ::bl::g_launch_events = ::bl::LaunchEvents{};                                         \
    } else {                                                                                 \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                   \
    }                                                                                        \
  } while (0)

struct EpiParams;

enum WeightType : int { WT_F32 = 0, WT_BF16 = 1, WT_INT8 = 2 };
enum LinearKind : int { LIN_F32 = 0, LIN_VALU = 3, LIN_LG = 4 };

// Vector-ALU GEMV: used for up to kValuMaxRows activation rows, 4 waves per block,
// 1 or 2 weight rows per wave.
constexpr int kValuMaxRows = 4;
// Columns of the LM-head partial-argmax buffer per activation row: one partial per
// kLmRowsPerPartial weight rows, the finest split any LM-head kernel uses.
constexpr int kLmRowsPerPartial = 4;
inline int lm_partial_stride(int vocab) {
  return (vocab + kLmRowsPerPartial - 1) / kLmRowsPerPartial;
}


// Minimum size of the split-K partial buffer (float32 elements) and the cap any one
// linear of the direct-to-LDS GEMM may use.
constexpr long kPartialCapFloats = 8l << 20;
constexpr long kLgPartialCapFloats = 48l << 20;

struct LinearPlan {
  int kind;
  int M, N, K;
  int mt;        // VALU: activation rows (1, 2, 4)
  int vr, vu;    // VALU: weight rows per wave, 16-byte pieces per row issued per batch
  bool vdb;      // VALU: double-buffered batches
  int ks;        // VALU: waves per weight row (1, or 2: the row's K range split in halves)
  int lg;        // LG: tile configuration (LgTile in gemm.hip)
  int grid_x, grid_y;
  int splits;    // K splits (> 1: partial sums + reduction kernel)
  int x_fmt;     // VALU: activation storage (ActFmt: AF_BF16, AF_F32 or AF_F16)
  int xs;        // LG: activation planes (1: bf16; 2: bf16 hi + lo planes of float32 values)
  bool x8;       // LG: int8 activation codes against int8 weights (W8A8)
  bool xh;       // LG: fp16 activations on the fp16 MFMA
  bool q8;       // the activations are int8-quantised rows (AF_I8)
};

// Vector-ALU GEMV (gemv.hip): plan for M <= kValuMaxRows rows, and its launch.
LinearPlan plan_valu(int wdtype, int M, int N, int K);
hipError_t launch_valu(int wdtype, const LinearPlan &p, const void *X, const void *W,
                       const EpiParams &ep, hipStream_t st);
// The one-row GEMVs of a folded LayerNorm (consumer: ep.ln_stats, ep.ln_cd; residual
// producer: ep.fold_g, fold_u, fold_stats): supported for this plan?
bool ln_fold_supported(int wdtype, const LinearPlan &p, const EpiParams &ep);
// LayerNorm fold vectors of one linear: c[n] = sum_k W[n][k] g[k], d[n] = sum_k W[n][k]
// b[k] + bias[n] (bf16 W [N][K], g, b [K], bias [N] nullable).
hipError_t launch_ln_fold(const void *W, const void *g, const void *b, const void *bias, int N,
                          int K, float *c, float *d, hipStream_t st);
// One-row GEMV whose prologue is the LayerNorm of the float32 row x (gamma g, beta b,
// bf16): out = epilogue(LN(x) . W^T); bf16 or int8 weights, K a multiple of 16 up to
// 4096 (gemv_ln_supported).
bool gemv_ln_supported(int wdtype, int M, int K);
hipError_t launch_gemv_ln(int wdtype, int x_fmt, int N, int K, const float *x, const void *g,
                          const void *b, float eps, const void *W, const EpiParams &ep,
                          hipStream_t st);
// act: the model's activation type (ActFmt AF_BF16, AF_F32, AF_F16 or, int8 weights
// only, AF_I8).  The vector-ALU GEMV reads activations in that type (int8 ones as codes,
// the row scales applied by the epilogue); the MFMA GEMM reads bf16, fp16 (on the fp16 MFMA),
// for float32 activations the two bf16 planes hi + lo, for int8 ones the codes (the
// epilogue multiplies by EpiParams::xscale).
LinearPlan plan_linear(int wdtype, int M, int N, int K, bool argmax, int act);
// Storage format (ActFmt) of the activations a linear of this plan reads.
int plan_x_fmt(const LinearPlan &p);
// (max, index) partials per activation row an argmax-mode launch of the plan writes.
int argmax_partials_per_row(const LinearPlan &p);
// Bytes of split-K partials the plan needs (0 without split-K).
size_t linear_partial_bytes(const LinearPlan &p);
// splitk_epilogue = false leaves a K-split launch's partials for the caller to reduce.
hipError_t launch_linear(int wdtype, const LinearPlan &p, const void *X, const void *W,
                         float *partial, const EpiParams &ep, hipStream_t st,
                         bool splitk_epilogue = true);
hipError_t launch_argmax_merge(const float *val, const int *idx, int stride, int nblk, int rows,
                               int *out, hipStream_t st);

hipError_t launch_alibi_softmax(const void *scores, bool in_bf16, const int *valid_len,
                                void *probs, bool out_bf16, int B, int H, int Q, int K,
                                int n_total, int head_off, hipStream_t stream);

// zero (nullable): nzero 64-bit words that block 0 also clears (the folded LayerNorms'
// accumulators of the pass)
hipError_t launch_embed(bool f32, const int *tokens, const void *embed, const void *g,
                        const void *b, float *x, int rows, int h, int vocab, int do_ln, float eps,
                        unsigned long long *zero, int nzero, hipStream_t stream);
// Split-K partials of a bf16 linear [splits][rows][h] -> x += sum * scale + bias, then
// out = LN(x) (bf16); only for splitk_resid_ln_supported(h, splits).
bool splitk_resid_ln_supported(int h, int splits);
// out is written in format fmt (ActFmt; for AF_BF16X2 the lo plane follows rows * h
// elements after the hi plane).
// xscale (nullable): per-row scales of int8 activations, applied to the partials' sum.
hipError_t launch_splitk_resid_ln(const float *partial, int splits, int rows, const float *xscale,
                                  const void *scale, const void *bias, float *x, const void *g,
                                  const void *b, void *out, int fmt, int h, float eps,
                                  hipStream_t stream);
// float32 rows [rows][K] -> per-row int8 (fmt AF_I8: scales rows * K bytes after the
// codes).
hipError_t launch_quant_rows(const float *in, int rows, int K, void *out, int fmt,
                             hipStream_t stream);
hipError_t launch_layernorm(bool f32, const float *x, int in_step, int in_off, const void *g,
                            const void *b, void *out, int fmt, float *out_f32, int rows, int h,
                            float eps, hipStream_t stream);

// kv_fmt: cache elements (AF_F32, AF_BF16 or AF_F16); o written in format o_fmt (ActFmt,
// lo plane rows * H * d elements after the hi plane).  With pos_dev set, the query
// position is read from device memory and clamped so that no slot at or past max_len is
// read.
// kv_fmt AF_I8: int8 codes with float32 scales ksc / vsc [max_batch][H][max_len] of this
// layer (else the scale pointers are unused).  A decode step over a long cache splits
// the keys over attention_splits(...) blocks per (row, head); part then holds
// rows * H * splits * (d + 2) floats (at most kAttnSplitBlocks * (d + 2)).
constexpr int kAttnSplitBlocks = 1024;
// Decode steps with at least this many (row, head) pairs and no key split run one wave
// per pair (k_attention_wave) instead of one block.
constexpr int kAttnWavePairs = 1024;
constexpr int kAttnMaxSplits = 16;
int attention_splits(int rows, int H, int max_len, int rows_per_seq);
hipError_t launch_attention(int kv_fmt, const float *q, const void *kc, const void *vc,
                            const float *ksc, const float *vsc, const int *valid_len, void *o, int o_fmt, int rows, int H, int d,
                            int max_len, int n_total, int head_off, int rows_per_seq,
                            int pos_base, const int *pos_dev, int prompt_len, float *part,
                            hipStream_t st);

// Per-row stop rule of the generation loop: done[i] set once row i has finished (its
// eos_id token emitted, or max_new[i] tokens); finished rows emit pad_id; out_len[i]
// (nullable) counts a row's tokens.  eos_id < 0: none; max_new nullable: no limit.
struct GenControl {
  int *done;
  int eos_id;
  int pad_id;
  const int *max_new;
  int *out_len;
};

// Bookkeeping of a generation step (state[0] = KV position, state[1] = index of the
// step being recorded): ids[step][b] and cur[b] = next[b] (pad_id once row b has
// finished), hout[step] = hfix (if hout), then state advances by one step.
hipError_t launch_gen_init(int *state, int pos, int step, int *done, int batch, hipStream_t st);
hipError_t launch_gen_record(const int *next, int *cur, int *ids, const float *hfix, float *hout,
                             int *state, int batch, int hidden, const GenControl &gc,
                             hipStream_t st);
// int8 KV cache writes (k_kv_quant): source element c of (row b, new token t, head h) is
// k[b * sb + t * st + h * sh + c] (v likewise); it goes to slot pos + t of the layer's
// int8 cache kc / vc [max_batch][H][max_len][d] and the slot's scale to ks / vs
// [max_batch][H][max_len]; pos = *pos_dev if set, else pos_base.
struct KvQuantArgs {
  const float *k, *v;
  long sb, st, sh;
  int batch, n, H, d;
  int8_t *kc, *vc;
  float *ks, *vs;
  int max_len, pos_base;
  const int *pos_dev;
};
hipError_t launch_kv_quant(const KvQuantArgs &a, hipStream_t st);
// KV-cache compaction: rows[i] -> row i (strictly increasing sources), slots [0, len),
// all layers and heads, in place (len * d * act bytes per row and head, a multiple of
// 4).  Sources are passed by value in chunks.
constexpr int kKvCompactChunk = 256;
hipError_t launch_kv_compact(void *kc, void *vc, int n_layer, int H, int max_batch, int max_len,
                             int d, size_t act, int len, const int *rows, int n_keep,
                             hipStream_t st);
// Per-row temperature + nucleus (top-p) sampling of float32 logits [batch][V] with one
// uniform number per row (sample.hip); temperature <= 0 is greedy.  `ws` holds
// sample_workspace_bytes(batch, V) bytes of partial results.
size_t sample_workspace_bytes(int batch, int vocab);
// With step_dev set, row b draws with uniform[*step_dev * batch + b] (a generation loop's
// step index in device memory), else with uniform[b].
hipError_t launch_sample_rows(const float *logits, int batch, int V, const float *temperature,
                              const float *top_p, const float *uniform, int *out, void *ws,
                              hipStream_t st, const int *step_dev = nullptr);
// The same sampling with the library's own device scratch array of kSampleScratchBytes
// per GPU instead of a caller workspace (no allocation); hipErrorInvalidValue when the
// rows need more than that.  Calls overlapping on one GPU share the array and race.
constexpr long kSampleScratchBytes = 16l << 20;
hipError_t launch_sample_rows_static(const float *logits, int batch, int V,
                                     const float *temperature, const float *top_p,
                                     const float *uniform, int *out, hipStream_t st);
// Device address of this GPU's sample scratch array (looked up once per device).
hipError_t sample_scratch_ptr(void **out);
// y = the n float32 values x in activation format fmt (ActFmt; two planes: the lo plane
// n elements after the hi plane).
hipError_t launch_f32_to_act(const float *x, void *y, int fmt, size_t n, hipStream_t st);
// Device KV length: *len = set when set >= 0, else *len = min(*len + add, max_len).
hipError_t launch_len_update(int *len, int set, int add, int max_len, hipStream_t st);
// Every tensor of the model in storage form from the counter-hash generator (bloom.h,
// bloom_init_weights): one launch per tensor.
struct InitTensor {
  void *out;
  size_t n;
  uint64_t key;     // SplitMix64(seed << 32 ^ tensor id)
  int op;           // 0 normal, 1 int8, 2 fp16 row scale
  int kind;         // normal: 0 float32, 1 bf16
  float mean, scale;
};
hipError_t launch_init_tensor(const InitTensor &t, hipStream_t st);
hipError_t launch_kv_append(bool f32, const void *k, const void *v, void *ck, void *cv,
                            int batch, int H, int n_new, int d, int max_len, int pos,
                            hipStream_t st);

}  // namespace bl
