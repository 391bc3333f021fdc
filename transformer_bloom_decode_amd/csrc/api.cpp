// C ABI of the BLOOM decode library: argument validation, workspace carve-up and the
// launch sequence of one forward pass (prompt pass or one generation step).
//
// Launch sequence for M = batch * tokens_per_row rows ("DeepSpeed Inference ...",
// Section III.D fused groups; "Incredibly Fast BLOOM Inference ...", Benchmark
// Environment for the greedy, KV-cached loop):
//   embed (+ embedding LayerNorm)                                    -> x (fp32)
//   per layer: LayerNorm1 -> QKV linear (+bias; q scaled to fp32, k/v into the cache)
//              -> attention -> dense linear (+bias, += x) -> LayerNorm2
//              -> up linear (+bias, tanh GeLU) -> down linear (+bias, += x)
//   final LayerNorm of each row's last position -> LM head (tied embedding) with a
//   per-tile argmax -> argmax merge -> next token ids.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/bloom.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace bl;

namespace {

constexpr int kMaxLen = 1 << 20;  // KV slots per row (positions are int32 throughout)

// HIP error behind the last BLOOM_EHIP returned on this thread.
thread_local hipError_t g_last_hip_error = hipSuccess;

// hipGetLastError() reports the last error of *any* runtime call on the thread (e.g. a
// hipErrorNotReady from an event query made by the caller's allocator), so each entry
// point clears it before launching and checks only its own launches.
void clear_stale_hip_error() { (void)hipGetLastError(); }

int hip_fail(hipError_t e) {
  g_last_hip_error = e;
  return BLOOM_EHIP;
}

struct WsPlan {
  size_t gen, cur, nxt, hfix, done;   // generation loop state (same offsets for every pass)
  size_t x, xa, q, o, u, af, amv, ami, part, total;
  size_t stg;   // int8 activations: float32 attention / GeLU rows before quantisation
  size_t kvs;   // int8 KV cache: float32 new keys and values [rows][H][2][d]
  size_t attn;  // key-split attention partials
  size_t stats; // folded LayerNorms: [n_layer][LN1, LN2][kStatWords] sum accumulators
  int lm_blocks;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int dtype_fmt(int dt) {
  switch (dt) {
    case BLOOM_F32: return AF_F32;
    case BLOOM_F16: return AF_F16;
    case BLOOM_INT8_ROWSCALE: return AF_I8;
    default: return AF_BF16;
  }
}
// The activation type as a storage format (ActFmt): AF_BF16, AF_F32, AF_F16 or AF_I8.
int act_fmt(const bloom_config *c) { return dtype_fmt(c->act_dtype); }
bool act_q8(const bloom_config *c) { return act_fmt(c) == AF_I8; }
// The final LayerNorm's output is never quantised: with int8 activations the LM head
// reads it as float32 activations.
int lm_act_fmt(const bloom_config *c) { return act_q8(c) ? AF_F32 : act_fmt(c); }
// Bytes per activation element in the workspace: bf16 2; float32 / fp16 activations 4
// (float32, fp16, or the two bf16 planes the MFMA GEMM reads); int8 4 (one code byte is
// used; the same regions hold the float32 final-LayerNorm rows the LM head reads) plus
// one float32 scale per row.
int act_bytes(const bloom_config *c) { return act_fmt(c) == AF_BF16 ? 2 : 4; }
size_t act_region(const bloom_config *c, size_t rows, size_t n) {
  return rows * n * act_bytes(c) + (act_q8(c) ? rows * 4 : 0);
}
int kv_fmt(const bloom_config *c) { return dtype_fmt(c->kv_dtype); }
bool kv_q8(const bloom_config *c) { return kv_fmt(c) == AF_I8; }
int kv_bytes(const bloom_config *c) {
  const int f = kv_fmt(c);
  return f == AF_F32 ? 4 : (f == AF_I8 ? 1 : 2);
}
int wtype(const bloom_config *c) {
  return c->weight_dtype == BLOOM_F32 ? WT_F32 : (c->weight_dtype == BLOOM_BF16 ? WT_BF16 : WT_INT8);
}
int lm_blocks(const bloom_config *c) {
  return c->weight_dtype == BLOOM_F32 ? (c->vocab + 255) / 256 : lm_partial_stride(c->vocab);
}

WsPlan plan_ws(const bloom_config *c, int batch, int tokens_per_row) {
  WsPlan p{};
  const size_t M = (size_t)batch * (size_t)std::max(tokens_per_row, 1);
  const size_t act = act_bytes(c);
  const size_t hd = (size_t)c->n_head_local * c->head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t o = off; off += align256(bytes); return o; };
  p.gen = take(2 * sizeof(int));
  p.cur = take((size_t)batch * sizeof(int));
  p.nxt = take((size_t)batch * sizeof(int));
  p.hfix = take((size_t)batch * c->hidden * sizeof(float));
  p.done = take((size_t)batch * sizeof(int));
  p.x = take(M * c->hidden * 4);
  p.xa = take(act_region(c, M, c->hidden));
  p.q = take(M * hd * 4);
  p.o = take(act_region(c, M, hd));
  p.u = take(act_region(c, M, (size_t)c->ffn));
  p.af = take((size_t)batch * c->hidden * act);
  p.stg = act_q8(c) ? take(M * std::max(hd, (size_t)c->ffn) * 4) : 0;
  p.kvs = kv_q8(c) ? take(M * hd * 2 * 4) : 0;
  p.attn = take((size_t)kAttnSplitBlocks * (c->head_dim + 2) * sizeof(float));
  p.stats = take((size_t)c->n_layer * 2 * kStatWords * sizeof(unsigned long long));
  p.lm_blocks = lm_blocks(c);
  p.amv = take((size_t)batch * p.lm_blocks * 4);
  p.ami = take((size_t)batch * p.lm_blocks * 4);
  size_t part = c->weight_dtype == BLOOM_F32 ? 0 : (size_t)kPartialCapFloats * 4;
  if (c->weight_dtype != BLOOM_F32) {
    // the prompt-pass GEMM may split K over more partials than the other kernels
    const int wdt = wtype(c);
    const int hd_ = c->n_head_local * c->head_dim;
    const int dims[4][2] = {{3 * hd_, c->hidden}, {c->hidden, hd_}, {c->ffn, c->hidden},
                            {c->hidden, c->ffn}};
    for (const int mrows : {(int)M, batch})
      for (const auto &nk : dims)
        part = std::max(part, linear_partial_bytes(
                                  plan_linear(wdt, mrows, nk[0], nk[1], false, act_fmt(c))));
  }
  p.part = take(part);
  p.total = off;
  return p;
}

bool pow2_dim(int d) { return d >= 8 && d <= 256 && (d & (d - 1)) == 0; }

int check_config(const bloom_config *c) {
  if (!c) return BLOOM_EINVAL;
  if (c->n_layer <= 0 || c->hidden <= 0 || c->n_head_total <= 0 || c->n_head_local <= 0 ||
      c->head_dim <= 0 || c->ffn <= 0 || c->vocab <= 0 || c->head_offset < 0)
    return BLOOM_EINVAL;
  if (c->head_offset + c->n_head_local > c->n_head_total) return BLOOM_EINVAL;
  if (!pow2_dim(c->head_dim)) return BLOOM_EINVAL;
  if (!(c->ln_eps >= 0.f)) return BLOOM_EINVAL;
  if (c->weight_dtype != BLOOM_F32 && c->weight_dtype != BLOOM_BF16 &&
      c->weight_dtype != BLOOM_INT8_ROWSCALE)
    return BLOOM_EDTYPE;
  // activations: float32, bf16, fp16, or int8 (with int8 weights: W8A8); float32 only
  // for float32 weights.  The KV cache holds the activation type, or int8.
  if (c->act_dtype != BLOOM_F32 && c->act_dtype != BLOOM_BF16 && c->act_dtype != BLOOM_F16 &&
      c->act_dtype != BLOOM_INT8_ROWSCALE)
    return BLOOM_EDTYPE;
  if (c->weight_dtype == BLOOM_F32 && c->act_dtype != BLOOM_F32) return BLOOM_EDTYPE;
  if (c->act_dtype == BLOOM_INT8_ROWSCALE && c->weight_dtype != BLOOM_INT8_ROWSCALE)
    return BLOOM_EDTYPE;
  if (c->kv_dtype != c->act_dtype &&
      !(c->kv_dtype == BLOOM_INT8_ROWSCALE && c->weight_dtype != BLOOM_F32))
    return BLOOM_EDTYPE;
  if (c->weight_dtype != BLOOM_F32) {
    const int hd = c->n_head_local * c->head_dim;
    if (c->hidden % 64 || c->ffn % 64 || hd % 64) return BLOOM_EINVAL;
  }
  // int8 activations: the LayerNorm kernels quantise whole rows held in registers
  if (c->act_dtype == BLOOM_INT8_ROWSCALE && c->hidden > 16384) return BLOOM_EINVAL;
  return BLOOM_OK;
}

int check_weights(const bloom_config *c, const bloom_weights *w) {
  if (!w || !w->embed || !w->lnf_g || !w->lnf_b || !w->layers) return BLOOM_EINVAL;
  if (c->embed_ln && (!w->emb_ln_g || !w->emb_ln_b)) return BLOOM_EINVAL;
  const bool i8 = c->weight_dtype == BLOOM_INT8_ROWSCALE;
  for (int l = 0; l < c->n_layer; ++l) {
    const bloom_layer_weights &L = w->layers[l];
    const void *need[] = {L.ln1_g, L.ln1_b, L.w_qkv, L.b_qkv, L.w_dense, L.b_dense,
                          L.ln2_g, L.ln2_b, L.w_up,  L.b_up,  L.w_down, L.b_down};
    for (const void *p : need)
      if (!p) return BLOOM_EINVAL;
    const void *sc[] = {L.s_qkv, L.s_dense, L.s_up, L.s_down};
    for (const void *p : sc)
      if ((p != nullptr) != i8) return BLOOM_EINVAL;
  }
  return BLOOM_OK;
}

int check_kv(const bloom_config *c, const bloom_kv_cache *kv) {
  if (!kv || !kv->k || !kv->v || kv->max_batch <= 0 || kv->max_len <= 0) return BLOOM_EINVAL;
  if (c->kv_dtype == BLOOM_INT8_ROWSCALE &&
      (!kv->k_scale || !kv->v_scale || ((uintptr_t)kv->k_scale & 3) || ((uintptr_t)kv->v_scale & 3)))
    return BLOOM_EINVAL;
  if (((uintptr_t)kv->d_len & 3) != 0) return BLOOM_EINVAL;
  if (kv->max_len > kMaxLen) return BLOOM_EINVAL;
  if (kv->len < 0 || kv->len > kv->max_len || kv->prompt_len < 0) return BLOOM_EINVAL;
  return BLOOM_OK;
}

// ---------------------------------------------------------------------------
// launch timer
// ---------------------------------------------------------------------------
// A process-wide measurement aid: its state is guarded by g_timer_mu, so calls from
// several threads stay safe, but their launches then share (and interleave in) one
// record list.
struct Timer {
  bool on = false;
  bool paused = false;
  bool capturing = false;   // launches being captured into a graph are never timed
  std::vector<hipEvent_t> start, stop;
  std::vector<int> cls;
  std::vector<double> bytes;
  int used = 0;
} g_timer;
std::mutex g_timer_mu;

void destroy_timer_events() {
  for (hipEvent_t e : g_timer.start) (void)hipEventDestroy(e);
  for (hipEvent_t e : g_timer.stop) (void)hipEventDestroy(e);
  g_timer.start.clear();
  g_timer.stop.clear();
  g_timer.cls.clear();
  g_timer.bytes.clear();
  g_timer.used = 0;
}

int kernel_class(const LinearPlan &p) {
  switch (p.kind) {
    case LIN_VALU: return BLOOM_KERNEL_GEMV;
    case LIN_LG: return BLOOM_KERNEL_GEMM_LDS;
    default: return BLOOM_KERNEL_GEMM_F32;
  }
}

// Times one linear-layer launch (`launch` is a callable returning hipError_t) when the
// timer is on: its first kernel is launched with the timer's event pair attached.
template <typename F>
hipError_t timed(int cls, double wbytes, hipStream_t st, F &&launch) {
  if (!g_timer.on) return launch();   // the common case: no lock taken
  // launches captured into a graph (the library's own or a caller's) are never timed
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess) cap = hipStreamCaptureStatusActive;
  std::lock_guard<std::mutex> lock(g_timer_mu);
  const bool on = g_timer.on && !g_timer.paused && !g_timer.capturing &&
                  cap == hipStreamCaptureStatusNone && g_timer.used < (int)g_timer.start.size();
  if (on) g_launch_events = LaunchEvents{g_timer.start[g_timer.used], g_timer.stop[g_timer.used]};
  hipError_t err = launch();
  g_launch_events = LaunchEvents{};
  if (err != hipSuccess) return err;
  if (on) {
    g_timer.cls[g_timer.used] = cls;
    g_timer.bytes[g_timer.used] = wbytes;
    g_timer.used++;
  }
  return hipSuccess;
}

hipError_t timed_linear(int wdt, const LinearPlan &p, const void *X, const void *W, float *part,
                        const EpiParams &ep, hipStream_t st, double wbytes,
                        bool splitk_epilogue = true) {
  return timed(kernel_class(p), wbytes, st,
               [&] { return launch_linear(wdt, p, X, W, part, ep, st, splitk_epilogue); });
}

// Non-blocking stream (default priority) per device on which bloom_generate captures its
// decode step; created on first use, kept for the life of the process.
hipStream_t capture_stream() {
  static hipStream_t side[64] = {};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!side[dev] && hipStreamCreateWithFlags(&side[dev], hipStreamNonBlocking) != hipSuccess)
    side[dev] = nullptr;
  return side[dev];
}

// ---------------------------------------------------------------------------
// one forward pass over `tpr` tokens per row
// ---------------------------------------------------------------------------
// d_pos (nullable): device position of the first row of each sequence (a decode step
// replayed from a graph, or the KV length a caller keeps on the device); else pos_base.
int run_forward(const bloom_config *c, const bloom_weights *w, bloom_kv_cache *kv, int batch,
                int tpr, int pos_base, int prompt_len, const int32_t *d_tokens,
                const int32_t *d_valid, int32_t *d_next, float *d_hidden, char *ws,
                hipStream_t st, const int *d_pos = nullptr, float *d_logits = nullptr) {
  const WsPlan wp = plan_ws(c, batch, tpr);
  const bool f32 = c->weight_dtype == BLOOM_F32;
  const int act = act_fmt(c);
  const int wdt = wtype(c);
  const int M = batch * tpr;
  const int h = c->hidden, H = c->n_head_local, d = c->head_dim, F = c->ffn;
  const int hd = H * d;
  const size_t wb = c->weight_dtype == BLOOM_F32 ? 4 : (c->weight_dtype == BLOOM_BF16 ? 2 : 1);
  const size_t pb = f32 ? 4 : 2;
  const size_t sb = c->weight_dtype == BLOOM_INT8_ROWSCALE ? 2 : 0;
  auto wbytes = [&](int N, int K) { return (double)((size_t)N * K * wb + (size_t)N * (pb + sb)); };

  float *x = (float *)(ws + wp.x);
  void *xa = ws + wp.xa;
  float *q = (float *)(ws + wp.q);
  void *o = ws + wp.o;
  void *u = ws + wp.u;
  void *af = ws + wp.af;
  float *amv = (float *)(ws + wp.amv);
  int *ami = (int *)(ws + wp.ami);
  float *part = (float *)(ws + wp.part);
  float *stg = act_q8(c) ? (float *)(ws + wp.stg) : nullptr;
  float *kvs = kv_q8(c) ? (float *)(ws + wp.kvs) : nullptr;


  const size_t layer_stride = (size_t)kv->max_batch * H * kv->max_len * d * kv_bytes(c);
  const size_t scale_stride = (size_t)kv->max_batch * H * kv->max_len;   // int8 cache
  const LinearPlan p_qkv = plan_linear(wdt, M, 3 * hd, h, false, act);
  const LinearPlan p_dense = plan_linear(wdt, M, h, hd, false, act);
  const LinearPlan p_up = plan_linear(wdt, M, F, h, false, act);
  const LinearPlan p_down = plan_linear(wdt, M, h, F, false, act);
  // every activation is written in the form its consumer reads
  const int fmt_qkv = plan_x_fmt(p_qkv), fmt_dense = plan_x_fmt(p_dense);
  const int fmt_up = plan_x_fmt(p_up), fmt_down = plan_x_fmt(p_down);
  // int8 activation codes (AF_I8) carry one scale per row after the codes, which the
  // consuming linear's epilogue applies
  auto xscale = [&](int fmt, const void *buf, size_t n) -> const float * {
    return fmt == AF_I8 ? (const float *)((const char *)buf + (size_t)M * n) : nullptr;
  };

  // K-split dense / down projections reduce their partials in the kernel that also adds
  // bias and residual and runs the next LayerNorm (LN2 after dense, the next layer's LN1
  // after down); unsplit ones keep the epilogue in the GEMM and a separate LayerNorm.
  auto fuse_ln = [&](const LinearPlan &p) {
    return !f32 && p.splits > 1 && splitk_resid_ln_supported(h, p.splits);
  };
  // One activation row and a short hidden size: LN1 and LN2 run as the prologue of the
  // QKV and MLP-up GEMVs instead of as launches of their own.
  const bool ln_in_gemv = !f32 && !act_q8(c) && gemv_ln_supported(wdt, M, h);
  // With the caller's fold vectors (bloom_ln_fold), a one-row pass folds LN1 and LN2
  // into the QKV and MLP-up GEMVs: the residual epilogues of dense and down also store
  // gamma * x and add their blocks' sums of x and x^2 to the LayerNorm's accumulators
  // (zeroed by the embedding kernel), and the consumers finish the LayerNorm in their
  // epilogue.  Layer 0's LN1 (after the embedding) stays a launch.
  unsigned long long *stats = (unsigned long long *)(ws + wp.stats);
  auto ln_stats = [&](int l, int which) { return stats + (2 * (size_t)l + which) * kStatWords; };
  const size_t fold_layer = 2 * (size_t)(3 * hd + F);
  EpiParams cons{}, prod{};
  cons.mode = EPI_QKV;
  cons.ln_stats = stats;
  cons.ln_cd = w->ln_fold;
  prod.mode = EPI_RESID;
  prod.fold_g = w->ln_fold;   // (any non-null pointer: only the plan is probed)
  prod.fold_u = xa;
  prod.fold_stats = stats;
  const bool ln_fold = w->ln_fold && !ln_in_gemv && M == 1 &&
                       ln_fold_supported(wdt, p_qkv, cons) &&
                       ln_fold_supported(wdt, p_up, cons) &&
                       ln_fold_supported(wdt, p_dense, prod) &&
                       ln_fold_supported(wdt, p_down, prod) && fmt_qkv == fmt_up;
  hipError_t err = launch_embed(f32, d_tokens, w->embed, w->emb_ln_g, w->emb_ln_b, x, M, h,
                                c->vocab, c->embed_ln, c->ln_eps, ln_fold ? stats : nullptr,
                                ln_fold ? c->n_layer * 2 * kStatWords : 0, st);
  if (err != hipSuccess) return hip_fail(err);
  bool ln1_done = false;   // xa already holds LN1(x) of this layer
  bool ln1_folded = false; // xa holds gamma1 * x (the previous down projection's epilogue)
  for (int l = 0; l < c->n_layer; ++l) {
    const bloom_layer_weights &L = w->layers[l];
    void *kc = (char *)kv->k + l * layer_stride;
    void *vc = (char *)kv->v + l * layer_stride;
    float *ksc = kvs ? (float *)kv->k_scale + l * scale_stride : nullptr;
    float *vsc = kvs ? (float *)kv->v_scale + l * scale_stride : nullptr;

    if (!ln1_done && !ln1_folded && !ln_in_gemv) {
      err = launch_layernorm(f32, x, 1, 0, L.ln1_g, L.ln1_b, xa, fmt_qkv, nullptr, M, h,
                             c->ln_eps, st);
      if (err != hipSuccess) return hip_fail(err);
    }
    ln1_done = false;

    EpiParams e{};
    e.mode = EPI_QKV;
    e.bias = L.b_qkv;
    e.scale = (const uint16_t *)L.s_qkv;
    e.q = q; e.kc = kc; e.vc = vc;
    e.kv_fmt = kv_fmt(c);
    e.H = H; e.d = d; e.max_len = kv->max_len;
    e.pos_base = pos_base; e.pos_dev = d_pos; e.rows_per_seq = tpr;
    e.q_scale = 1.0f / sqrtf((float)d);
    e.xscale = xscale(fmt_qkv, xa, h);
    e.kv_stage = kvs;
    if (ln1_folded) {
      // d_qkv holds the bias
      e.bias = nullptr;
      e.ln_stats = ln_stats(l, 0);
      e.ln_cd = w->ln_fold + l * fold_layer;
      e.ln_eps = c->ln_eps;
    }
    if (ln_in_gemv)
      err = timed(kernel_class(p_qkv), wbytes(3 * hd, h), st, [&] {
        return launch_gemv_ln(wdt, act, 3 * hd, h, x, L.ln1_g, L.ln1_b, c->ln_eps, L.w_qkv, e,
                              st);
      });
    else
      err = timed_linear(wdt, p_qkv, xa, L.w_qkv, part, e, st, wbytes(3 * hd, h));
    if (err != hipSuccess) return hip_fail(err);
    if (kvs) {
      // int8 cache: the staged new keys and values [M][H][2][d] -> codes + slot scales
      KvQuantArgs qa{};
      qa.k = kvs; qa.v = kvs + d;
      qa.sb = (long)tpr * H * 2 * d; qa.st = (long)H * 2 * d; qa.sh = 2 * d;
      qa.batch = batch; qa.n = tpr; qa.H = H; qa.d = d;
      qa.kc = (int8_t *)kc; qa.vc = (int8_t *)vc; qa.ks = ksc; qa.vs = vsc;
      qa.max_len = kv->max_len; qa.pos_base = pos_base; qa.pos_dev = d_pos;
      err = launch_kv_quant(qa, st);
      if (err != hipSuccess) return hip_fail(err);
    }

    // int8 activations: attention writes float32 rows, quantised per row for the dense
    // projection
    err = launch_attention(kv_fmt(c), q, kc, vc, ksc, vsc, d_valid, stg ? (void *)stg : o,
                           stg ? AF_F32 : fmt_dense, M, H, d, kv->max_len, c->n_head_total,
                           c->head_offset, tpr, pos_base, d_pos, prompt_len,
                           (float *)(ws + wp.attn), st);
    if (err == hipSuccess && stg) err = launch_quant_rows(stg, M, hd, o, fmt_dense, st);
    if (err != hipSuccess) return hip_fail(err);

    EpiParams r{};
    r.mode = EPI_RESID;
    r.bias = L.b_dense;
    r.scale = (const uint16_t *)L.s_dense;
    r.out = x; r.ld = h;
    r.xscale = xscale(fmt_dense, o, hd);
    if (ln_fold) {
      r.fold_g = L.ln2_g;
      r.fold_u = xa;
      r.fold_fmt = fmt_up;
      r.fold_stats = ln_stats(l, 1);
    }
    const bool fuse_dense = fuse_ln(p_dense);
    err = timed_linear(wdt, p_dense, o, L.w_dense, part, r, st, wbytes(h, hd), !fuse_dense);
    if (err != hipSuccess) return hip_fail(err);

    if (fuse_dense)
      err = launch_splitk_resid_ln(part, p_dense.splits, M, r.xscale, L.s_dense, L.b_dense, x,
                                   L.ln2_g, L.ln2_b, xa, fmt_up, h, c->ln_eps, st);
    else if (!ln_in_gemv && !ln_fold)
      err = launch_layernorm(f32, x, 1, 0, L.ln2_g, L.ln2_b, xa, fmt_up, nullptr, M, h,
                             c->ln_eps, st);
    if (err != hipSuccess) return hip_fail(err);

    EpiParams g{};
    g.mode = EPI_GELU;
    g.bias = L.b_up;
    g.scale = (const uint16_t *)L.s_up;
    g.out = u; g.ld = F;
    g.out_fmt = fmt_down;
    g.plane = (size_t)M * F;
    g.xscale = xscale(fmt_up, xa, h);
    if (stg) {   // int8 activations: GeLU rows in float32, then quantised per row
      g.out = stg;
      g.out_fmt = AF_F32;
    }
    if (ln_fold) {
      g.bias = nullptr;   // d_up holds it
      g.ln_stats = ln_stats(l, 1);
      g.ln_cd = w->ln_fold + l * fold_layer + 2 * (size_t)(3 * hd);
      g.ln_eps = c->ln_eps;
    }
    if (ln_in_gemv && !fuse_dense)
      err = timed(kernel_class(p_up), wbytes(F, h), st, [&] {
        return launch_gemv_ln(wdt, act, F, h, x, L.ln2_g, L.ln2_b, c->ln_eps, L.w_up, g, st);
      });
    else
      err = timed_linear(wdt, p_up, xa, L.w_up, part, g, st, wbytes(F, h));
    if (err == hipSuccess && stg) err = launch_quant_rows(stg, M, F, u, fmt_down, st);
    if (err != hipSuccess) return hip_fail(err);

    EpiParams dn{};
    dn.mode = EPI_RESID;
    dn.bias = L.b_down;
    dn.scale = (const uint16_t *)L.s_down;
    dn.out = x; dn.ld = h;
    dn.xscale = xscale(fmt_down, u, F);
    const bool fuse_down = l + 1 < c->n_layer && fuse_ln(p_down) && !ln_in_gemv;
    ln1_folded = ln_fold && l + 1 < c->n_layer;
    if (ln1_folded) {
      dn.fold_g = w->layers[l + 1].ln1_g;
      dn.fold_u = xa;
      dn.fold_fmt = fmt_qkv;
      dn.fold_stats = ln_stats(l + 1, 0);
    }
    err = timed_linear(wdt, p_down, u, L.w_down, part, dn, st, wbytes(h, F), !fuse_down);
    if (err != hipSuccess) return hip_fail(err);
    if (fuse_down) {
      const bloom_layer_weights &N1 = w->layers[l + 1];
      err = launch_splitk_resid_ln(part, p_down.splits, M, dn.xscale, L.s_down, L.b_down, x,
                                   N1.ln1_g, N1.ln1_b, xa, fmt_qkv, h, c->ln_eps, st);
      if (err != hipSuccess) return hip_fail(err);
      ln1_done = true;
    }
  }

  // final LayerNorm of each row's last position, then the tied LM head + argmax (the
  // LM head is skipped when the caller asked for the hidden states only)
  const int nblk = wp.lm_blocks;
  const int wdt_lm = f32 ? WT_F32 : WT_BF16;  // the embedding is never int8
  const double lm_bytes = (double)c->vocab * h * pb;
  const bool lm_head = d_logits || d_next;
  if (!lm_head) {
    err = launch_layernorm(f32, x, tpr, tpr - 1, w->lnf_g, w->lnf_b, af, f32 ? AF_F32 : AF_BF16,
                           d_hidden, batch, h, c->ln_eps, st);
    return err == hipSuccess ? BLOOM_OK : hip_fail(err);
  }
  const size_t abytes = act_bytes(c);
  for (int r0 = 0; r0 < batch; r0 += 128) {
    // the LM head runs on chunks of up to 128 rows; the final LayerNorm writes each
    // chunk in the form its plan reads (two bf16 planes: each chunk its own pair)
    const int rows = std::min(128, batch - r0);
    const LinearPlan p_lm = plan_linear(wdt_lm, rows, c->vocab, h, true, lm_act_fmt(c));
    void *X = (char *)af + (size_t)r0 * h * abytes;
    err = launch_layernorm(f32, x + (size_t)r0 * tpr * h, tpr, tpr - 1, w->lnf_g, w->lnf_b, X,
                           plan_x_fmt(p_lm), d_hidden ? d_hidden + (size_t)r0 * h : nullptr, rows,
                           h, c->ln_eps, st);
    if (err != hipSuccess) return hip_fail(err);
    EpiParams a{};
    if (d_logits) {
      // the LM head's float32 logits [batch][vocab] instead of its argmax (sampling), with
      // the greedy head's plan, so a greedy row of the sampler ranks the same values
      a.mode = EPI_STORE;
      a.out = d_logits + (size_t)r0 * c->vocab;
      a.ld = c->vocab;
    } else {
      a.mode = EPI_ARGMAX;
      a.am_val = amv + (size_t)r0 * nblk;
      a.am_idx = ami + (size_t)r0 * nblk;
      a.am_stride = nblk;
    }
    err = timed_linear(wdt_lm, p_lm, X, w->embed, part, a, st, lm_bytes);
    if (err != hipSuccess) return hip_fail(err);
    if (!d_logits) {
      // this chunk's kernel wrote one partial per row per weight tile
      err = launch_argmax_merge(a.am_val, a.am_idx, nblk, argmax_partials_per_row(p_lm), rows,
                                d_next + r0, st);
      if (err != hipSuccess) return hip_fail(err);
    }
  }
  return BLOOM_OK;
}

}  // namespace

extern "C" {

const char *bloom_status_string(int s) {
  switch (s) {
    case BLOOM_OK: return "ok";
    case BLOOM_EINVAL: return "invalid argument (shape, pointer or index)";
    case BLOOM_EDTYPE: return "unsupported data type";
    case BLOOM_ECAPACITY: return "KV cache capacity exceeded";
    case BLOOM_EWORKSPACE: return "workspace too small";
    case BLOOM_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *bloom_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

int bloom_workspace_bytes(const bloom_config *cfg, int32_t max_batch, int32_t max_prompt,
                          size_t *bytes) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if (!bytes || max_batch < 0 || max_prompt < 0) return BLOOM_EINVAL;
  *bytes = plan_ws(cfg, max_batch, std::max(max_prompt, 1)).total;
  return BLOOM_OK;
}

int bloom_prefill(const bloom_config *cfg, const bloom_weights *w, bloom_kv_cache *kv,
                  int32_t batch, int32_t prompt_len, const int32_t *d_tokens,
                  const int32_t *d_valid_len, int32_t *d_next_tokens, float *d_hidden_out,
                  void *d_ws, size_t ws_bytes, void *stream) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if ((s = check_weights(cfg, w)) != BLOOM_OK) return s;
  if ((s = check_kv(cfg, kv)) != BLOOM_OK) return s;
  if (batch < 0 || prompt_len < 1) return BLOOM_EINVAL;
  if (batch > kv->max_batch || prompt_len > kv->max_len) return BLOOM_ECAPACITY;
  if (batch == 0) return BLOOM_OK;
  if (!d_tokens || !d_valid_len || !d_ws || (!d_next_tokens && !d_hidden_out)) return BLOOM_EINVAL;
  if (ws_bytes < plan_ws(cfg, batch, prompt_len).total) return BLOOM_EWORKSPACE;
  clear_stale_hip_error();
  s = run_forward(cfg, w, kv, batch, prompt_len, 0, prompt_len, d_tokens, d_valid_len,
                  d_next_tokens, d_hidden_out, (char *)d_ws, (hipStream_t)stream);
  if (s == BLOOM_OK && kv->d_len) {
    const hipError_t e = launch_len_update(kv->d_len, prompt_len, 0, kv->max_len,
                                           (hipStream_t)stream);
    if (e != hipSuccess) s = hip_fail(e);
  }
  if (s == BLOOM_OK) {
    kv->prompt_len = prompt_len;
    kv->len = prompt_len;
  }
  return s;
}

int bloom_decode_step(const bloom_config *cfg, const bloom_weights *w, bloom_kv_cache *kv,
                      int32_t batch, const int32_t *d_tokens, const int32_t *d_valid_len,
                      int32_t *d_next_tokens, float *d_hidden_out, void *d_ws, size_t ws_bytes,
                      void *stream) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if ((s = check_weights(cfg, w)) != BLOOM_OK) return s;
  if ((s = check_kv(cfg, kv)) != BLOOM_OK) return s;
  if (batch < 0) return BLOOM_EINVAL;
  if (kv->prompt_len <= 0 || kv->len < kv->prompt_len) return BLOOM_EINVAL;
  if (batch > kv->max_batch || kv->len >= kv->max_len) return BLOOM_ECAPACITY;
  if (batch == 0) return BLOOM_OK;
  if (!d_tokens || !d_valid_len || !d_ws || (!d_next_tokens && !d_hidden_out)) return BLOOM_EINVAL;
  if (ws_bytes < plan_ws(cfg, batch, 1).total) return BLOOM_EWORKSPACE;
  clear_stale_hip_error();
  // with a device-resident length the step reads its position from it and advances it
  // (so a captured step can be replayed); the host count follows the calls
  s = run_forward(cfg, w, kv, batch, 1, kv->len, kv->prompt_len, d_tokens, d_valid_len,
                  d_next_tokens, d_hidden_out, (char *)d_ws, (hipStream_t)stream, kv->d_len);
  if (s == BLOOM_OK && kv->d_len) {
    const hipError_t e = launch_len_update(kv->d_len, -1, 1, kv->max_len, (hipStream_t)stream);
    if (e != hipSuccess) s = hip_fail(e);
  }
  if (s == BLOOM_OK) kv->len += 1;
  return s;
}

int bloom_generate(const bloom_config *cfg, const bloom_weights *w, bloom_kv_cache *kv,
                   int32_t batch, int32_t prompt_len, const int32_t *d_tokens,
                   const int32_t *d_valid_len, int32_t n_new, int32_t *d_ids, float *d_hidden,
                   const bloom_gen_control *ctl, void *d_ws, size_t ws_bytes, void *stream) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if ((s = check_weights(cfg, w)) != BLOOM_OK) return s;
  if ((s = check_kv(cfg, kv)) != BLOOM_OK) return s;
  if (batch < 0 || prompt_len < 1 || n_new < 1) return BLOOM_EINVAL;
  if (batch > kv->max_batch || (long)prompt_len + n_new - 1 > kv->max_len) return BLOOM_ECAPACITY;
  if (batch == 0) return BLOOM_OK;
  if (!d_tokens || !d_valid_len || !d_ids || !d_ws) return BLOOM_EINVAL;
  if (ctl && ctl->eos_id >= cfg->vocab) return BLOOM_EINVAL;
  if (ws_bytes < plan_ws(cfg, batch, prompt_len).total) return BLOOM_EWORKSPACE;
  const bool sampled = ctl && (ctl->d_temperature || ctl->d_top_p || ctl->d_uniform ||
                               ctl->d_logits || ctl->d_sample_ws);
  if (sampled) {
    if (!ctl->d_temperature || !ctl->d_top_p || !ctl->d_uniform || !ctl->d_logits ||
        !ctl->d_sample_ws || cfg->vocab > (1 << 23))
      return BLOOM_EINVAL;
    if (ctl->sample_ws_bytes < sample_workspace_bytes(batch, cfg->vocab)) return BLOOM_EWORKSPACE;
  }
  clear_stale_hip_error();
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)d_ws;
  // generation state, current / next ids and the hidden rows of a step: the same
  // workspace offsets for every pass
  const WsPlan wp = plan_ws(cfg, batch, 1);
  int *state = (int *)(ws + wp.gen);
  int *cur = (int *)(ws + wp.cur);
  int *nxt = (int *)(ws + wp.nxt);
  float *hfix = d_hidden ? (float *)(ws + wp.hfix) : nullptr;
  GenControl gc{};
  gc.done = (int *)(ws + wp.done);
  gc.eos_id = ctl ? ctl->eos_id : -1;
  gc.pad_id = ctl ? ctl->pad_id : 0;
  gc.max_new = ctl ? ctl->d_max_new : nullptr;
  gc.out_len = ctl ? ctl->d_out_len : nullptr;

  // One pass and its token: the greedy LM head's argmax, or (sampling) its logits and
  // a draw with the uniform number of the step being recorded (state[1]).
  float *logits = sampled ? ctl->d_logits : nullptr;
  auto pass = [&](int tpr, int pos_base, const int32_t *toks, hipStream_t sst,
                  const int *d_pos) -> int {
    int r = run_forward(cfg, w, kv, batch, tpr, pos_base, prompt_len, toks, d_valid_len, nxt,
                        hfix, ws, sst, d_pos, logits);
    if (r != BLOOM_OK || !sampled) return r;
    const hipError_t e = launch_sample_rows(logits, batch, cfg->vocab, ctl->d_temperature,
                                            ctl->d_top_p, ctl->d_uniform, nxt, ctl->d_sample_ws,
                                            sst, state + 1);
    return e == hipSuccess ? BLOOM_OK : hip_fail(e);
  };
  // the prompt pass and the first decode step run eagerly (they also run any one-time
  // set-up); every step's ids go through the same recording kernel
  hipError_t err = launch_gen_init(state, prompt_len - 1, 0, gc.done, batch, st);
  if (err != hipSuccess) return hip_fail(err);
  s = pass(prompt_len, 0, d_tokens, st, nullptr);
  if (s != BLOOM_OK) return s;
  if ((err = launch_gen_record(nxt, cur, d_ids, hfix, d_hidden, state, batch, cfg->hidden, gc,
                               st)) != hipSuccess)
    return hip_fail(err);
  kv->prompt_len = prompt_len;
  kv->len = prompt_len;
  if (n_new >= 2) {
    s = pass(1, kv->len, cur, st, nullptr);
    if (s != BLOOM_OK) return s;
    if ((err = launch_gen_record(nxt, cur, d_ids, hfix, d_hidden, state, batch, cfg->hidden, gc,
                                 st)) != hipSuccess)
      return hip_fail(err);
    kv->len += 1;
  }
  if (n_new <= 2) {
    if (kv->d_len &&
        (err = launch_len_update(kv->d_len, kv->len, 0, kv->max_len, st)) != hipSuccess)
      return hip_fail(err);
    const hipError_t serr = hipStreamSynchronize(st);
    return serr == hipSuccess ? BLOOM_OK : hip_fail(serr);
  }

  // One decode step captured on a side stream: position and input tokens come from
  // device memory, so the same graph is replayed for every remaining step.
  hipStream_t side = capture_stream();
  if (!side) return hip_fail(hipErrorInvalidResourceHandle);
  if ((err = hipStreamBeginCapture(side, hipStreamCaptureModeThreadLocal)) != hipSuccess)
    return hip_fail(err);
  g_timer.capturing = true;
  s = pass(1, 0, cur, side, state);
  g_timer.capturing = false;
  if (s == BLOOM_OK) {
    err = launch_gen_record(nxt, cur, d_ids, hfix, d_hidden, state, batch, cfg->hidden, gc, side);
    if (err != hipSuccess) s = hip_fail(err);
  }
  hipGraph_t graph = nullptr;
  const hipError_t cerr = hipStreamEndCapture(side, &graph);
  if (s != BLOOM_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return s;
  }
  if (cerr != hipSuccess) return hip_fail(cerr);
  hipGraphExec_t exec = nullptr;
  err = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (err != hipSuccess) return hip_fail(err);
  for (int t = 2; t < n_new && err == hipSuccess; ++t) err = hipGraphLaunch(exec, st);
  if (err == hipSuccess && kv->d_len)
    err = launch_len_update(kv->d_len, prompt_len + n_new - 1, 0, kv->max_len, st);
  // the executable graph is released once its launches have finished
  const hipError_t serr = hipStreamSynchronize(st);
  (void)hipGraphExecDestroy(exec);
  if (err != hipSuccess) return hip_fail(err);
  if (serr != hipSuccess) return hip_fail(serr);
  kv->len = prompt_len + n_new - 1;
  return BLOOM_OK;
}

int alibi_masked_softmax(const void *d_scores, int32_t in_dtype, const int32_t *d_valid_len,
                         int32_t B, int32_t H, int32_t Q, int32_t K, int32_t n_head_total,
                         int32_t head_offset, void *d_probs, int32_t out_dtype, void *stream) {
  if (B < 0 || H < 0 || Q < 0 || K < 0 || Q > K) return BLOOM_EINVAL;
  if (n_head_total < 1 || head_offset < 0 || head_offset + H > n_head_total) return BLOOM_EINVAL;
  if ((in_dtype != BLOOM_F32 && in_dtype != BLOOM_BF16) ||
      (out_dtype != BLOOM_F32 && out_dtype != BLOOM_BF16))
    return BLOOM_EDTYPE;
  if ((long)B * H * Q == 0 || K == 0) return BLOOM_OK;
  if (!d_scores || !d_valid_len || !d_probs) return BLOOM_EINVAL;
  clear_stale_hip_error();
  hipError_t err = launch_alibi_softmax(d_scores, in_dtype == BLOOM_BF16, d_valid_len, d_probs,
                                        out_dtype == BLOOM_BF16, B, H, Q, K, n_head_total,
                                        head_offset, (hipStream_t)stream);
  return err == hipSuccess ? BLOOM_OK : hip_fail(err);
}

int kv_cache_append(const bloom_config *cfg, bloom_kv_cache *kv, int32_t layer, int32_t batch,
                    int32_t pos, const void *d_k, const void *d_v, int32_t n_new, void *stream) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if ((s = check_kv(cfg, kv)) != BLOOM_OK) return s;
  if (layer < 0 || layer >= cfg->n_layer || batch < 0 || pos < 0 || n_new < 0)
    return BLOOM_EINVAL;
  if (batch > kv->max_batch || (long)pos + n_new > kv->max_len) return BLOOM_ECAPACITY;
  if (batch == 0 || n_new == 0) return BLOOM_OK;
  if (!d_k || !d_v) return BLOOM_EINVAL;
  clear_stale_hip_error();
  const size_t kvb = kv_bytes(cfg);
  const size_t layer_stride =
      (size_t)kv->max_batch * cfg->n_head_local * kv->max_len * cfg->head_dim * kvb;
  if (kv_q8(cfg)) {
    // float32 inputs, quantised per (row, head, slot) as the forward pass does
    const int H = cfg->n_head_local, d = cfg->head_dim;
    const size_t scale_stride = (size_t)kv->max_batch * H * kv->max_len;
    KvQuantArgs qa{};
    qa.k = (const float *)d_k; qa.v = (const float *)d_v;
    qa.sb = (long)H * n_new * d; qa.st = d; qa.sh = (long)n_new * d;
    qa.batch = batch; qa.n = n_new; qa.H = H; qa.d = d;
    qa.kc = (int8_t *)kv->k + layer * layer_stride;
    qa.vc = (int8_t *)kv->v + layer * layer_stride;
    qa.ks = (float *)kv->k_scale + layer * scale_stride;
    qa.vs = (float *)kv->v_scale + layer * scale_stride;
    qa.max_len = kv->max_len; qa.pos_base = pos;
    const hipError_t qe = launch_kv_quant(qa, (hipStream_t)stream);
    return qe == hipSuccess ? BLOOM_OK : hip_fail(qe);
  }
  hipError_t err = launch_kv_append(kv_fmt(cfg) == AF_F32, d_k, d_v,
                                    (char *)kv->k + layer * layer_stride,
                                    (char *)kv->v + layer * layer_stride, batch,
                                    cfg->n_head_local, n_new, cfg->head_dim, kv->max_len, pos,
                                    (hipStream_t)stream);
  return err == hipSuccess ? BLOOM_OK : hip_fail(err);
}

int kv_cache_compact(const bloom_config *cfg, bloom_kv_cache *kv, int32_t batch,
                     const int32_t *keep, int32_t n_keep, void *stream) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if ((s = check_kv(cfg, kv)) != BLOOM_OK) return s;
  if (batch < 0 || n_keep < 0 || n_keep > batch) return BLOOM_EINVAL;
  if (batch > kv->max_batch) return BLOOM_ECAPACITY;
  if (n_keep == 0) return BLOOM_OK;
  if (!keep) return BLOOM_EINVAL;
  for (int i = 0; i < n_keep; ++i)
    if (keep[i] < 0 || keep[i] >= batch || (i > 0 && keep[i] <= keep[i - 1])) return BLOOM_EINVAL;
  clear_stale_hip_error();
  hipError_t err = launch_kv_compact(kv->k, kv->v, cfg->n_layer, cfg->n_head_local,
                                     kv->max_batch, kv->max_len, cfg->head_dim, kv_bytes(cfg),
                                     kv->len, keep, n_keep, (hipStream_t)stream);
  // an int8 cache's slot scales move with their rows (one float32 per slot)
  if (err == hipSuccess && kv_q8(cfg))
    err = launch_kv_compact(kv->k_scale, kv->v_scale, cfg->n_layer, cfg->n_head_local,
                            kv->max_batch, kv->max_len, 1, 4, kv->len, keep, n_keep,
                            (hipStream_t)stream);
  return err == hipSuccess ? BLOOM_OK : hip_fail(err);
}

int bloom_lm_logits(const bloom_config *cfg, const bloom_weights *w, int32_t batch,
                    const float *d_hidden, float *d_logits, void *d_ws, size_t ws_bytes,
                    void *stream) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if (!w || !w->embed || batch < 0) return BLOOM_EINVAL;
  if (batch == 0) return BLOOM_OK;
  if (!d_hidden || !d_logits || !d_ws) return BLOOM_EINVAL;
  const WsPlan wp = plan_ws(cfg, batch, 1);
  if (ws_bytes < wp.total) return BLOOM_EWORKSPACE;
  clear_stale_hip_error();
  hipStream_t st = (hipStream_t)stream;
  const bool f32 = cfg->weight_dtype == BLOOM_F32;
  const int h = cfg->hidden;
  const int wdt_lm = f32 ? WT_F32 : WT_BF16;
  const size_t act = act_bytes(cfg);
  float *part = (float *)((char *)d_ws + wp.part);
  for (int r0 = 0; r0 < batch; r0 += 128) {
    const int rows = std::min(128, batch - r0);
    EpiParams e{};
    e.mode = EPI_STORE;
    e.out = d_logits + (size_t)r0 * cfg->vocab;
    e.ld = cfg->vocab;
    // the greedy LM head's plan (never split) and operand form, so the logits are the
    // ones it ranks
    const LinearPlan p = plan_linear(wdt_lm, rows, cfg->vocab, h, true, lm_act_fmt(cfg));
    const float *hr = d_hidden + (size_t)r0 * h;
    const void *X = hr;
    if (plan_x_fmt(p) != AF_F32) {
      void *af = (char *)d_ws + wp.af + (size_t)r0 * h * act;
      const hipError_t ce = launch_f32_to_act(hr, af, plan_x_fmt(p), (size_t)rows * h, st);
      if (ce != hipSuccess) return hip_fail(ce);
      X = af;
    }
    const hipError_t err = launch_linear(wdt_lm, p, X, w->embed, part, e, st);
    if (err != hipSuccess) return hip_fail(err);
  }
  return BLOOM_OK;
}

}  // extern "C"

namespace {

// Workspace of a standalone linear: the activations in the form the plan reads, then
// the split-K partials.
struct LinearWs {
  LinearPlan plan;
  int fmt;
  size_t x_bytes, total;
};

LinearWs plan_linear_ws(const bloom_config *c, int M, int N, int K) {
  LinearWs w{};
  w.plan = plan_linear(wtype(c), M, N, K, false, act_fmt(c));
  w.fmt = plan_x_fmt(w.plan);
  w.x_bytes = w.fmt == AF_F32 ? 0 : align256(act_region(c, M, K));
  w.total = w.x_bytes + align256(linear_partial_bytes(w.plan));
  return w;
}

int check_linear(const bloom_config *cfg, int32_t M, int32_t N, int32_t K) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if (M < 0 || N < 1 || K < 1) return BLOOM_EINVAL;
  if (cfg->weight_dtype != BLOOM_F32 && K % 64) return BLOOM_EINVAL;
  if (cfg->act_dtype == BLOOM_INT8_ROWSCALE && K > 1 << 24) return BLOOM_EINVAL;
  return BLOOM_OK;
}

}  // namespace

extern "C" {

int bloom_linear_workspace_bytes(const bloom_config *cfg, int32_t M, int32_t N, int32_t K,
                                 size_t *bytes) {
  int s = check_linear(cfg, M, N, K);
  if (s != BLOOM_OK) return s;
  if (!bytes) return BLOOM_EINVAL;
  *bytes = M == 0 ? 0 : plan_linear_ws(cfg, M, N, K).total;
  return BLOOM_OK;
}

int bloom_linear(const bloom_config *cfg, int32_t M, int32_t N, int32_t K, const float *d_x,
                 const void *d_w, const void *d_s, const void *d_b, float *d_y, void *d_ws,
                 size_t ws_bytes, void *stream) {
  int s = check_linear(cfg, M, N, K);
  if (s != BLOOM_OK) return s;
  if (M == 0) return BLOOM_OK;
  if (!d_x || !d_w || !d_y) return BLOOM_EINVAL;
  if ((d_s != nullptr) != (cfg->weight_dtype == BLOOM_INT8_ROWSCALE)) return BLOOM_EINVAL;
  const LinearWs lw = plan_linear_ws(cfg, M, N, K);
  if (lw.total > 0 && (!d_ws || ws_bytes < lw.total)) return BLOOM_EWORKSPACE;
  clear_stale_hip_error();
  hipStream_t st = (hipStream_t)stream;
  // the activations stored as the forward pass stores them for a linear of this plan
  const void *X = d_x;
  char *xs = (char *)d_ws;
  hipError_t err = hipSuccess;
  if (lw.fmt == AF_I8)
    err = launch_quant_rows(d_x, M, K, xs, lw.fmt, st);
  else if (lw.fmt != AF_F32)
    err = launch_f32_to_act(d_x, xs, lw.fmt, (size_t)M * K, st);
  if (err != hipSuccess) return hip_fail(err);
  if (lw.fmt != AF_F32) X = xs;
  EpiParams e{};
  e.mode = EPI_STORE;
  e.out = d_y;
  e.ld = N;
  e.bias = d_b;
  e.scale = (const uint16_t *)d_s;
  e.xscale = lw.fmt == AF_I8 ? (const float *)(xs + (size_t)M * K) : nullptr;
  err = launch_linear(wtype(cfg), lw.plan, X, d_w, (float *)((char *)d_ws + lw.x_bytes), e, st);
  return err == hipSuccess ? BLOOM_OK : hip_fail(err);
}

int bloom_ln_fold_bytes(const bloom_config *cfg, size_t *bytes) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if (!bytes) return BLOOM_EINVAL;
  const size_t hd = (size_t)cfg->n_head_local * cfg->head_dim;
  *bytes = (size_t)cfg->n_layer * 2 * (3 * hd + (size_t)cfg->ffn) * sizeof(float);
  return BLOOM_OK;
}

int bloom_ln_fold(const bloom_config *cfg, const bloom_weights *w, float *d_fold, size_t bytes,
                  void *stream) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if ((s = check_weights(cfg, w)) != BLOOM_OK) return s;
  if (cfg->weight_dtype != BLOOM_BF16) return BLOOM_EDTYPE;
  if (!d_fold) return BLOOM_EINVAL;
  size_t need = 0;
  bloom_ln_fold_bytes(cfg, &need);
  if (bytes < need) return BLOOM_EWORKSPACE;
  clear_stale_hip_error();
  hipStream_t st = (hipStream_t)stream;
  const int h = cfg->hidden, F = cfg->ffn, n3 = 3 * cfg->n_head_local * cfg->head_dim;
  for (int l = 0; l < cfg->n_layer; ++l) {
    const bloom_layer_weights &L = w->layers[l];
    float *f = d_fold + (size_t)l * 2 * (n3 + F);
    hipError_t e = launch_ln_fold(L.w_qkv, L.ln1_g, L.ln1_b, L.b_qkv, n3, h, f, f + n3, st);
    if (e == hipSuccess)
      e = launch_ln_fold(L.w_up, L.ln2_g, L.ln2_b, L.b_up, F, h, f + 2 * n3, f + 2 * n3 + F, st);
    if (e != hipSuccess) return hip_fail(e);
  }
  return BLOOM_OK;
}

int bloom_init_weights(const bloom_config *cfg, const bloom_weights *w, uint64_t seed,
                       double sigma, void *stream) {
  int s = check_config(cfg);
  if (s != BLOOM_OK) return s;
  if ((s = check_weights(cfg, w)) != BLOOM_OK) return s;
  if (!(sigma >= 0.0) || !(sigma < 1e30)) return BLOOM_EINVAL;
  clear_stale_hip_error();
  hipStream_t st = (hipStream_t)stream;
  auto smix = [](uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  };
  // scales of the specification, computed in double and rounded to float32 once
  const float nscale = (float)(sigma / std::sqrt((65536.0 * 65536.0 - 1.0) / 3.0));
  const float s0 = (float)(sigma / std::sqrt((255.0 * 255.0 - 1.0) / 12.0));
  const int pkind = cfg->weight_dtype == BLOOM_F32 ? 0 : 1;   // float32 or bf16 storage
  const bool i8 = cfg->weight_dtype == BLOOM_INT8_ROWSCALE;
  auto fill = [&](const void *p, size_t n, uint64_t tid, int op, int kind, float mean,
                  float scale) -> hipError_t {
    InitTensor t{};
    t.out = const_cast<void *>(p);
    t.n = n;
    t.key = smix((seed << 32) ^ tid);
    t.op = op; t.kind = kind; t.mean = mean; t.scale = scale;
    return launch_init_tensor(t, st);
  };
  auto normal = [&](const void *p, size_t n, uint64_t tid, float mean) {
    return fill(p, n, tid, 0, pkind, mean, nscale);
  };
  const size_t h = cfg->hidden, hd = (size_t)cfg->n_head_local * cfg->head_dim, F = cfg->ffn;
  hipError_t e = normal(w->embed, (size_t)cfg->vocab * h, 1, 0.f);
  if (e == hipSuccess && cfg->embed_ln) e = normal(w->emb_ln_g, h, 2, 1.f);
  if (e == hipSuccess && cfg->embed_ln) e = normal(w->emb_ln_b, h, 3, 0.f);
  if (e == hipSuccess) e = normal(w->lnf_g, h, 4, 1.f);
  if (e == hipSuccess) e = normal(w->lnf_b, h, 5, 0.f);
  for (int l = 0; l < cfg->n_layer && e == hipSuccess; ++l) {
    const bloom_layer_weights &L = w->layers[l];
    const uint64_t base = 1024 + 16 * (uint64_t)l;   // tensor ids of layer l, in field order
    auto mat = [&](const void *p, size_t n, int idx) {
      return i8 ? fill(p, n, base + idx, 1, 0, 0.f, 0.f) : normal(p, n, base + idx, 0.f);
    };
    const struct { const void *p; size_t n; int idx; int what; } t[] = {
        {L.ln1_g, h, 0, 1},  {L.ln1_b, h, 1, 0},      {L.w_qkv, 3 * hd * h, 2, 2},
        {L.b_qkv, 3 * hd, 3, 0}, {L.w_dense, h * hd, 4, 2}, {L.b_dense, h, 5, 0},
        {L.ln2_g, h, 6, 1},  {L.ln2_b, h, 7, 0},      {L.w_up, F * h, 8, 2},
        {L.b_up, F, 9, 0},   {L.w_down, h * F, 10, 2}, {L.b_down, h, 11, 0},
        {L.s_qkv, 3 * hd, 12, 3}, {L.s_dense, h, 13, 3}, {L.s_up, F, 14, 3}, {L.s_down, h, 15, 3}};
    for (const auto &x : t) {
      if (e != hipSuccess) break;
      if (x.what == 0) e = normal(x.p, x.n, base + x.idx, 0.f);
      else if (x.what == 1) e = normal(x.p, x.n, base + x.idx, 1.f);
      else if (x.what == 2) e = mat(x.p, x.n, x.idx);
      else if (i8) e = fill(x.p, x.n, base + x.idx, 2, 0, 0.f, s0);
    }
  }
  return e == hipSuccess ? BLOOM_OK : hip_fail(e);
}

int bloom_sample_workspace_bytes(int32_t batch, int32_t vocab, size_t *bytes) {
  if (!bytes || batch < 0 || vocab < 1 || vocab > (1 << 23)) return BLOOM_EINVAL;
  *bytes = sample_workspace_bytes(batch, vocab);
  return BLOOM_OK;
}

int bloom_sample_tokens(const float *d_logits, int32_t batch, int32_t vocab,
                        const float *d_temperature, const float *d_top_p,
                        const float *d_uniform, int32_t *d_tokens, void *d_ws, size_t ws_bytes,
                        void *stream) {
  if (batch < 0 || vocab < 1 || vocab > (1 << 23)) return BLOOM_EINVAL;
  if (batch == 0) return BLOOM_OK;
  if (!d_logits || !d_temperature || !d_top_p || !d_uniform || !d_tokens || !d_ws)
    return BLOOM_EINVAL;
  if (ws_bytes < sample_workspace_bytes(batch, vocab)) return BLOOM_EWORKSPACE;
  clear_stale_hip_error();
  const hipError_t err = launch_sample_rows(d_logits, batch, vocab, d_temperature, d_top_p,
                                            d_uniform, d_tokens, d_ws, (hipStream_t)stream);
  return err == hipSuccess ? BLOOM_OK : hip_fail(err);
}

int bloom_sample_tokens_static(const float *d_logits, int32_t batch, int32_t vocab,
                               const float *d_temperature, const float *d_top_p,
                               const float *d_uniform, int32_t *d_tokens, void *stream) {
  if (batch < 0 || vocab < 1 || vocab > (1 << 23)) return BLOOM_EINVAL;
  if (batch == 0) return BLOOM_OK;
  if (!d_logits || !d_temperature || !d_top_p || !d_uniform || !d_tokens) return BLOOM_EINVAL;
  if (sample_workspace_bytes(batch, vocab) > (size_t)kSampleScratchBytes) return BLOOM_EWORKSPACE;
  clear_stale_hip_error();
  const hipError_t err = launch_sample_rows_static(d_logits, batch, vocab, d_temperature,
                                                   d_top_p, d_uniform, d_tokens,
                                                   (hipStream_t)stream);
  return err == hipSuccess ? BLOOM_OK : hip_fail(err);
}

int bloom_sample_scratch_limit(int32_t batch, int32_t vocab, int32_t *fits, size_t *max_bytes) {
  if (!fits || !max_bytes || batch < 0 || vocab < 1 || vocab > (1 << 23)) return BLOOM_EINVAL;
  *max_bytes = (size_t)kSampleScratchBytes;
  *fits = sample_workspace_bytes(batch, vocab) <= (size_t)kSampleScratchBytes;
  return BLOOM_OK;
}

int bloom_timer_enable(int32_t max_launches) {
  if (max_launches <= 0) return BLOOM_EINVAL;
  destroy_timer_events();
  g_timer.start.resize(max_launches);
  g_timer.stop.resize(max_launches);
  g_timer.cls.assign(max_launches, 0);
  g_timer.bytes.assign(max_launches, 0.0);
  for (int i = 0; i < max_launches; ++i) {
    if (hipEventCreate(&g_timer.start[i]) != hipSuccess ||
        hipEventCreate(&g_timer.stop[i]) != hipSuccess) {
      g_timer.start.resize(i);
      g_timer.stop.resize(i);
      destroy_timer_events();
      return BLOOM_EHIP;
    }
  }
  g_timer.on = true;
  g_timer.paused = false;
  return BLOOM_OK;
}

int bloom_timer_disable(void) {
  g_timer.on = false;
  destroy_timer_events();
  return BLOOM_OK;
}

int bloom_timer_pause(int32_t paused) {
  g_timer.paused = paused != 0;
  return BLOOM_OK;
}

int bloom_timer_read(int32_t kernel_class, double *total_ms, int32_t *n_launches,
                     double *weight_bytes) {
  if (!total_ms || !n_launches || !weight_bytes) return BLOOM_EINVAL;
  double total = 0.0, bytes = 0.0;
  int n = 0;
  if (g_timer.used > 0 && hipEventSynchronize(g_timer.stop[g_timer.used - 1]) != hipSuccess)
    return BLOOM_EHIP;
  for (int i = 0; i < g_timer.used; ++i) {
    if (kernel_class >= 0 && g_timer.cls[i] != kernel_class) continue;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, g_timer.start[i], g_timer.stop[i]) != hipSuccess)
      return BLOOM_EHIP;
    total += ms;
    bytes += g_timer.bytes[i];
    ++n;
  }
  *total_ms = total;
  *n_launches = n;
  *weight_bytes = bytes;
  return BLOOM_OK;
}

}  // extern "C"
