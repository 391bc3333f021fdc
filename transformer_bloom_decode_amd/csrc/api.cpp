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
#include <cstring>
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
  int lm_blocks;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int act_bytes(const bloom_config *c) { return c->weight_dtype == BLOOM_F32 ? 4 : 2; }
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
  p.xa = take(M * c->hidden * act);
  p.q = take(M * hd * 4);
  p.o = take(M * hd * act);
  p.u = take(M * (size_t)c->ffn * act);
  p.af = take((size_t)batch * c->hidden * act);
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
        part = std::max(part, linear_partial_bytes(plan_linear(wdt, mrows, nk[0], nk[1], false)));
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
  if (c->weight_dtype != BLOOM_F32) {
    const int hd = c->n_head_local * c->head_dim;
    if (c->hidden % 64 || c->ffn % 64 || hd % 64) return BLOOM_EINVAL;
  }
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
  (void)c;
  if (!kv || !kv->k || !kv->v || kv->max_batch <= 0 || kv->max_len <= 0) return BLOOM_EINVAL;
  if (kv->max_len > kMaxLen) return BLOOM_EINVAL;
  if (kv->len < 0 || kv->len > kv->max_len || kv->prompt_len < 0) return BLOOM_EINVAL;
  return BLOOM_OK;
}

// ---------------------------------------------------------------------------
// launch timer
// ---------------------------------------------------------------------------
struct Timer {
  bool on = false;
  bool paused = false;
  bool capturing = false;   // launches being captured into a graph are never timed
  std::vector<hipEvent_t> start, stop;
  std::vector<int> cls;
  std::vector<double> bytes;
  int used = 0;
} g_timer;

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
  (void)st;
  const bool on = g_timer.on && !g_timer.paused && !g_timer.capturing &&
                  g_timer.used < (int)g_timer.start.size();
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
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!side[dev] && hipStreamCreateWithFlags(&side[dev], hipStreamNonBlocking) != hipSuccess)
    side[dev] = nullptr;
  return side[dev];
}

// ---------------------------------------------------------------------------
// one forward pass over `tpr` tokens per row
// ---------------------------------------------------------------------------
int run_forward(const bloom_config *c, const bloom_weights *w, bloom_kv_cache *kv, int batch,
                int tpr, int pos_base, int prompt_len, const int32_t *d_tokens,
                const int32_t *d_valid, int32_t *d_next, float *d_hidden, char *ws,
                hipStream_t st, const int *d_pos = nullptr, float *d_logits = nullptr) {
  const WsPlan wp = plan_ws(c, batch, tpr);
  const bool f32 = c->weight_dtype == BLOOM_F32;
  const int wdt = wtype(c);
  const int M = batch * tpr;
  const int h = c->hidden, H = c->n_head_local, d = c->head_dim, F = c->ffn;
  const int hd = H * d;
  const size_t wb = c->weight_dtype == BLOOM_F32 ? 4 : (c->weight_dtype == BLOOM_BF16 ? 2 : 1);
  const size_t pb = f32 ? 4 : 2;
  const size_t sb = c->weight_dtype == BLOOM_INT8_ROWSCALE ? 2 : 0;
  const size_t act = act_bytes(c);
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

  hipError_t err = launch_embed(f32, d_tokens, w->embed, w->emb_ln_g, w->emb_ln_b, x, M, h,
                                c->vocab, c->embed_ln, c->ln_eps, st);
  if (err != hipSuccess) return hip_fail(err);

  const size_t layer_stride = (size_t)kv->max_batch * H * kv->max_len * d * act;
  const LinearPlan p_qkv = plan_linear(wdt, M, 3 * hd, h, false);
  const LinearPlan p_dense = plan_linear(wdt, M, h, hd, false);
  const LinearPlan p_up = plan_linear(wdt, M, F, h, false);
  const LinearPlan p_down = plan_linear(wdt, M, h, F, false);

  // K-split dense / down projections reduce their partials in the kernel that also adds
  // bias and residual and runs the next LayerNorm (LN2 after dense, the next layer's LN1
  // after down); unsplit ones keep the epilogue in the GEMM and a separate LayerNorm.
  auto fuse_ln = [&](const LinearPlan &p) {
    return !f32 && p.splits > 1 && splitk_resid_ln_supported(h, p.splits);
  };
  // One activation row and a short hidden size: LN1 and LN2 run as the prologue of the
  // QKV and MLP-up GEMVs instead of as launches of their own.
  const bool ln_in_gemv = !f32 && gemv_ln_supported(wdt, M, h);
  bool ln1_done = false;   // xa already holds LN1(x) of this layer
  for (int l = 0; l < c->n_layer; ++l) {
    const bloom_layer_weights &L = w->layers[l];
    void *kc = (char *)kv->k + l * layer_stride;
    void *vc = (char *)kv->v + l * layer_stride;

    if (!ln1_done && !ln_in_gemv) {
      err = launch_layernorm(f32, x, 1, 0, L.ln1_g, L.ln1_b, xa, nullptr, M, h, c->ln_eps, st);
      if (err != hipSuccess) return hip_fail(err);
    }
    ln1_done = false;

    EpiParams e{};
    e.mode = EPI_QKV;
    e.bias = L.b_qkv;
    e.scale = (const uint16_t *)L.s_qkv;
    e.q = q; e.kc = kc; e.vc = vc;
    e.H = H; e.d = d; e.max_len = kv->max_len;
    e.pos_base = pos_base; e.pos_dev = d_pos; e.rows_per_seq = tpr;
    e.q_scale = 1.0f / sqrtf((float)d);
    if (ln_in_gemv)
      err = timed(kernel_class(p_qkv), wbytes(3 * hd, h), st, [&] {
        return launch_gemv_ln(wdt, 3 * hd, h, x, L.ln1_g, L.ln1_b, c->ln_eps, L.w_qkv, e, st);
      });
    else
      err = timed_linear(wdt, p_qkv, xa, L.w_qkv, part, e, st, wbytes(3 * hd, h));
    if (err != hipSuccess) return hip_fail(err);

    err = launch_attention(f32, q, kc, vc, d_valid, o, M, H, d, kv->max_len, c->n_head_total,
                           c->head_offset, tpr, pos_base, d_pos, prompt_len, st);
    if (err != hipSuccess) return hip_fail(err);

    EpiParams r{};
    r.mode = EPI_RESID;
    r.bias = L.b_dense;
    r.scale = (const uint16_t *)L.s_dense;
    r.out = x; r.ld = h;
    const bool fuse_dense = fuse_ln(p_dense);
    err = timed_linear(wdt, p_dense, o, L.w_dense, part, r, st, wbytes(h, hd), !fuse_dense);
    if (err != hipSuccess) return hip_fail(err);

    if (fuse_dense)
      err = launch_splitk_resid_ln(part, p_dense.splits, M, L.s_dense, L.b_dense, x, L.ln2_g,
                                   L.ln2_b, xa, h, c->ln_eps, st);
    else if (!ln_in_gemv)
      err = launch_layernorm(f32, x, 1, 0, L.ln2_g, L.ln2_b, xa, nullptr, M, h, c->ln_eps, st);
    if (err != hipSuccess) return hip_fail(err);

    EpiParams g{};
    g.mode = EPI_GELU;
    g.bias = L.b_up;
    g.scale = (const uint16_t *)L.s_up;
    g.out = u; g.ld = F;
    if (ln_in_gemv && !fuse_dense)
      err = timed(kernel_class(p_up), wbytes(F, h), st, [&] {
        return launch_gemv_ln(wdt, F, h, x, L.ln2_g, L.ln2_b, c->ln_eps, L.w_up, g, st);
      });
    else
      err = timed_linear(wdt, p_up, xa, L.w_up, part, g, st, wbytes(F, h));
    if (err != hipSuccess) return hip_fail(err);

    EpiParams dn{};
    dn.mode = EPI_RESID;
    dn.bias = L.b_down;
    dn.scale = (const uint16_t *)L.s_down;
    dn.out = x; dn.ld = h;
    const bool fuse_down = l + 1 < c->n_layer && fuse_ln(p_down) && !ln_in_gemv;
    err = timed_linear(wdt, p_down, u, L.w_down, part, dn, st, wbytes(h, F), !fuse_down);
    if (err != hipSuccess) return hip_fail(err);
    if (fuse_down) {
      const bloom_layer_weights &N1 = w->layers[l + 1];
      err = launch_splitk_resid_ln(part, p_down.splits, M, L.s_down, L.b_down, x, N1.ln1_g,
                                   N1.ln1_b, xa, h, c->ln_eps, st);
      if (err != hipSuccess) return hip_fail(err);
      ln1_done = true;
    }
  }

  // final LayerNorm of each row's last position, then the tied LM head + argmax (the
  // LM head is skipped when the caller asked for the hidden states only)
  const int nblk = wp.lm_blocks;
  const int wdt_lm = f32 ? WT_F32 : WT_BF16;  // the embedding is never int8
  const double lm_bytes = (double)c->vocab * h * pb;
  err = launch_layernorm(f32, x, tpr, tpr - 1, w->lnf_g, w->lnf_b, af, d_hidden, batch, h,
                         c->ln_eps, st);
  if (err != hipSuccess) return hip_fail(err);
  if (d_logits) {
    // the LM head's float32 logits [batch][vocab] instead of its argmax (sampling), with
    // the greedy head's plan, so a greedy row of the sampler ranks the same values
    for (int r0 = 0; r0 < batch; r0 += 128) {
      const int rows = std::min(128, batch - r0);
      EpiParams e{};
      e.mode = EPI_STORE;
      e.out = d_logits + (size_t)r0 * c->vocab;
      e.ld = c->vocab;
      const LinearPlan p_lm = plan_linear(wdt_lm, rows, c->vocab, h, true);
      err = timed_linear(wdt_lm, p_lm, (const char *)af + (size_t)r0 * h * act, w->embed, part,
                         e, st, lm_bytes);
      if (err != hipSuccess) return hip_fail(err);
    }
    return BLOOM_OK;
  }
  for (int r0 = 0; d_next && r0 < batch; r0 += 128) {
    const int rows = std::min(128, batch - r0);
    EpiParams a{};
    a.mode = EPI_ARGMAX;
    a.am_val = amv + (size_t)r0 * nblk;
    a.am_idx = ami + (size_t)r0 * nblk;
    a.am_stride = nblk;
    const LinearPlan p_lm = plan_linear(wdt_lm, rows, c->vocab, h, true);
    err = timed_linear(wdt_lm, p_lm, (const char *)af + (size_t)r0 * h * act, w->embed, part, a,
                       st, lm_bytes);
    if (err != hipSuccess) return hip_fail(err);
    // this chunk's kernel wrote one partial per row per weight tile
    err = launch_argmax_merge(a.am_val, a.am_idx, nblk, argmax_partials_per_row(p_lm), rows,
                              d_next + r0, st);
    if (err != hipSuccess) return hip_fail(err);
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
  s = run_forward(cfg, w, kv, batch, 1, kv->len, kv->prompt_len, d_tokens, d_valid_len,
                  d_next_tokens, d_hidden_out, (char *)d_ws, (hipStream_t)stream);
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
  const size_t act = act_bytes(cfg);
  const size_t layer_stride =
      (size_t)kv->max_batch * cfg->n_head_local * kv->max_len * cfg->head_dim * act;
  hipError_t err = launch_kv_append(cfg->weight_dtype == BLOOM_F32, d_k, d_v,
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
  const hipError_t err = launch_kv_compact(kv->k, kv->v, cfg->n_layer, cfg->n_head_local,
                                           kv->max_batch, kv->max_len, cfg->head_dim,
                                           act_bytes(cfg), kv->len, keep, n_keep,
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
  const void *X = d_hidden;
  if (!f32) {
    // the same bf16 rounding of the final-LayerNorm state as the greedy LM head's input
    void *af = (char *)d_ws + wp.af;
    const hipError_t e = launch_f32_to_bf16(d_hidden, af, (size_t)batch * h, st);
    if (e != hipSuccess) return hip_fail(e);
    X = af;
  }
  const int wdt_lm = f32 ? WT_F32 : WT_BF16;
  const size_t act = act_bytes(cfg);
  float *part = (float *)((char *)d_ws + wp.part);
  for (int r0 = 0; r0 < batch; r0 += 128) {
    const int rows = std::min(128, batch - r0);
    EpiParams e{};
    e.mode = EPI_STORE;
    e.out = d_logits + (size_t)r0 * cfg->vocab;
    e.ld = cfg->vocab;
    // the greedy LM head's plan (never split), so the logits are the ones it ranks
    const LinearPlan p = plan_linear(wdt_lm, rows, cfg->vocab, h, true);
    const hipError_t err =
        launch_linear(wdt_lm, p, (const char *)X + (size_t)r0 * h * act, w->embed, part, e, st);
    if (err != hipSuccess) return hip_fail(err);
  }
  return BLOOM_OK;
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
