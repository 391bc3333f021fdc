/*
 * bloom.h -- C ABI of the MI355X (gfx950) BLOOM greedy-decode library.
 *
 * The library runs the hot path of BLOOM text generation with a KV cache: the
 * pre-LayerNorm decoder layer (input LayerNorm, fused QKV projection, ALiBi
 * attention over the cached keys with masked fill and an fp32 softmax, output
 * projection with bias and residual, post-attention LayerNorm, tanh-GeLU MLP),
 * the final LayerNorm and the tied LM head with a greedy argmax, or per-row
 * temperature / top-p sampling from its logits.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "Incredibly Fast BLOOM Inference with DeepSpeed and Accelerate",
 *        Benchmark Environment: greedy generation (do_sample=False) of 100 tokens with
 *        the KV cache on; ms/token = wall time / (batch x tokens).
 *   [P3] "DeepSpeed Inference: Enabling Efficient Inference of Transformer Models at
 *        Unprecedented Scale", Section III.D (Putting It Together): the fused groups
 *        input-LayerNorm + QKV GeMM, attention, post-attention LayerNorm + intermediate
 *        GeMM, bias + residual; Section III.A: small batches are bound by weight reads.
 *   [P4] "Hugging Face BLOOM Inference Optimization": Kernel Fusion with
 *        torch.jit.script (fused tanh GeLU), Efficient PyTorch Implementation (ALiBi
 *        computed once; KV "past" laid out to avoid reshapes), Custom CUDA Kernels and
 *        Hardware Acceleration (masked_fill then a float32 softmax), Webserver
 *        Architecture and Request Handling (a custom generation loop with per-request
 *        parameters, e.g. sampling and top-p, and the extraction of finished requests).
 *
 * Conventions
 *   - Every pointer named d_* (and every pointer inside the structs below) is device
 *     memory allocated and owned by the caller.  The library allocates nothing on
 *     the call path; scratch space comes from the caller's workspace.
 *   - Calls are asynchronous on the given HIP stream (a hipStream_t passed as void*;
 *     NULL = the null stream).  The return value reports only synchronous checks and
 *     launch errors; device faults surface at the caller's next synchronisation.
 *   - Errors: BLOOM_EINVAL (bad shape, null pointer, bad index), BLOOM_EDTYPE (dtype
 *     or dtype combination not built), BLOOM_ECAPACITY (KV cache too short or too
 *     narrow), BLOOM_EWORKSPACE (workspace too small), BLOOM_EHIP (a HIP call
 *     failed).  On any error nothing is launched and no host-side state changes.
 *   - A batch of 0 rows is a valid no-op.
 *   - Calls are re-entrant: concurrent calls (from several threads, on one or several
 *     GPUs) are safe when they use distinct KV caches and workspaces.  The library's
 *     own process-wide state (per-device kernel attributes, the graph-capture stream,
 *     the launch timer) is guarded by locks; the launch timer is one process-wide
 *     record, so concurrent timed calls share it.  bloom_sample_tokens_static shares
 *     one scratch array per GPU (see there).
 *
 * Data types
 *   - weight_dtype BLOOM_F32: all tensors float32 (a generic, unoptimised path);
 *     act_dtype and kv_dtype must be BLOOM_F32.
 *   - weight_dtype BLOOM_BF16: linear weights, embedding, biases and LayerNorm
 *     parameters are bf16; the residual stream, LayerNorm statistics, GEMM
 *     accumulation, softmax and logits are float32.
 *   - weight_dtype BLOOM_INT8_ROWSCALE: as BF16, except the four per-layer linear
 *     weights are int8 [out][in] with one fp16 scale per output row in s_*:
 *     W[r][k] = s[r] * q[r][k] (weight-only).
 *   - act_dtype (BF16 / INT8_ROWSCALE weights): the activations the linears read
 *     (LayerNorm outputs, attention output, GeLU output) are held as bf16
 *     (BLOOM_BF16), fp16 (BLOOM_F16: 8x finer than bf16 at the same size; values
 *     beyond fp16's range, 65504, become infinite) or float32 (BLOOM_F32).  The
 *     vector-ALU GEMV (batches of up to 4 rows) reads them in that type.  The MFMA GEMM
 *     (5+ rows) reads bf16 activations as bf16; fp16 ones on the fp16 MFMA, with the
 *     weights turned into fp16 as they are read (int8 exactly; bf16 exactly from 2^-14
 *     in magnitude, smaller ones to the nearest multiple of 2^-24); float32 ones as two
 *     bf16 planes hi + lo of each value, each multiplied with the weights, which keeps
 *     the product to ~2^-17 of the float32 one.
 *   - act_dtype BLOOM_INT8_ROWSCALE (INT8_ROWSCALE weights only; hidden <= 16384):
 *     W8A8, a variant of DeepSpeed's INT8 inference ([P3] Section VII.B names it
 *     without its scheme).  Each of the four linears' input rows (one token's
 *     LayerNorm output, attention output or GeLU output) is quantised symmetrically
 *     with one float32 scale per row: scale = amax / 127 (amax = the row's largest
 *     magnitude), code = nearest integer, ties to even, to v * (127 / amax) in float32,
 *     clamped to [-127, 127]; a row of zeros has scale 0.  The linear is then
 *     y = scale_row * s[r] * sum_k code[k] q[r][k] + bias (int32 sums on the int8 MFMA
 *     for 5+ rows, float32 sums in the vector-ALU GEMV of up to 4 rows).  The residual stream, q, the final LayerNorm output and the LM head
 *     stay as with F32 activations.
 *   - kv_dtype equals act_dtype, or is BLOOM_INT8_ROWSCALE (any non-F32 weights): an
 *     int8 KV cache holds, per (layer, row, head, slot), head_dim int8 codes of the key
 *     (and of the value) with one float32 scale each in k_scale / v_scale, quantised as
 *     above over the head_dim values; attention multiplies a key's dot product by its
 *     scale and a value's probability weight by its scale.
 *
 * Layouts (all row-major, C order)
 *   embed            [vocab][hidden]             also the LM head (tied embeddings)
 *   w_qkv            [3*n_head_local*head_dim][hidden], rows ordered [head][q,k,v][dim]
 *   w_dense          [hidden][n_head_local*head_dim]
 *   w_up             [ffn][hidden]
 *   w_down           [hidden][ffn]
 *   biases, scales   [out]
 *   LayerNorm g, b   [hidden]
 *   KV cache k, v    [n_layer][max_batch][n_head_local][max_len][head_dim]
 */
#ifndef BLOOM_MI355X_H
#define BLOOM_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bloom_status {
  BLOOM_OK = 0,
  BLOOM_EINVAL = -1,
  BLOOM_EDTYPE = -2,
  BLOOM_ECAPACITY = -3,
  BLOOM_EWORKSPACE = -4,
  BLOOM_EHIP = -5
};

enum bloom_dtype { BLOOM_F32 = 0, BLOOM_BF16 = 1, BLOOM_INT8_ROWSCALE = 2, BLOOM_F16 = 3 };

/* Shape of one BLOOM stack held on this GPU: a whole model, or one tensor-parallel
 * share of it (n_head_local heads starting at global head head_offset, ffn columns of
 * the MLP).  n_head_total fixes the ALiBi slopes.  Requirements (else BLOOM_EINVAL):
 * all sizes > 0; head_offset + n_head_local <= n_head_total; head_dim a power of two
 * in [8, 256]; ln_eps >= 0; for BF16 / INT8_ROWSCALE, hidden, ffn and
 * n_head_local*head_dim multiples of 64.  Device pointers must be 16-byte aligned. */
typedef struct bloom_config {
  int32_t n_layer;
  int32_t hidden;
  int32_t n_head_total;
  int32_t head_offset;
  int32_t n_head_local;
  int32_t head_dim;
  int32_t ffn;
  int32_t vocab;
  int32_t weight_dtype; /* enum bloom_dtype */
  int32_t embed_ln;     /* 1: LayerNorm right after the embedding gather */
  float ln_eps;         /* LayerNorm epsilon (biased variance) */
  int32_t act_dtype;    /* BLOOM_BF16, BLOOM_F16, BLOOM_F32 or BLOOM_INT8_ROWSCALE (W8A8) */
  int32_t kv_dtype;     /* KV cache element type: act_dtype or BLOOM_INT8_ROWSCALE */
} bloom_config;

/* Device pointers of one decoder layer.  s_* are the int8 row scales (fp16) and must be
 * NULL for F32 / BF16 weights. */
typedef struct bloom_layer_weights {
  const void *ln1_g, *ln1_b;
  const void *w_qkv, *b_qkv, *s_qkv;
  const void *w_dense, *b_dense, *s_dense;
  const void *ln2_g, *ln2_b;
  const void *w_up, *b_up, *s_up;
  const void *w_down, *b_down, *s_down;
} bloom_layer_weights;

/* emb_ln_* may be NULL when embed_ln == 0.  `layers` is a HOST array of n_layer
 * entries (each holding device pointers); it is read during the call only.
 * ln_fold (nullable) holds the LayerNorm fold vectors written by bloom_ln_fold for these
 * weights; when set, one-row forward passes of BF16-weight models whose hidden size is
 * above 4096 fold the input and post-attention LayerNorms into the QKV and MLP-up GEMVs
 * (see bloom_ln_fold).  The vectors must be rewritten whenever the weights change. */
typedef struct bloom_weights {
  const void *embed;
  const void *emb_ln_g, *emb_ln_b;
  const void *lnf_g, *lnf_b;
  const bloom_layer_weights *layers;
  const float *ln_fold;
} bloom_weights;

/* KV cache.  k and v are caller-owned device buffers of
 * n_layer * max_batch * n_head_local * max_len * head_dim elements of kv_dtype
 * (float32, bf16, fp16 or int8).  For an int8 cache, k_scale and v_scale are
 * caller-owned float32 device buffers [n_layer][max_batch][n_head_local][max_len]
 * (4-byte aligned; EINVAL if missing), one scale per key / value vector; for other
 * types they are ignored.  len and prompt_len are host-side: bloom_prefill sets prompt_len
 * and len = prompt_len; bloom_decode_step writes slot len and then increments it, and
 * its capacity check uses len.  Slot j holds absolute position j of every row (left
 * padding slots are written but never attended).  A caller may reset len to 0.
 * max_len is at most 2^20.
 * d_len (device int32 [1], 4-byte aligned, nullable) is the same length kept in device
 * memory ("DeepSpeed Inference ...", Section III.D: the forward is captured once as a
 * graph and replayed): bloom_prefill sets *d_len = prompt_len on the device,
 * bloom_generate sets it to the final length, and bloom_decode_step reads the step's
 * position from *d_len (not from len) and advances it by one on the device, so a
 * caller may capture one bloom_decode_step call in a graph and replay it.  Replays do
 * not advance the host-side len; the device guards the cache: a step that finds
 * *d_len == max_len writes no slot, attends over slots [.., max_len - 1], leaves
 * *d_len at max_len, and its outputs are undefined. */
typedef struct bloom_kv_cache {
  void *k, *v;
  int32_t max_batch, max_len;
  int32_t len;
  int32_t prompt_len;
  int32_t *d_len;
  void *k_scale, *v_scale;
} bloom_kv_cache;

/* Seeded synthetic weights, written on the GPU into the caller's buffers behind w (the
 * const pointers of bloom_weights are written through here).  Specification: every
 * element is a pure function of (seed, tensor id, flat row-major index i):
 *   key = SM(seed << 32 xor id), r = SM(key + i), with SM the SplitMix64 finaliser
 *   (Steele, Lea and Flood, "Fast splittable pseudorandom number generators", 2014);
 *   normal: z = (r & 0xffff) + (r >> 16 & 0xffff) + (r >> 32 & 0xffff) + (r >> 48)
 *     - 131070 (Irwin-Hall of four 16-bit uniforms, centred), v = mean + fp32(z) * c with
 *     c = fp32(sigma / sqrt((65536^2 - 1) / 3)), float32 round-to-nearest-even steps (no
 *     fused multiply-add), stored as float32 (F32 models) or bf16 (nearest even);
 *   int8 weights: r mod 255 - 127; fp16 row scales: fp16 of
 *     fp32(sigma / sqrt((255^2 - 1) / 12)) * (0.5 + (r >> 40) * 2^-24) in float32.
 * Tensor ids: embed 1, emb_ln_g 2, emb_ln_b 3, lnf_g 4, lnf_b 5; layer l: 1024 + 16 l +
 * the field's index in (ln1_g, ln1_b, w_qkv, b_qkv, w_dense, b_dense, ln2_g, ln2_b,
 * w_up, b_up, w_down, b_down, s_qkv, s_dense, s_up, s_down).  LayerNorm gammas (*_g)
 * have mean 1, everything else mean 0; linear weights and the embedding N(0, sigma),
 * biases and betas N(0, sigma).  Asynchronous on `stream`; EINVAL for a bad config,
 * missing pointers or sigma < 0. */
int bloom_init_weights(const bloom_config *cfg, const bloom_weights *w, uint64_t seed,
                       double sigma, void *stream);

/* Human-readable text for a status code. */
const char *bloom_status_string(int status);

/* Text of the HIP error behind the last BLOOM_EHIP returned on the calling thread. */
const char *bloom_last_hip_error(void);

/* Bytes of device workspace bloom_prefill / bloom_decode_step need for batches of up
 * to max_batch rows and prompts of up to max_prompt tokens.  Writes *bytes. */
int bloom_workspace_bytes(const bloom_config *cfg, int32_t max_batch, int32_t max_prompt,
                          size_t *bytes);

/* Prompt pass ([P1] Benchmark Environment: generation starts from a short prompt).
 * d_tokens [batch][prompt_len] int32, LEFT-padded: row b has d_valid_len[b] real
 * tokens (1 <= valid_len <= prompt_len) at its right end; pad ids are ignored.
 * Token ids are not checked on the host (they are device data): an id outside
 * [0, vocab) is clamped to the nearest valid id by the embedding gather.
 * Runs every prompt position through the stack, writes KV slots [0, prompt_len),
 * sets kv->prompt_len = kv->len = prompt_len, and writes the greedy next token of
 * each row to d_next_tokens [batch] (lowest id among equal float32 logits).
 * d_hidden_out (nullable) [batch][hidden] float32 receives the final-LayerNorm state
 * of each row's last position.  d_next_tokens may be NULL when d_hidden_out is not:
 * the LM head and its argmax are then skipped (a caller that samples its tokens with
 * bloom_lm_logits + bloom_sample_tokens).  ECAPACITY if batch > kv->max_batch or
 * prompt_len > kv->max_len. */
int bloom_prefill(const bloom_config *cfg, const bloom_weights *w, bloom_kv_cache *kv,
                  int32_t batch, int32_t prompt_len, const int32_t *d_tokens,
                  const int32_t *d_valid_len, int32_t *d_next_tokens, float *d_hidden_out,
                  void *d_ws, size_t ws_bytes, void *stream);

/* One generation step ([P1] Benchmark Environment; [P3] III.D fused groups).
 * d_tokens [batch] int32 are the tokens at position kv->len (ids outside [0, vocab)
 * clamped, as in bloom_prefill); d_valid_len [batch] are
 * the same valid prompt lengths given to bloom_prefill (left-pad masking).  Writes
 * KV slot kv->len of every layer, attends over slots [prompt_len - valid_len[b],
 * kv->len], writes the greedy next token to d_next_tokens and optionally the
 * final-LayerNorm state to d_hidden_out [batch][hidden], then increments kv->len.
 * With kv->d_len set, the position is *d_len instead (read on the device, advanced by
 * one on the device at the end of the step), so the call can be captured in a graph.
 * As in bloom_prefill, d_next_tokens may be NULL when d_hidden_out is not (no LM head).
 * ECAPACITY if kv->len >= kv->max_len or batch > kv->max_batch; EINVAL if
 * bloom_prefill has not run (kv->prompt_len <= 0). */
int bloom_decode_step(const bloom_config *cfg, const bloom_weights *w, bloom_kv_cache *kv,
                      int32_t batch, const int32_t *d_tokens, const int32_t *d_valid_len,
                      int32_t *d_next_tokens, float *d_hidden_out, void *d_ws,
                      size_t ws_bytes, void *stream);

/* Per-row generation control of bloom_generate ("Hugging Face BLOOM Inference
 * Optimization", Webserver Architecture and Request Handling: a custom generation loop
 * with per-request parameters in one batch).  Row b finishes at the step where it
 * emits eos_id (that token is kept) or where it has d_max_new[b] tokens; its later
 * steps record pad_id (the row is still computed, fed pad_id, so its KV slots and
 * hidden states of those steps are those of pad tokens).  eos_id < 0: no end token;
 * d_max_new (device [batch] int32) nullable: no per-row limit; d_out_len (device
 * [batch] int32, nullable) receives each row's token count (n_new if it never
 * finished).  Finished rows can be taken out between calls with kv_cache_compact.
 * Sampling (the same page: sampling parameters per member of the batch): with
 * d_temperature, d_top_p (device float32 [batch]) and d_uniform (device float32
 * [n_new][batch], the caller's random numbers in [0, 1); all n_new * batch values are
 * read, so a shorter buffer is read out of bounds) set, every step's token is
 * drawn as bloom_sample_tokens does, from the tied LM head's logits (written to the
 * caller's d_logits [batch][vocab] float32 scratch) with d_uniform[step][b]; rows with
 * temperature <= 0 stay greedy.  d_sample_ws is a device workspace of
 * bloom_sample_workspace_bytes(batch, vocab) bytes.  All five NULL: greedy. */
typedef struct {
  int32_t eos_id;
  int32_t pad_id;
  const int32_t *d_max_new;
  int32_t *d_out_len;
  const float *d_temperature;
  const float *d_top_p;
  const float *d_uniform;
  float *d_logits;
  void *d_sample_ws;
  size_t sample_ws_bytes;
} bloom_gen_control;

/* Generation loop ([P1] Benchmark Environment: greedy generation of new tokens with the
 * KV cache; [P3] III.D: launch overhead at small batch is removed with graphs; [P4]
 * Webserver Architecture: per-row stop rules and sampling through ctl, above).
 * Runs the prompt pass (as bloom_prefill), then n_new - 1 decode steps: the first
 * eagerly, the rest as replays of one HIP graph captured from a decode step whose KV
 * position and input tokens live in device memory.  d_ids [n_new][batch] int32
 * receives the token of every step (row 0 from the prompt pass); d_hidden (nullable)
 * [n_new][batch][hidden] float32 the final-LayerNorm states; ctl (host struct,
 * nullable: plain greedy) the per-row stop rule above.  kv->len ends at prompt_len +
 * n_new - 1.  Returns after the generation has finished (the graph is released).
 * ECAPACITY if prompt_len + n_new - 1 > kv->max_len or batch > kv->max_batch; EINVAL if
 * ctl->eos_id >= vocab or the sampling fields are set in part; EWORKSPACE if the
 * workspace is smaller than bloom_workspace_bytes(cfg, batch, prompt_len) or the
 * sampling workspace than bloom_sample_workspace_bytes(batch, vocab). */
int bloom_generate(const bloom_config *cfg, const bloom_weights *w, bloom_kv_cache *kv,
                   int32_t batch, int32_t prompt_len, const int32_t *d_tokens,
                   const int32_t *d_valid_len, int32_t n_new, int32_t *d_ids, float *d_hidden,
                   const bloom_gen_control *ctl, void *d_ws, size_t ws_bytes, void *stream);

/* Logits of the tied LM head for caller-held final-LayerNorm states ("Hugging Face
 * BLOOM Inference Optimization", Webserver Architecture and Request Handling: the custom
 * generation loop needs the distribution, not only its argmax, to sample).
 * d_hidden [batch][hidden] float32 (as bloom_prefill / bloom_decode_step write to
 * d_hidden_out) -> d_logits [batch][vocab] float32, d_logits[b][v] = hidden_b . E_v with
 * hidden rounded to bf16 for BF16 / INT8 models (the same operands and kernel plan as
 * the greedy LM head, so the argmax of these logits is the token bloom_decode_step
 * returns).  Buffers are caller-owned device memory; the workspace is
 * bloom_workspace_bytes(cfg, batch, 1).  Only w->embed is read.  Asynchronous. */
int bloom_lm_logits(const bloom_config *cfg, const bloom_weights *w, int32_t batch,
                    const float *d_hidden, float *d_logits, void *d_ws, size_t ws_bytes,
                    void *stream);

/* Per-row sampling ("Hugging Face BLOOM Inference Optimization", Webserver Architecture
 * and Request Handling: different sampling parameters, e.g. top-p, for each member of a
 * batch; nucleus sampling as defined by Holtzman et al., "The Curious Case of Neural
 * Text Degeneration", Section 3.1).  For row b of d_logits [batch][vocab] float32 (no
 * NaN), with T = d_temperature[b], p = d_top_p[b], u = d_uniform[b] (device float32
 * [batch] each; u is clamped to [0, 1)):
 *   T <= 0, or T so small that 1/T overflows float32 (below ~2.9e-39): the greedy
 *   token (lowest id among the largest logits);
 *   else q = softmax(logits / T); the nucleus is the shortest run of tokens in
 *   decreasing q whose mass reaches p, plus every token tied with its last one (p >= 1:
 *   all tokens; p <= 0: the largest logits only); the token is the first id, in
 *   increasing id order over the nucleus, whose cumulative mass exceeds u times the
 *   nucleus mass.
 * Writes d_tokens [batch] int32.  Probabilities are float32, masses exact sums of
 * 2^-40 fixed-point units (the same inputs give the same tokens).  The random numbers
 * are the caller's.  d_ws: device workspace of bloom_sample_workspace_bytes(batch,
 * vocab) bytes (partial results between the kernels; its contents need no
 * initialisation).  EINVAL for batch < 0, vocab outside [1, 2^23] or a NULL pointer;
 * EWORKSPACE if ws_bytes is too small.  Asynchronous on `stream`. */
int bloom_sample_tokens(const float *d_logits, int32_t batch, int32_t vocab,
                        const float *d_temperature, const float *d_top_p,
                        const float *d_uniform, int32_t *d_tokens, void *d_ws,
                        size_t ws_bytes, void *stream);

/* Workspace bytes bloom_sample_tokens needs for `batch` rows of `vocab` logits. */
int bloom_sample_workspace_bytes(int32_t batch, int32_t vocab, size_t *bytes);

/* bloom_sample_tokens without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same inputs, outputs and results as bloom_sample_tokens; the
 * partial results live in a scratch array the library holds in each GPU's memory
 * (16 MiB per GPU, kept until the process ends; nothing is allocated by the call).
 * Calls on one GPU share that array: calls that overlap in time on one GPU race, so a
 * caller serialises them (one stream, or its own ordering).  EWORKSPACE if the rows
 * need more scratch than the array holds (bloom_sample_scratch_limit tells; up to
 * batch 1396 at vocab 250880); EINVAL as bloom_sample_tokens. */
int bloom_sample_tokens_static(const float *d_logits, int32_t batch, int32_t vocab,
                               const float *d_temperature, const float *d_top_p,
                               const float *d_uniform, int32_t *d_tokens, void *stream);

/* Whether bloom_sample_tokens_static accepts `batch` rows of `vocab` logits (*fits = 1)
 * and the scratch array's size in bytes (*max_bytes).  Host-only. */
int bloom_sample_scratch_limit(int32_t batch, int32_t vocab, int32_t *fits, size_t *max_bytes);

/* Standalone fused ALiBi bias + masked fill + float32 softmax ([P4] Custom CUDA Kernels
 * and Hardware Acceleration; Efficient PyTorch Implementation for ALiBi).
 * d_scores [B][H][Q][K] (in_dtype BLOOM_BF16 or BLOOM_F32) are attention scores
 * already scaled by 1/sqrt(head_dim).  Row b keeps keys j >= K - d_valid_len[b] (left
 * padding; 0 <= valid_len <= K); query i sits at key position K - Q + i and keeps keys
 * j <= K - Q + i.  Head h uses the ALiBi slope of global head head_offset + h of an
 * n_head_total-head model.  p = softmax over kept keys of score + slope * (j - (K-Q+i));
 * dropped keys get exactly 0, and a row with no kept key is all 0.  All arithmetic is
 * float32; d_probs [B][H][Q][K] is written in out_dtype (BLOOM_F32 or BLOOM_BF16). */
int alibi_masked_softmax(const void *d_scores, int32_t in_dtype, const int32_t *d_valid_len,
                         int32_t B, int32_t H, int32_t Q, int32_t K, int32_t n_head_total,
                         int32_t head_offset, void *d_probs, int32_t out_dtype, void *stream);

/* Copy n_new new key/value vectors into the cache ([P4] Efficient PyTorch
 * Implementation: the KV "past" kept in a layout that needs no reshape or transpose).
 * d_k, d_v [batch][n_head_local][n_new][head_dim] (the cache's element type; float32
 * for an int8 cache, which quantises each vector as the forward pass does and writes
 * its scale) go to slots [pos, pos + n_new) of layer `layer`, rows 0..batch-1.  Does
 * not change kv->len.
 * ECAPACITY if pos + n_new > kv->max_len or batch > kv->max_batch. */
int kv_cache_append(const bloom_config *cfg, bloom_kv_cache *kv, int32_t layer, int32_t batch,
                    int32_t pos, const void *d_k, const void *d_v, int32_t n_new, void *stream);

/* One linear layer of the decoder as a standalone call ("DeepSpeed Inference ...",
 * Section III.C: the weight-streaming GeMM of the QKV, output, MLP-up and MLP-down
 * projections; the same kernels and plans as the forward pass at these sizes):
 *   y[m][n] = sum_k x[m][k] W[n][k]  (* s[n] for int8 weights)  (+ b[n] if d_b),
 * for m < M, n < N.  d_x float32 [M][K] is first stored as the forward pass stores a
 * linear's input under cfg->act_dtype (bf16 or fp16 rounding; float32 / two bf16
 * planes; int8 codes with one scale per row, see Data types); d_w [N][K] of
 * cfg->weight_dtype; d_s fp16 [N] for INT8_ROWSCALE weights (NULL otherwise); d_b [N]
 * bias in the parameter type (bf16; float32 for F32 weights), nullable; d_y float32
 * [M][N].  The other fields of cfg only select types.  EINVAL for M < 0, N < 1, K < 1,
 * K not a multiple of 64 (BF16 / INT8_ROWSCALE weights) or missing pointers;
 * EWORKSPACE if ws_bytes < bloom_linear_workspace_bytes (d_ws may be NULL when that is
 * 0).  M = 0 is a no-op. */
int bloom_linear_workspace_bytes(const bloom_config *cfg, int32_t M, int32_t N, int32_t K,
                                 size_t *bytes);
int bloom_linear(const bloom_config *cfg, int32_t M, int32_t N, int32_t K, const float *d_x,
                 const void *d_w, const void *d_s, const void *d_b, float *d_y, void *d_ws,
                 size_t ws_bytes, void *stream);

/* LayerNorm fold ("DeepSpeed Inference ...", Section III.D: the input LayerNorm is
 * fused with the QKV GeMM and the post-attention LayerNorm with the intermediate GeMM).
 * A LayerNorm followed by a linear is, per output n,
 *   y_n = sum_k W[n][k] (g_k (x_k - mean) rstd + b_k) + bias_n
 *       = rstd (sum_k W[n][k] g_k x_k - mean c_n) + d_n,
 *   c_n = sum_k W[n][k] g_k,   d_n = sum_k W[n][k] b_k + bias_n,
 * so the linear can run on g * x while the row's statistics are formed beside it.  With
 * the vectors c and d, a one-row pass has the residual epilogue of the dense (MLP-down)
 * projection also store g2 * x (the next layer's g1 * x) in the activation type, and
 * that projection's blocks add their sums of x and x^2 to integer accumulators in the
 * workspace (one 64-bit fixed-point value per block and sum: x in 2^-32, x^2 in 2^-24
 * units, so that the totals do not depend on the order of the additions; valid while
 * |sum of x| < 2^31 and the sum of x^2 < 2^38 per row, and below 1e-6 relative error
 * of the variance while it is above about 0.007 at hidden 14336; the pass's embedding
 * launch zeroes them).  The MLP-up (next QKV) GEMV reads g * x as its activations, forms
 * mean and rstd of x from the totals and applies the formula in its epilogue, and the
 * separate LayerNorm launches go away.  Activations are then rounded as g * x instead
 * of as the LayerNorm output.
 * bloom_ln_fold writes, for every layer l, float32 [c_qkv (3 Hd) | d_qkv (3 Hd) | c_up (F)
 * | d_up (F)] at d_fold + l * (6 Hd + 2 F) (sums in float64, rounded once), from the
 * BF16 weights behind w; bloom_ln_fold_bytes gives the size.  Asynchronous on `stream`.
 * EDTYPE for weights other than BF16; EINVAL for missing pointers; EWORKSPACE if bytes
 * is too small. */
int bloom_ln_fold_bytes(const bloom_config *cfg, size_t *bytes);
int bloom_ln_fold(const bloom_config *cfg, const bloom_weights *w, float *d_fold,
                  size_t bytes, void *stream);

/* Dynamic batch extraction ("Hugging Face BLOOM Inference Optimization", Webserver
 * Architecture and Request Handling: requests that have finished are taken out of the
 * running batch instead of waiting for the longest one).  Compacts the KV cache in
 * place: for i < n_keep, row i of every layer and head takes the slots [0, kv->len) of
 * row keep[i] (an int8 cache's slot scales with them).  keep is a HOST array of n_keep row indices, strictly increasing, each
 * in [0, batch); rows n_keep .. batch-1 keep stale contents.  The caller compacts its
 * own per-row arrays (tokens, valid lengths) the same way and continues with batch =
 * n_keep.  Asynchronous on `stream` (the indices are passed by value, so keep may be
 * reused at once).  EINVAL for a bad index list, ECAPACITY if batch > kv->max_batch;
 * n_keep = 0 is a no-op.  Does not change kv->len or kv->prompt_len. */
int kv_cache_compact(const bloom_config *cfg, bloom_kv_cache *kv, int32_t batch,
                     const int32_t *keep, int32_t n_keep, void *stream);

/* Launch timer for measurement.  While enabled (and not paused), every launch of the
 * library's linear-layer kernels (the weight-streaming GEMV / GEMM of the four layer
 * linears and the LM head) is made with hipExtLaunchKernelGGL and a pair of hipEvents,
 * which the kernel's dispatch packet itself timestamps, for up to max_launches
 * launches; each is tagged with its kernel class below.
 * bloom_timer_enable creates the events (not on the call path) and clears old
 * records; bloom_timer_read synchronises on the last event and returns, for one
 * kernel class (or all, kernel_class = -1), the summed launch time in ms, the number
 * of launches and the summed weight bytes (weights, biases, scales) they streamed;
 * reading does not clear.  (A split-K reduction kernel is not included.) */
enum bloom_kernel_class {
  BLOOM_KERNEL_GEMV = 2,        /* vector-ALU GEMV (up to 4 rows) */
  BLOOM_KERNEL_GEMM_F32 = 5,    /* float32 model */
  BLOOM_KERNEL_GEMM_LDS = 6     /* direct-to-LDS MFMA GEMM (5+ rows, bf16 or int8 weights) */
};
int bloom_timer_enable(int32_t max_launches);
int bloom_timer_disable(void);
int bloom_timer_read(int32_t kernel_class, double *total_ms, int32_t *n_launches,
                     double *weight_bytes);
/* While an enabled timer is paused (paused != 0) launches are not recorded. */
int bloom_timer_pause(int32_t paused);

#ifdef __cplusplus
}
#endif

#endif /* BLOOM_MI355X_H */
