// Device-side bookkeeping of the greedy generation loop ("Incredibly Fast BLOOM
// Inference with DeepSpeed and Accelerate", Benchmark Environment: greedy decoding of
// new tokens with the KV cache).  The decode step that bloom_generate captures in a HIP
// graph reads its KV position and input tokens from device memory, so one graph serves
// every step; these kernels record each step's output, apply the per-row stop rule and
// advance the position.
#include "common.hpp"
#include "kernels.hpp"

namespace bl {

__global__ void k_gen_init(int *__restrict__ state, int pos, int step, int *__restrict__ done,
                           int batch) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < batch; i += gridDim.x * blockDim.x)
    done[i] = 0;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    state[0] = pos;
    state[1] = step;
  }
}

// One block: every thread reads the step index before thread 0 advances it.  Row i's
// token of step t is next[i] until the row has finished, pad_id after; a row finishes
// at the step where it emits eos_id (that token is kept) or reaches max_new[i] tokens
// ("Hugging Face BLOOM Inference Optimization", Webserver Architecture and Request
// Handling: per-request limits in one batch).  out_len[i] counts the row's tokens.
__global__ __launch_bounds__(1024) void k_gen_record(const int *__restrict__ next,
                                                     int *__restrict__ cur, int *__restrict__ ids,
                                                     const float *__restrict__ hfix,
                                                     float *__restrict__ hout, int *state,
                                                     int batch, int hidden, GenControl gc) {
  const int t = state[1];
  for (int i = threadIdx.x; i < batch; i += blockDim.x) {
    int tok = next[i];
    if (gc.done[i]) {
      tok = gc.pad_id;
    } else {
      if (gc.out_len) gc.out_len[i] = t + 1;
      if ((gc.eos_id >= 0 && tok == gc.eos_id) || (gc.max_new && t + 1 >= gc.max_new[i]))
        gc.done[i] = 1;
    }
    ids[(size_t)t * batch + i] = tok;
    cur[i] = tok;
  }
  if (hout) {
    const size_t n = (size_t)batch * hidden;
    float *dst = hout + (size_t)t * n;
    for (size_t i = threadIdx.x; i < n; i += blockDim.x) dst[i] = hfix[i];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    state[0] += 1;
    state[1] = t + 1;
  }
}

// Device-resident KV length of a cache (bloom_kv_cache.d_len).
__global__ void k_len_update(int *len, int set, int add, int max_len) {
  if (threadIdx.x == 0) *len = set >= 0 ? set : min(*len + add, max_len);
}

hipError_t launch_len_update(int *len, int set, int add, int max_len, hipStream_t st) {
  hipLaunchKernelGGL(k_len_update, dim3(1), dim3(64), 0, st, len, set, add, max_len);
  return hipGetLastError();
}

hipError_t launch_gen_init(int *state, int pos, int step, int *done, int batch, hipStream_t st) {
  hipLaunchKernelGGL(k_gen_init, dim3(1), dim3(256), 0, st, state, pos, step, done, batch);
  return hipGetLastError();
}

hipError_t launch_gen_record(const int *next, int *cur, int *ids, const float *hfix, float *hout,
                             int *state, int batch, int hidden, const GenControl &gc,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_gen_record, dim3(1), dim3(1024), 0, st, next, cur, ids, hfix, hout, state,
                     batch, hidden, gc);
  return hipGetLastError();
}

}  // namespace bl
