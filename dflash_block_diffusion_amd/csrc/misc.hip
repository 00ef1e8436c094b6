// Small kernels of the step: RMSNorm, embedding gather, longest-prefix
// acceptance, commit/rollback bookkeeping, benchmark draft injection.
#include "common.h"

namespace dfl {

// RMSNorm(z) = z * (mean(z^2) + eps)^-1/2 * g, one work-group per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ x, int xtype, int ldx, void* out,
                                                      int otype, int ldo, const float* __restrict__ gain, int h,
                                                      float eps, int fmK) {
  const int row = blockIdx.x;
  const size_t xb = (size_t)row * ldx, ob = (size_t)row * ldo;
  float ss = 0.f;
  for (int j = threadIdx.x; j < h; j += 256) {
    const float v = load_act(x, xb + j, xtype);
    ss += v * v;
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / (float)h + eps);
  for (int j = threadIdx.x; j < h; j += 256)
    store_act(out, fmK ? fm_index(row, j, fmK) : ob + j, otype, load_act(x, xb + j, xtype) * r * gain[j]);
}

hipError_t launch_rmsnorm(const void* x, int xtype, int ldx, void* out, int otype, int ldo, const float* gain,
                          int rows, int h, float eps, hipStream_t s, int tiled) {
  if (rows <= 0) return hipSuccess;
  const int fmK = (tiled && otype != T_F32) ? h : 0;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, x, xtype, ldx, out, otype, ldo, gain, h, eps, fmK);
  return hipGetLastError();
}

// x[i] = E[token_i]; mask_mode: slot 0 takes tokens[0] (the anchor), the
// other slots the mask token (the drafter's noise block).
__global__ __launch_bounds__(256) void embed_kernel(const void* __restrict__ table, int ttype, int h, int vocab,
                                                    const int32_t* __restrict__ tokens, int mask_mode,
                                                    int mask_token, void* out, int ldo, int32_t* status) {
  const int row = blockIdx.x;
  int tok = (mask_mode && row > 0) ? mask_token : tokens[row];
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0 && status) atomicOr(status, 2);
    tok = tok < 0 ? 0 : vocab - 1;
  }
  const size_t tb = (size_t)tok * h, ob = (size_t)row * ldo;
  if (ttype == T_F32) {
    for (int j = threadIdx.x; j < h; j += 256) ((float*)out)[ob + j] = ((const float*)table)[tb + j];
  } else {
    for (int j = threadIdx.x; j < h; j += 256) ((uint16_t*)out)[ob + j] = ((const uint16_t*)table)[tb + j];
  }
}

hipError_t launch_embed(const void* table, int ttype, int h, int vocab, const int32_t* tokens, int mask_mode,
                        int mask_token, int rows, void* out, int ldo, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, s, table, ttype, h, vocab, tokens, mask_mode,
                     mask_token, out, ldo, status);
  return hipGetLastError();
}

// a = max{k <= B-1 : d_j == y_{j-1} for all j <= k}: the first mismatching
// slot j gives a = j-1; no mismatch gives a = B-1 (all drafts kept, y_{B-1}
// is the bonus token).  One wavefront, B <= 64.
__global__ __launch_bounds__(64) void accept_kernel(const int32_t* block, const int32_t* y, int B, int32_t* acc,
                                                    int32_t* emit, int32_t* next_anchor) {
  const int lane = threadIdx.x;
  const int dj = (lane >= 1 && lane < B) ? block[lane] : 0;
  const int yj = (lane >= 1 && lane < B) ? y[lane - 1] : 0;
  const int nxt = (lane + 1 < B) ? block[lane + 1] : 0;
  const bool miss = lane >= 1 && lane < B && dj != yj;
  const unsigned long long mask = __ballot(miss);
  const int a = mask ? (__ffsll((long long)mask) - 1) - 1 : B - 1;
  const int ya = y[a];
  if (lane < B) emit[lane] = lane < a ? nxt : (lane == a ? ya : -1);
  if (lane == 0) {
    acc[0] = a;
    if (next_anchor) next_anchor[0] = ya;
  }
}

hipError_t launch_accept(const int32_t* block, const int32_t* y, int B, int32_t* acc, int32_t* emit,
                         int32_t* next_anchor, hipStream_t s) {
  hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64), 0, s, block, y, B, acc, emit, next_anchor);
  return hipGetLastError();
}

// Commit cnt = a+1 tokens (a from the device, or host_count during prefill):
// n <- n + cnt, the emitted tokens go to the log at n+1..n+cnt, the cnt
// verified rows become pending drafter context rows.  A commit that would
// leave no room for the next block is refused (status bit 1).
__global__ void commit_kernel(int32_t* scal, const int32_t* d_acc, int host_count, const int32_t* emit,
                              int32_t* tokens, int32_t* acc_log, int acc_log_len, int capacity, int B) {
  const int cnt = d_acc ? d_acc[0] + 1 : host_count;
  const int n = scal[SC_N];
  if (n + cnt + B > capacity) { scal[SC_STATUS] |= 1; return; }
  if (emit) for (int j = 0; j < cnt; ++j) tokens[n + 1 + j] = emit[j];
  scal[SC_N] = n + cnt;
  scal[SC_P] = cnt;
  if (d_acc) {
    acc_log[scal[SC_STEP] % acc_log_len] = cnt - 1;
    scal[SC_STEP] += 1;
  }
}

hipError_t launch_commit(int32_t* scal, const int32_t* d_acc, int host_count, const int32_t* emit,
                         int32_t* tokens, int32_t* acc_log, int acc_log_len, int capacity, int B, hipStream_t s) {
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(1), 0, s, scal, d_acc, host_count, emit, tokens, acc_log,
                     acc_log_len, capacity, B);
  return hipGetLastError();
}

__global__ void set_scalars_kernel(int32_t* scal, int n, int p, int clear) {
  if (n >= 0) scal[SC_N] = n;
  if (p >= 0) scal[SC_P] = p;
  if (clear) { scal[SC_STATUS] = 0; scal[SC_STEP] = 0; }
}

hipError_t launch_set_scalars(int32_t* scal, int n, int p, int clear_status, hipStream_t s) {
  hipLaunchKernelGGL(set_scalars_kernel, dim3(1), dim3(1), 0, s, scal, n, p, clear_status);
  return hipGetLastError();
}

__global__ void copy_i32_kernel(const int32_t* src, int32_t* dst, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) dst[i] = src[i];
}

hipError_t launch_copy_tokens(const int32_t* src, int32_t* dst, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_i32_kernel, dim3((count + 255) / 256), dim3(256), 0, s, src, dst, count);
  return hipGetLastError();
}

__global__ void rollback_kernel(int32_t* scal, int new_len, const int32_t* tokens, int32_t* block) {
  scal[SC_N] = new_len;
  scal[SC_P] = 0;
  if (block) block[0] = tokens[new_len];
}

hipError_t launch_rollback(int32_t* scal, int new_len, const int32_t* tokens, int32_t* block, hipStream_t s) {
  hipLaunchKernelGGL(rollback_kernel, dim3(1), dim3(1), 0, s, scal, new_len, tokens, block);
  return hipGetLastError();
}

// Benchmark harness: drafts 1..k copy the reference stream, draft k+1 is a
// filler token forced to differ from it, later drafts are filler.
__global__ __launch_bounds__(64) void inject_kernel(const int32_t* scal, int32_t* block, int B, const int32_t* ref,
                                                    int ref_len, const int32_t* sched, int n_sched,
                                                    const int32_t* filler, int vocab) {
  const int j = threadIdx.x;
  if (j < 1 || j >= B) return;
  const int n = scal[SC_N];
  const int s = scal[SC_STEP] % n_sched;
  const int k = sched[s];
  const int p = n + j;
  int tok;
  if (j <= k && p < ref_len) {
    tok = ref[p];
  } else {
    tok = filler[(size_t)s * B + j];
    if (j == k + 1 && p < ref_len && tok == ref[p]) tok = (tok + 1) % vocab;
  }
  block[j] = tok;
}

hipError_t launch_inject(const int32_t* scal, int32_t* block, int B, const int32_t* ref, int ref_len,
                         const int32_t* sched, int n_sched, const int32_t* filler, int vocab, hipStream_t s) {
  hipLaunchKernelGGL(inject_kernel, dim3(1), dim3(64), 0, s, scal, block, B, ref, ref_len, sched, n_sched,
                     filler, vocab);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, size_t count, int32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, size_t count, int32_t v, hipStream_t s) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(2048), dim3(256), 0, s, p, count, v);
  return hipGetLastError();
}

__global__ void copy_f32_kernel(const float* src, float* dst, size_t count) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

hipError_t launch_copy_f32(const float* src, float* dst, size_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, dim3(2048), dim3(256), 0, s, src, dst, count);
  return hipGetLastError();
}

}  // namespace dfl
