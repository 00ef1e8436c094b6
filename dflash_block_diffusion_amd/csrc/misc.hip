// Small kernels of the step: RMSNorm, embedding gather, longest-prefix
// acceptance, commit/rollback bookkeeping, benchmark draft injection.
#include "common.h"

namespace dfl {

// RMSNorm(z) = z * (mean(z^2) + eps)^-1/2 * g, one work-group per row.
// Each thread owns whole 8-column chunks: one 16-byte load (bf16) or two
// (fp32) per chunk, kept in registers between the reduction and the output,
// and one 16-byte store per chunk (8 consecutive columns are contiguous in the
// tiled layout as well as in a row-major one).  h % 8 == 0, h <= 8192.
constexpr int NORM_CHUNKS = 4;

__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* __restrict__ x, int xtype, int ldx, void* out,
                                                      int otype, int ldo, const float* __restrict__ gain, int h,
                                                      float eps, int fmK) {
  const int row = blockIdx.x;
  const int nch = h >> 3;
  float v[NORM_CHUNKS][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NORM_CHUNKS; ++c) {
    const int ch = threadIdx.x + 256 * c;
    if (ch < nch) {
      if (xtype == T_F32) {
        const float4* p = (const float4*)((const float*)x + (size_t)row * ldx + ch * 8);
        const float4 a = p[0], b = p[1];
        v[c][0] = a.x; v[c][1] = a.y; v[c][2] = a.z; v[c][3] = a.w;
        v[c][4] = b.x; v[c][5] = b.y; v[c][6] = b.z; v[c][7] = b.w;
      } else {
        const uint4 q = *(const uint4*)((const uint16_t*)x + (size_t)row * ldx + ch * 8);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[c][e] = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[c][e] * v[c][e];
    }
  }
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / (float)h + eps);
#pragma unroll
  for (int c = 0; c < NORM_CHUNKS; ++c) {
    const int ch = threadIdx.x + 256 * c;
    if (ch >= nch) continue;
    const int j0 = ch * 8;
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = v[c][e] * r * gain[j0 + e];
    const size_t o = fmK ? fm_index(row, j0, fmK) : (size_t)row * ldo + j0;
    if (otype == T_F32) {
      float4* p = (float4*)((float*)out + o);
      p[0] = float4{y[0], y[1], y[2], y[3]};
      p[1] = float4{y[4], y[5], y[6], y[7]};
    } else {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint32_t lo = f32_to_bf16_bits(y[2 * e]), hi = f32_to_bf16_bits(y[2 * e + 1]);
        if (otype == T_F16) {
          lo = __builtin_bit_cast(uint16_t, (_Float16)bf16_bits_to_f32(lo));
          hi = __builtin_bit_cast(uint16_t, (_Float16)bf16_bits_to_f32(hi));
        }
        w[e] = lo | (hi << 16);
      }
      *(uint4*)((uint16_t*)out + o) = uint4{w[0], w[1], w[2], w[3]};
    }
  }
}

hipError_t launch_rmsnorm(const void* x, int xtype, int ldx, void* out, int otype, int ldo, const float* gain,
                          int rows, int h, float eps, hipStream_t s, int tiled) {
  if (rows <= 0) return hipSuccess;
  if (h % 8 || h > 8 * 256 * NORM_CHUNKS) return hipErrorInvalidValue;
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
