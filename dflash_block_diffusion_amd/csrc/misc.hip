// Small kernels of the step: RMSNorm, embedding gather, longest-prefix
// acceptance, commit/rollback bookkeeping, benchmark draft injection.
#include "common.h"

namespace dfl {

// Residual update + RMSNorm(z) = z * (mean(z^2) + eps)^-1/2 * g, one
// work-group per row.  The producing GEMM left fp32 partial sums of S K
// ranges; they are added here in split order, rounded to the activation
// format (the GEMM output's materialisation point), added to the residual
// stream and rounded again, then normalised.  Each thread owns whole 8-column
// chunks, kept in registers between the reduction and the output, and writes
// one 16-byte store per chunk (8 consecutive columns are contiguous in the
// tiled layout as well as in a row-major one).  h % 8 == 0, h <= 8192.
__device__ __forceinline__ void store8_act(void* p, size_t i, int t, const float (&y)[8],
                                           int32_t* status = nullptr) {
  if (t == T_F32) {
    float4* q = (float4*)((float*)p + i);
    q[0] = float4{y[0], y[1], y[2], y[3]};
    q[1] = float4{y[4], y[5], y[6], y[7]};
    return;
  }
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t lo = f32_to_bf16_bits(y[2 * e]), hi = f32_to_bf16_bits(y[2 * e + 1]);
    if (t == T_F16) {
      flag_f16_range(t, bf16_bits_to_f32(lo), status);
      flag_f16_range(t, bf16_bits_to_f32(hi), status);
      lo = __builtin_bit_cast(uint16_t, (_Float16)bf16_bits_to_f32(lo));
      hi = __builtin_bit_cast(uint16_t, (_Float16)bf16_bits_to_f32(hi));
    }
    w[e] = lo | (hi << 16);
  }
  *(uint4*)((uint16_t*)p + i) = uint4{w[0], w[1], w[2], w[3]};
}

// one thread per 8-column chunk (blockDim = h/8 rounded up to a wave, <= 1024).
// Every load of the row (the splits' partial sums, the residual chunk, the
// gains) is issued before any loaded value is used, so the kernel waits for
// memory once rather than once per operand.
__global__ __launch_bounds__(1024) void norm_kernel(NormCall c) {
  const int row = blockIdx.x;
  const int nch = c.h >> 3;
  const int ch = threadIdx.x;
  const bool live = ch < nch;
  const int j0 = live ? ch * 8 : 0;
  const int rt = c.xtype;                       // activation (rounding) type of the stack
  float4 pa[MAX_SPLITS], pb[MAX_SPLITS];
  float4 xa = {0.f, 0.f, 0.f, 0.f}, xb = xa;    // fp32 residual chunk, or the 16-bit one in xa's bits
  float g[8];
  if (live) {
    if (c.mode != NORM_ONLY) {
      const float* q = c.in.p + (size_t)row * c.in.ld + j0;
#pragma unroll
      for (int s = 0; s < MAX_SPLITS; ++s) {
        if (s < c.in.S) {
          pa[s] = *(const float4*)(q + (size_t)s * c.in.stride);
          pb[s] = *(const float4*)(q + (size_t)s * c.in.stride + 4);
        }
      }
    }
    if (c.mode != NORM_PROJ) {
      const size_t xi = (size_t)row * c.ldx + j0;
      if (c.xtype == T_F32) {
        xa = *(const float4*)((const float*)c.x + xi);
        xb = *(const float4*)((const float*)c.x + xi + 4);
      } else {
        xa = __builtin_bit_cast(float4, *(const uint4*)((const uint16_t*)c.x + xi));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = c.gain[j0 + e];
  }
  float v[8];
  if (c.mode != NORM_PROJ) {
    if (c.xtype == T_F32) {
      v[0] = xa.x; v[1] = xa.y; v[2] = xa.z; v[3] = xa.w; v[4] = xb.x; v[5] = xb.y; v[6] = xb.z; v[7] = xb.w;
    } else {
      const uint4 q = __builtin_bit_cast(uint4, xa);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hb = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        v[e] = c.xtype == T_BF16 ? bf16_bits_to_f32(hb) : (float)__builtin_bit_cast(_Float16, (uint16_t)hb);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  if (live && c.mode != NORM_ONLY) {
    // the splits are added in split order
    float y[8] = {pa[0].x, pa[0].y, pa[0].z, pa[0].w, pb[0].x, pb[0].y, pb[0].z, pb[0].w};
#pragma unroll
    for (int s = 1; s < MAX_SPLITS; ++s) {
      if (s < c.in.S) {
        y[0] = y[0] + pa[s].x; y[1] = y[1] + pa[s].y; y[2] = y[2] + pa[s].z; y[3] = y[3] + pa[s].w;
        y[4] = y[4] + pb[s].x; y[5] = y[5] + pb[s].y; y[6] = y[6] + pb[s].z; y[7] = y[7] + pb[s].w;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = c.mode == NORM_RESID ? act_round(rt, v[e] + act_round(rt, y[e])) : act_round(rt, y[e]);
    if (c.mode == NORM_RESID) {
      store8_act(c.x, (size_t)row * c.ldx + j0, c.xtype, v);
      if (c.side) {
        const int col = c.side_col0 + j0;
        const size_t o = c.side_type == T_F32 ? (size_t)row * c.ld_side + col : fm_index(row, col, c.ld_side);
        store8_act(c.side, o, c.side_type, v, c.status);
      }
    }
  }
  if (!live) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
  ss = wave_sum(ss);
  __shared__ float part[16];
  const int nw = (blockDim.x + 63) >> 6;
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  // fixed-order sum of the wave partials
  float tot = part[0];
  for (int w = 1; w < nw; ++w) tot = tot + part[w];
  const float r = 1.0f / sqrtf(tot / (float)c.h + c.eps);
  if (!live) return;
  const int fmK = (c.tiled && c.otype != T_F32) ? c.h : 0;
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = v[e] * r * g[e];
  const size_t o = fmK ? fm_index(row, j0, fmK) : (size_t)row * c.ldo + j0;
  store8_act(c.out, o, c.otype, y, c.status);
}

// 8 fp32 values -> 8 16-bit codes: bf16 (round to nearest even), or for
// OT = T_F16 the fp16 encoding of that bf16 value; bad is set when an fp16
// code lies outside the finite fp16 range
template <int OT>
__device__ __forceinline__ uint4 pack8_act(const float (&y)[8], bool& bad) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w[e] = pack_bf16_rne(y[2 * e], y[2 * e + 1]);
    if (OT == T_F16) {
      const float fl = __uint_as_float(w[e] << 16), fh = __uint_as_float(w[e] & 0xffff0000u);
      bad = bad || !(fabsf(fl) <= 65504.0f) || !(fabsf(fh) <= 65504.0f);
      w[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)fl) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)fh) << 16);
    }
  }
  return uint4{w[0], w[1], w[2], w[3]};
}

// The case every bf16-activation step takes: a bf16 residual stream, a tiled
// 16-bit output (OT = T_BF16, or T_F16 for the fp16 encoding of the bf16
// value), SS pending splits (0: NORM_ONLY) and h a multiple of 512, so that
// every thread owns exactly one chunk and every wave is full.  The arithmetic
// and its order are norm_kernel's; what goes is the run-time type and mode
// dispatch, the dead-lane handling, the per-element range atomics (one
// atomic per wave that met an out-of-range fp16 code), the integer bf16
// rounding (one v_cvt_pk_bf16_f32 per pair instead) and the LDS shuffles of
// the wave sum (DPP instead), which on this one-wave-chain-per-row kernel
// cost about as much time as the memory round trips: 6.2 -> 4.0 us a launch
// at 32 rows x 4096.  Only the wave sum's association order differs.
template <int SS, int OT>
__global__ __launch_bounds__(1024) void norm_bf16_kernel(NormCall c) {
  const int row = blockIdx.x;
  const int j0 = threadIdx.x * 8;
  float4 pa[SS > 0 ? SS : 1], pb[SS > 0 ? SS : 1];
  if (SS > 0) {
    const float* q = c.in.p + (size_t)row * c.in.ld + j0;
#pragma unroll
    for (int s = 0; s < SS; ++s) {
      pa[s] = *(const float4*)(q + (size_t)s * c.in.stride);
      pb[s] = *(const float4*)(q + (size_t)s * c.in.stride + 4);
    }
  }
  uint16_t* xr = (uint16_t*)c.x + (size_t)row * c.ldx + j0;
  const uint4 xw = *(const uint4*)xr;
  const float4 g0 = *(const float4*)(c.gain + j0), g1 = *(const float4*)(c.gain + j0 + 4);
  const uint32_t w[4] = {xw.x, xw.y, xw.z, xw.w};
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
  if (SS > 0) {
    // the splits are added in split order
    float y[8] = {pa[0].x, pa[0].y, pa[0].z, pa[0].w, pb[0].x, pb[0].y, pb[0].z, pb[0].w};
#pragma unroll
    for (int s = 1; s < SS; ++s) {
      y[0] = y[0] + pa[s].x; y[1] = y[1] + pa[s].y; y[2] = y[2] + pa[s].z; y[3] = y[3] + pa[s].w;
      y[4] = y[4] + pb[s].x; y[5] = y[5] + pb[s].y; y[6] = y[6] + pb[s].z; y[7] = y[7] + pb[s].w;
    }
    uint32_t nb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t r = pack_bf16_rne(y[2 * e], y[2 * e + 1]);
      nb[e] = pack_bf16_rne(v[2 * e] + __uint_as_float(r << 16), v[2 * e + 1] + __uint_as_float(r & 0xffff0000u));
      v[2 * e] = __uint_as_float(nb[e] << 16);
      v[2 * e + 1] = __uint_as_float(nb[e] & 0xffff0000u);
    }
    *(uint4*)xr = uint4{nb[0], nb[1], nb[2], nb[3]};
    if (c.side) {
      const int col = c.side_col0 + j0;
      const size_t o = c.side_type == T_F32 ? (size_t)row * c.ld_side + col : fm_index(row, col, c.ld_side);
      store8_act(c.side, o, c.side_type, v, c.status);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
  ss = wave_sum_full(ss);
  __shared__ float part[16];
  const int nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  // fixed-order sum of the wave partials
  float tot = part[0];
  for (int i = 1; i < nw; ++i) tot = tot + part[i];
  const float r = 1.0f / sqrtf(tot / (float)c.h + c.eps);
  const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = v[e] * r * g[e];
  bool bad = false;
  *(uint4*)((uint16_t*)c.out + fm_index(row, j0, c.h)) = pack8_act<OT>(y, bad);
  if (OT == T_F16 && c.status) {
    const uint64_t b = __ballot(bad);
    if (b && (threadIdx.x & 63) == __builtin_ctzll(b)) atomicOr(c.status, STATUS_ACT_RANGE);
  }
}

template <int SS>
static void launch_norm_bf16(const NormCall& c, hipStream_t s) {
  const dim3 grid(c.rows), block(c.h / 8);
  if (c.otype == T_F16) hipLaunchKernelGGL((norm_bf16_kernel<SS, T_F16>), grid, block, 0, s, c);
  else hipLaunchKernelGGL((norm_bf16_kernel<SS, T_BF16>), grid, block, 0, s, c);
}

hipError_t launch_norm(const NormCall& c, hipStream_t s) {
  if (c.rows <= 0) return hipSuccess;
  if (c.h % 8 || c.h > 8 * 1024 || c.in.S > MAX_SPLITS) return hipErrorInvalidValue;
  const bool bf16_path = c.xtype == T_BF16 && c.tiled && (c.otype == T_F16 || c.otype == T_BF16) &&
                         c.h % 512 == 0 && (c.mode == NORM_ONLY || (c.mode == NORM_RESID && c.in.S >= 1));
  if (bf16_path) {
    switch (c.mode == NORM_ONLY ? 0 : c.in.S) {
      case 0: launch_norm_bf16<0>(c, s); break;
      case 1: launch_norm_bf16<1>(c, s); break;
      case 2: launch_norm_bf16<2>(c, s); break;
      case 3: launch_norm_bf16<3>(c, s); break;
      case 4: launch_norm_bf16<4>(c, s); break;
      case 5: launch_norm_bf16<5>(c, s); break;
      case 6: launch_norm_bf16<6>(c, s); break;
      case 7: launch_norm_bf16<7>(c, s); break;
      default: launch_norm_bf16<8>(c, s); break;
    }
    return hipGetLastError();
  }
  const int threads = ((c.h / 8 + 63) / 64) * 64;
  hipLaunchKernelGGL(norm_kernel, dim3(c.rows), dim3(threads), 0, s, c);
  return hipGetLastError();
}

// x[i] = E[token_i]; mask_mode: slot 0 takes tokens[0] (the anchor), the
// other slots the mask token (the drafter's noise block).
__global__ __launch_bounds__(256) void embed_kernel(const void* __restrict__ table, int ttype, int h, int vocab,
                                                    const int32_t* __restrict__ tokens, int mask_mode,
                                                    int mask_token, void* out, int ldo, int32_t* status,
                                                    int vec16) {
  const int row = blockIdx.x;
  int tok = (mask_mode && row > 0) ? mask_token : tokens[row];
  if (tok < 0 || tok >= vocab) {
    if (threadIdx.x == 0 && status) atomicOr(status, 2);
    tok = tok < 0 ? 0 : vocab - 1;
  }
  const size_t tb = (size_t)tok * h, ob = (size_t)row * ldo;
  if (ttype == T_F32) {
    for (int j = threadIdx.x; j < h; j += 256) ((float*)out)[ob + j] = ((const float*)table)[tb + j];
  } else if (vec16) {
    // 8 elements (16 bytes) a lane: the launcher checked h % 8, ldo % 8 and
    // the 16-byte alignment of both bases
    const uint4* src = (const uint4*)((const uint16_t*)table + tb);
    uint4* dst = (uint4*)((uint16_t*)out + ob);
    for (int j = threadIdx.x; j < (h >> 3); j += 256) dst[j] = src[j];
  } else {
    for (int j = threadIdx.x; j < h; j += 256) ((uint16_t*)out)[ob + j] = ((const uint16_t*)table)[tb + j];
  }
}

hipError_t launch_embed(const void* table, int ttype, int h, int vocab, const int32_t* tokens, int mask_mode,
                        int mask_token, int rows, void* out, int ldo, int32_t* status, hipStream_t s) {
  const int vec16 = ttype != T_F32 && h % 8 == 0 && ldo % 8 == 0 && (uintptr_t)table % 16 == 0 &&
                    (uintptr_t)out % 16 == 0;
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, s, table, ttype, h, vocab, tokens, mask_mode,
                     mask_token, out, ldo, status, vec16);
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
  if (clear) { scal[SC_STATUS] = 0; scal[SC_STATUS2] = 0; scal[SC_STEP] = 0; }
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

// ------------------------------------------------------------------ read floor
// The bytes of one weight-streaming launch, read by a kernel that does
// nothing else: each work-group reads a contiguous share with 16-byte
// non-temporal loads, eight in flight per lane.  It measures what a launch
// of that size and grid can reach at all on this part; the sink is written
// only if the data's XOR equals a value it never takes.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void read_floor_kernel(const u32x4_t* __restrict__ w, size_t n16,
                                                         uint32_t* sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b = blockIdx.x * per, e = min(n16, b + per);
  uint32_t acc = 0;
  for (size_t i = b + threadIdx.x; i < e; i += 256 * 8) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t j = i + 256 * u;
      v[u] = j < e ? __builtin_nontemporal_load(w + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u && threadIdx.x == 0) sink[blockIdx.x] = acc;
}

hipError_t launch_read_floor(const void* buf, size_t bytes, int nwg, uint32_t* sink, hipStream_t s) {
  if (nwg < 1 || bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(read_floor_kernel, dim3(nwg), dim3(256), 0, s, (const u32x4_t*)buf, bytes / 16, sink);
  return hipGetLastError();
}

// ------------------------------------------------------------------ bf16 rounding check
// Every fp32 bit pattern a, paired with b = a ^ 0x9e3779b9 so both halves of
// the packed conversion see every pattern: pack_bf16_rne (v_cvt_pk_bf16_f32)
// against the integer round-to-nearest-even f32_to_bf16_bits.  counts[0]
// gets the mismatches on non-NaN inputs, counts[1] those on NaN inputs.
__global__ __launch_bounds__(256) void bf16_round_check_kernel(unsigned long long* counts) {
  unsigned long long bad_num = 0, bad_nan = 0;
  const uint64_t nthreads = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < (1ull << 32); i += nthreads) {
    const uint32_t a = (uint32_t)i, b = a ^ 0x9e3779b9u;
    const uint32_t hw = pack_bf16_rne(__uint_as_float(a), __uint_as_float(b));
    const uint32_t sw = f32_to_bf16_bits(__uint_as_float(a)) | (f32_to_bf16_bits(__uint_as_float(b)) << 16);
    const bool nan_a = (a & 0x7fffffffu) > 0x7f800000u, nan_b = (b & 0x7fffffffu) > 0x7f800000u;
    if ((hw ^ sw) & 0xffffu) { if (nan_a) ++bad_nan; else ++bad_num; }
    if ((hw ^ sw) >> 16) { if (nan_b) ++bad_nan; else ++bad_num; }
  }
  if (bad_num) atomicAdd(&counts[0], bad_num);
  if (bad_nan) atomicAdd(&counts[1], bad_nan);
}

hipError_t launch_bf16_round_check(unsigned long long* counts, hipStream_t s) {
  hipLaunchKernelGGL(bf16_round_check_kernel, dim3(16384), dim3(256), 0, s, counts);
  return hipGetLastError();
}

}  // namespace dfl
