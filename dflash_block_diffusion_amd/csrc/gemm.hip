// Skinny dequant-GEMM for the draft+verify step: Y[m][n] = X[m][k] * W[n][k]^T
// with m <= 64 token rows (one block of B = 16/32 slots, or block + context rows
// for the drafter's QKV), weights streamed once from HBM.
//
// Formats (mirror-sd README, "The Story": int8 weights with per-channel fp16
// scales and 16-bit activations; "Results": a 4-bit target):
//   BF16  bf16 weights, bf16 activations, MFMA f32_16x16x32_bf16
//   W8    int8 codes + fp16 scale per output row; fp16 MFMA on the raw codes,
//         scale applied to the fp32 sum
//   W4    int4 codes + fp16 scale per (row, 64-wide K group); fp16 MFMA on the
//         raw codes, one fp32 partial per group, scaled and accumulated
// Integer codes are exact in fp16, so the MFMA products are the exact products
// of the dequantised weights (scale * code is applied in fp32 afterwards).
// X for the quantised formats is stored as the fp16 encoding of its bf16 value.
//
// Packed layout: per tile of 16 weight rows x KT columns (KT = 32/64/128 for
// BF16/W8/W4) one contiguous 1 KiB block; lane l of a wave loads bytes
// [16l, 16l+16), which hold row (l % 16) and, for each 32-wide MFMA sub-step
// ss of the tile, the 8 columns KT*t + 32*ss + 8*(l/16) + e, e = 0..7 --
// exactly the A-operand of v_mfma_f32_16x16x32 for that lane.  So every wave
// load is one fully coalesced 1 KiB read and needs no shuffling.
//
// Work split: a work-group (4 waves) owns R row-tiles (16R rows) and one of
// `splits` K ranges; its 4 waves split that range again.  The 4 wave partials
// are summed in LDS in a fixed order; with splits > 1 the last-arriving
// work-group of a row block sums the split partials in a fixed order (so the
// result is bit-reproducible) and runs the epilogue.
#include "common.h"

namespace dfl {

// ------------------------------------------------------------------ packing
__device__ __forceinline__ int canon_row(int rt, int lr, int n, int gate_up) {
  if (!gate_up) return rt * 16 + lr;
  return (rt & 1) * (n / 2) + (rt >> 1) * 16 + lr;   // tile pairs: (gate j, up j)
}

template <int FMT>
__global__ void pack_kernel(int n, int k, int gate_up, const void* __restrict__ src,
                            uint8_t* __restrict__ dst) {
  constexpr int KT = tile_k(FMT);
  const int ktiles = k / KT;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)(n / 16) * ktiles * 64;
  if (idx >= total) return;
  const int lane = idx & 63;
  const size_t tile = idx >> 6;
  const int t = (int)(tile % ktiles);
  const int rt = (int)(tile / ktiles);
  const int lr = lane & 15, g = lane >> 4;
  const size_t row = (size_t)canon_row(rt, lr, n, gate_up) * k;
  uint32_t out[4] = {0, 0, 0, 0};
  if (FMT == W_BF16) {
    const uint16_t* s = (const uint16_t*)src + row + (size_t)KT * t + 8 * g;
    for (int e = 0; e < 8; ++e) out[e >> 1] |= (uint32_t)s[e] << (16 * (e & 1));
  } else if (FMT == W_W8) {
    for (int ss = 0; ss < 2; ++ss) {
      const int8_t* s = (const int8_t*)src + row + (size_t)KT * t + 32 * ss + 8 * g;
      for (int e = 0; e < 8; ++e) {
        uint32_t u = (uint32_t)(s[e] + 128) & 0xffu;          // offset binary
        out[ss * 2 + (e >> 2)] |= u << (8 * (e & 3));
      }
    }
  } else {  // W4: dword ss; nibble slot j holds column e = 2j (j<4) or 2(j-4)+1
    for (int ss = 0; ss < 4; ++ss) {
      const int8_t* s = (const int8_t*)src + row + (size_t)KT * t + 32 * ss + 8 * g;
      uint32_t d = 0;
      for (int j = 0; j < 8; ++j) {
        const int e = j < 4 ? 2 * j : 2 * (j - 4) + 1;
        d |= ((uint32_t)(s[e] + 8) & 0xfu) << (4 * j);          // offset binary
      }
      out[ss] = d;
    }
  }
  uint4 v = {out[0], out[1], out[2], out[3]};
  *(uint4*)(dst + tile * 1024 + (size_t)lane * 16) = v;
}

// W4 scales: per (row tile, K tile) 32 halves; lane quarter q reads 8 halves
// [group 0: rows 4q..4q+3][group 1: rows 4q..4q+3] with one 16-byte load.
__global__ void pack_scales_w4(int n, int k, int gate_up, const uint16_t* __restrict__ src,
                               uint16_t* __restrict__ dst) {
  const int ktiles = k / 128;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)(n / 16) * ktiles * 32;
  if (idx >= total) return;
  const int v = idx & 3, gg = (idx >> 2) & 1, q = (idx >> 3) & 3;
  const size_t tile = idx >> 5;
  const int t = (int)(tile % ktiles), rt = (int)(tile / ktiles);
  const int row = canon_row(rt, 4 * q + v, n, gate_up);
  dst[idx] = src[(size_t)row * (k / 64) + 2 * t + gg];
}

__global__ void pack_scales_w8(int n, int gate_up, const uint16_t* __restrict__ src,
                               uint16_t* __restrict__ dst) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  dst[idx] = src[canon_row(idx / 16, idx % 16, n, gate_up)];
}

__global__ void copy_bytes(const uint8_t* __restrict__ s, uint8_t* __restrict__ d, size_t nb) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nb;
       i += (size_t)gridDim.x * blockDim.x)
    d[i] = s[i];
}

void packed_bytes(int fmt, int n, int k, size_t* wb, size_t* sb) {
  if (fmt == W_F32) { *wb = (size_t)n * k * 4; *sb = 0; return; }
  const int kt = tile_k(fmt);
  *wb = (size_t)(n / 16) * (k / kt) * 1024;
  *sb = fmt == W_W8 ? (size_t)n * 2 : fmt == W_W4 ? (size_t)n * (k / 64) * 2 : 0;
}

hipError_t launch_pack(int fmt, int n, int k, int gate_up, const void* src, const void* src_scales,
                       void* dst, void* dst_scales, hipStream_t s) {
  if (fmt == W_F32) {
    size_t nb = (size_t)n * k * 4;
    hipLaunchKernelGGL(copy_bytes, dim3(1024), dim3(256), 0, s, (const uint8_t*)src, (uint8_t*)dst, nb);
    return hipGetLastError();
  }
  const size_t lanes = (size_t)(n / 16) * (k / tile_k(fmt)) * 64;
  dim3 grid((unsigned)((lanes + 255) / 256));
  if (fmt == W_BF16)
    hipLaunchKernelGGL(pack_kernel<W_BF16>, grid, dim3(256), 0, s, n, k, gate_up, src, (uint8_t*)dst);
  else if (fmt == W_W8)
    hipLaunchKernelGGL(pack_kernel<W_W8>, grid, dim3(256), 0, s, n, k, gate_up, src, (uint8_t*)dst);
  else
    hipLaunchKernelGGL(pack_kernel<W_W4>, grid, dim3(256), 0, s, n, k, gate_up, src, (uint8_t*)dst);
  if (fmt == W_W8) {
    hipLaunchKernelGGL(pack_scales_w8, dim3((n + 255) / 256), dim3(256), 0, s, n, gate_up,
                       (const uint16_t*)src_scales, (uint16_t*)dst_scales);
  } else if (fmt == W_W4) {
    const size_t tot = (size_t)(n / 16) * (k / 128) * 32;
    hipLaunchKernelGGL(pack_scales_w4, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, s, n, k,
                       gate_up, (const uint16_t*)src_scales, (uint16_t*)dst_scales);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------- dequant
__device__ __forceinline__ half2v h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// 8 int4 codes (one dword, offset binary, nibble slots as packed) -> 8 halves
// 0x6400 | u is the fp16 value 1024 + u; (0x6400 | 16u) scaled by 1/16 is 64 + u.
__device__ __forceinline__ half8 deq_w4(uint32_t w) {
  const half2v c0 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2v s16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2v c1 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w2 = w >> 8;
  half2v a = h2((w & 0x000F000Fu) | 0x64006400u) + c0;
  half2v b = h2((w & 0x00F000F0u) | 0x64006400u) * s16 + c1;
  half2v c = h2((w2 & 0x000F000Fu) | 0x64006400u) + c0;
  half2v d = h2((w2 & 0x00F000F0u) | 0x64006400u) * s16 + c1;
  half8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// 8 int8 codes (two dwords, bytes in column order, offset binary) -> 8 halves
__device__ __forceinline__ half8 deq_w8(uint32_t lo, uint32_t hi) {
  const half2v c = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  half2v a = h2((lo & 0xFFu) | ((lo & 0xFF00u) << 8) | 0x64006400u) + c;
  half2v b = h2(((lo >> 16) & 0xFFu) | ((lo >> 8) & 0xFF0000u) | 0x64006400u) + c;
  half2v d = h2((hi & 0xFFu) | ((hi & 0xFF00u) << 8) | 0x64006400u) + c;
  half2v e = h2(((hi >> 16) & 0xFFu) | ((hi >> 8) & 0xFF0000u) | 0x64006400u) + c;
  half8 r = {a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
  return r;
}

__device__ __forceinline__ float half_at(const uint4& v, int i) {
  const uint32_t d = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
  const uint16_t h = (i & 1) ? (uint16_t)(d >> 16) : (uint16_t)(d & 0xffffu);
  return (float)__builtin_bit_cast(_Float16, h);
}

// ------------------------------------------------------------------ kernel
struct GemmArgs {
  const uint8_t* w; const uint16_t* s; const uint16_t* x; int ldx;
  int n, k, ktiles, ntile16, nrb, splits, m;
  int epi; void* out; int ldo; int otype;
  void* side; int ld_side; int side_type;
  float* logits; int ldl; int row0;
  float* am_val; int* am_idx;
  float* ws; int* ctr;
};

template <int FMT, int R, int MB>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(GemmArgs a) {
  constexpr int KT = tile_k(FMT);
  constexpr int SS = KT / 32;
  constexpr int ROWS = 16 * R;          // weight rows of this work-group
  constexpr int TOK = 16 * MB;          // token rows computed
  constexpr int TS = ROWS * TOK;        // tile floats
  __shared__ float red[3][R * MB * 4][64];
  __shared__ float tileT[TOK][ROWS + 1];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  const int rb = blockIdx.x / a.splits, sp = blockIdx.x % a.splits;
  const int rt0 = rb * R;
  const int nsl = a.splits * 4, q = sp * 4 + wave;
  const int t0 = (int)((long long)a.ktiles * q / nsl);
  const int t1 = (int)((long long)a.ktiles * (q + 1) / nsl);

  floatx4 acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    // rows past m are recomputed from row m-1 (never read past the caller's [m][k])
    const int row = min(mb * 16 + lr, a.m - 1);
    xrow[mb] = a.x + (size_t)row * a.ldx + 8 * g;
  }

  for (int t = t0; t < t1; ++t) {
    uint4 wr[R];
    uint4 sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int rt = rt0 + r;
      if (rt < a.ntile16) {
        wr[r] = *(const uint4*)(a.w + ((size_t)rt * a.ktiles + t) * 1024 + lane * 16);
        if (FMT == W_W4) sc[r] = *(const uint4*)(a.s + ((size_t)rt * a.ktiles + t) * 32 + g * 8);
      } else {
        wr[r] = uint4{0, 0, 0, 0};
        sc[r] = uint4{0, 0, 0, 0};
      }
    }
    uint4 xf[MB][SS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ss = 0; ss < SS; ++ss) xf[mb][ss] = *(const uint4*)(xrow[mb] + (size_t)t * KT + 32 * ss);

#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (FMT == W_BF16) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, wr[r]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              av, __builtin_bit_cast(bf16x8, xf[mb][0]), acc[r][mb], 0, 0, 0);
      } else if (FMT == W_W8) {
        const half8 a0 = deq_w8(wr[r].x, wr[r].y);
        const half8 a1 = deq_w8(wr[r].z, wr[r].w);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              a0, __builtin_bit_cast(half8, xf[mb][0]), acc[r][mb], 0, 0, 0);
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              a1, __builtin_bit_cast(half8, xf[mb][1]), acc[r][mb], 0, 0, 0);
        }
      } else {  // W4: two 64-wide groups per tile, sub-steps (0,1) and (2,3)
        const uint32_t wd[4] = {wr[r].x, wr[r].y, wr[r].z, wr[r].w};
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const half8 a0 = deq_w4(wd[2 * gg]);
          const half8 a1 = deq_w4(wd[2 * gg + 1]);
          float s4[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) s4[v] = half_at(sc[r], gg * 4 + v);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            floatx4 tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a0, __builtin_bit_cast(half8, xf[mb][2 * gg]), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a1, __builtin_bit_cast(half8, xf[mb][2 * gg + 1]), tmp, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[r][mb][v] += s4[v] * tmp[v];
          }
        }
      }
    }
  }

  // ---- fixed-order reduction of the 4 wave partials
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[wave - 1][(r * MB + mb) * 4 + v][lane] = acc[r][mb][v];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = (r * MB + mb) * 4 + v;
          float s = acc[r][mb][v] + red[0][j][lane];
          s = s + red[1][j][lane];
          s = s + red[2][j][lane];
          // D layout of 16x16 MFMA: lane holds column (token) lane%16, rows 4*(lane/16)+v
          tileT[mb * 16 + lr][r * 16 + 4 * g + v] = s;
        }
  }
  __syncthreads();

  // ---- split-K: the last work-group of this row block sums all partials
  if (a.splits > 1) {
    float* mine = a.ws + ((size_t)rb * a.splits + sp) * TS;
    for (int e = tid; e < TS; e += 256) mine[e] = tileT[e / ROWS][e % ROWS];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const int prev = atomicAdd(&a.ctr[rb], 1);
      s_last = (prev == a.splits - 1);
      if (s_last) a.ctr[rb] = 0;      // every split has arrived: reset for the next launch
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float* base = a.ws + (size_t)rb * a.splits * TS;
    for (int e = tid; e < TS; e += 256) {
      float v = 0.f;
      for (int s2 = 0; s2 < a.splits; ++s2)
        v += (s2 == sp) ? tileT[e / ROWS][e % ROWS] : __builtin_nontemporal_load(base + (size_t)s2 * TS + e);
      // written back after every thread has read its own elements (same e only)
      tileT[e / ROWS][e % ROWS] = v;
    }
    __syncthreads();
  }

  // ---- epilogues
  const int n0 = rt0 * 16;
  const uint16_t* sc8 = (FMT == W_W8) ? a.s : nullptr;
  auto scale_of = [&](int n) -> float {
    return FMT == W_W8 ? (float)__builtin_bit_cast(_Float16, sc8[n]) : 1.0f;
  };
  if (a.epi == EPI_STORE || a.epi == EPI_RESID) {
    for (int e = tid; e < TS; e += 256) {
      const int t = e / ROWS, nl = e % ROWS, n = n0 + nl;
      if (t >= a.m || n >= a.n) continue;
      const float y = tileT[t][nl] * scale_of(n);
      const size_t o = (size_t)t * a.ldo + n;
      if (a.epi == EPI_STORE) {
        store_act(a.out, o, a.otype, y);
      } else {
        const float xo = load_act(a.out, o, a.otype);
        const float nv = act_round(a.otype, xo + act_round(a.otype, y));
        store_act(a.out, o, a.otype, nv);
        if (a.side) store_act(a.side, (size_t)t * a.ld_side + n, a.side_type, nv);
      }
    }
  } else if (a.epi == EPI_SILU) {
    constexpr int HALF = ROWS / 2;
    for (int e = tid; e < TOK * HALF; e += 256) {
      const int t = e / HALF, j = e % HALF;
      const int pr = j / 16, w = j % 16;
      const int gl = (2 * pr) * 16 + w, ul = (2 * pr + 1) * 16 + w;
      const int n_out = (rt0 / 2 + pr) * 16 + w;
      if (t >= a.m || n_out >= a.n / 2) continue;
      const int rnd = a.otype == T_F32 ? T_F32 : T_BF16;
      const float gv = act_round(rnd, tileT[t][gl] * scale_of(n0 + gl));
      const float uv = act_round(rnd, tileT[t][ul] * scale_of(n0 + ul));
      const float sv = gv / (1.0f + expf(-gv));
      store_act(a.out, (size_t)t * a.ldo + n_out, a.otype, sv * uv);
    }
  } else {  // EPI_ARGMAX
    if (a.logits) {
      for (int e = tid; e < TS; e += 256) {
        const int t = e / ROWS, nl = e % ROWS, n = n0 + nl;
        if (t < a.row0 || t >= a.m || n >= a.n) continue;
        a.logits[(size_t)(t - a.row0) * a.ldl + n] = tileT[t][nl] * scale_of(n);
      }
    }
    if (tid < TOK) {
      const int t = tid;
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int nl = 0; nl < ROWS; ++nl) {
        const int n = n0 + nl;
        if (n >= a.n) break;
        const float y = tileT[t][nl] * scale_of(n);
        if (y > best) { best = y; bi = n; }   // ascending n: first (lowest) index kept on ties
      }
      a.am_val[(size_t)rb * 64 + t] = best;
      a.am_idx[(size_t)rb * 64 + t] = bi;
    }
  }
}

// ------------------------------------------------------------------ fp32 path
// Plain fp32 GEMM for fp32 models (the small sanity configuration): one
// thread per output column, all token rows; weights in canonical [N][K].
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ W, const float* __restrict__ X,
                                                       int ldx, int n, int k, int m, int epi, void* out,
                                                       int ldo, void* side, int ld_side, int side_type,
                                                       float* logits, int ldl) {
  const int col = blockIdx.x * blockDim.x + threadIdx.x;
  const int ncols = epi == EPI_SILU ? n / 2 : n;
  if (col >= ncols) return;
  float acc[MAX_ROWS], acc2[MAX_ROWS];
#pragma unroll
  for (int t = 0; t < MAX_ROWS; ++t) { acc[t] = 0.f; acc2[t] = 0.f; }
  const float* w = W + (size_t)col * k;
  const float* w2 = W + (size_t)(col + n / 2) * k;
  for (int kk = 0; kk < k; ++kk) {
    const float wv = w[kk];
    const float wv2 = epi == EPI_SILU ? w2[kk] : 0.f;
#pragma unroll
    for (int t = 0; t < MAX_ROWS; ++t) {
      if (t < m) {
        const float xv = X[(size_t)t * ldx + kk];
        acc[t] += xv * wv;
        acc2[t] += xv * wv2;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MAX_ROWS; ++t) {
    if (t >= m) continue;
    if (epi == EPI_STORE) {
      ((float*)out)[(size_t)t * ldo + col] = acc[t];
    } else if (epi == EPI_RESID) {
      float* o = (float*)out + (size_t)t * ldo + col;
      const float nv = *o + acc[t];
      *o = nv;
      if (side) store_act(side, (size_t)t * ld_side + col, side_type, nv);
    } else if (epi == EPI_SILU) {
      const float gv = acc[t];
      ((float*)out)[(size_t)t * ldo + col] = gv / (1.0f + expf(-gv)) * acc2[t];
    } else {
      logits[(size_t)t * ldl + col] = acc[t];
    }
  }
}

// ------------------------------------------------------------------ argmax
// (value, index) maximum with the lowest index among equal values.
__device__ __forceinline__ void am_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

__global__ __launch_bounds__(256) void argmax_final_kernel(const float* __restrict__ val,
                                                           const int* __restrict__ idx, int nblocks,
                                                           int row0, int32_t* out) {
  const int t = row0 + blockIdx.x;
  float v = -INFINITY;
  int i = 0x7fffffff;
  for (int b = threadIdx.x; b < nblocks; b += 256) am_merge(v, i, val[(size_t)b * 64 + t], idx[(size_t)b * 64 + t]);
  __shared__ float sv[256];
  __shared__ int si[256];
  sv[threadIdx.x] = v;
  si[threadIdx.x] = i;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      float a = sv[threadIdx.x];
      int ai = si[threadIdx.x];
      am_merge(a, ai, sv[threadIdx.x + o], si[threadIdx.x + o]);
      sv[threadIdx.x] = a;
      si[threadIdx.x] = ai;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = si[0] == 0x7fffffff ? 0 : si[0];
}

__global__ __launch_bounds__(256) void argmax_rows_kernel(const float* __restrict__ logits, int ld, int vocab,
                                                          int row0, int32_t* out, float* copy, int ldc) {
  const int t = row0 + blockIdx.x;
  const float* row = logits + (size_t)t * ld;
  float v = -INFINITY;
  int i = 0x7fffffff;
  for (int c = threadIdx.x; c < vocab; c += 256) {
    const float x = row[c];
    if (copy) copy[(size_t)blockIdx.x * ldc + c] = x;
    am_merge(v, i, x, c);
  }
  __shared__ float sv[256];
  __shared__ int si[256];
  sv[threadIdx.x] = v;
  si[threadIdx.x] = i;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      float a = sv[threadIdx.x];
      int ai = si[threadIdx.x];
      am_merge(a, ai, sv[threadIdx.x + o], si[threadIdx.x + o]);
      sv[threadIdx.x] = a;
      si[threadIdx.x] = ai;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[blockIdx.x] = si[0] == 0x7fffffff ? 0 : si[0];
}

hipError_t launch_argmax_final(const float* am_val, const int* am_idx, int nblocks, int row0, int rows,
                               int32_t* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_final_kernel, dim3(rows), dim3(256), 0, s, am_val, am_idx, nblocks, row0, out);
  return hipGetLastError();
}

hipError_t launch_argmax_rows(const float* logits, int ld, int vocab, int row0, int rows, int32_t* out,
                              float* copy, int ldc, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_rows_kernel, dim3(rows), dim3(256), 0, s, logits, ld, vocab, row0, out, copy, ldc);
  return hipGetLastError();
}

// ------------------------------------------------------------------ planning
struct Plan { int R, MB, nrb, splits, ktiles, ntile16; };

static Plan make_plan(int fmt, int n, int k, int m) {
  Plan p;
  p.MB = (m + 15) / 16;
  p.R = p.MB <= 2 ? 4 : 2;
  p.ntile16 = n / 16;
  p.nrb = (p.ntile16 + p.R - 1) / p.R;
  p.ktiles = k / tile_k(fmt);
  int sp = (512 + p.nrb - 1) / p.nrb;
  sp = sp < 1 ? 1 : sp > 8 ? 8 : sp;
  while (sp > 1 && p.ktiles < 4 * sp) --sp;
  p.splits = sp;
  return p;
}

size_t gemm_ws_floats(int fmt, int n, int k, int m) {
  if (fmt == W_F32) return 0;
  Plan p = make_plan(fmt, n, k, m);
  if (p.splits == 1) return 0;
  return (size_t)p.nrb * p.splits * (16 * p.R) * (16 * p.MB);
}

int gemm_am_blocks(int fmt, int n, int m) {
  if (fmt == W_F32) return 0;
  const int MB = (m + 15) / 16, R = MB <= 2 ? 4 : 2;
  return (n / 16 + R - 1) / R;     // same row blocking as make_plan
}

template <int FMT>
static hipError_t dispatch_mfma(const Plan& p, const GemmArgs& a, hipStream_t s) {
  dim3 grid(p.nrb * p.splits), block(256);
  if (p.R == 4 && p.MB == 1) hipLaunchKernelGGL((gemm_mfma_kernel<FMT, 4, 1>), grid, block, 0, s, a);
  else if (p.R == 4 && p.MB == 2) hipLaunchKernelGGL((gemm_mfma_kernel<FMT, 4, 2>), grid, block, 0, s, a);
  else if (p.R == 2 && p.MB == 3) hipLaunchKernelGGL((gemm_mfma_kernel<FMT, 2, 3>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((gemm_mfma_kernel<FMT, 2, 4>), grid, block, 0, s, a);
  return hipGetLastError();
}

static const char* variant_name(int fmt, const Plan& p) {
  static const char* names[4][4] = {
      {"gemm_f32", "gemm_f32", "gemm_f32", "gemm_f32"},
      {"gemm_bf16_r4m1", "gemm_bf16_r4m2", "gemm_bf16_r2m3", "gemm_bf16_r2m4"},
      {"gemm_w8_r4m1", "gemm_w8_r4m2", "gemm_w8_r2m3", "gemm_w8_r2m4"},
      {"gemm_w4_r4m1", "gemm_w4_r4m2", "gemm_w4_r2m3", "gemm_w4_r2m4"}};
  return names[fmt][p.MB - 1];
}

hipError_t launch_gemm(const GemmCall& c, const Workspace& w, hipStream_t s, const char** variant,
                       double* bytes) {
  const GemmW& W = *c.W;
  size_t wb, sb;
  packed_bytes(W.fmt, W.n, W.k, &wb, &sb);
  if (bytes) *bytes = (double)(wb + sb);
  if (W.fmt == W_F32) {
    if (variant) *variant = "gemm_f32";
    const int ncols = c.epi == EPI_SILU ? W.n / 2 : W.n;
    float* lg = c.epi == EPI_ARGMAX ? w.logits_tmp : nullptr;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((ncols + 255) / 256), dim3(256), 0, s, (const float*)W.w,
                       (const float*)c.x, c.ldx, W.n, W.k, c.m, c.epi, c.out, c.ldo, c.side, c.ld_side,
                       c.side_type, lg, W.n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || c.epi != EPI_ARGMAX) return e;
    return launch_argmax_rows(w.logits_tmp, W.n, W.n, c.row0, c.m - c.row0, c.am_out, c.logits, c.ldl, s);
  }
  Plan p = make_plan(W.fmt, W.n, W.k, c.m);
  if (variant) *variant = variant_name(W.fmt, p);
  GemmArgs a;
  a.w = (const uint8_t*)W.w; a.s = (const uint16_t*)W.s; a.x = (const uint16_t*)c.x; a.ldx = c.ldx;
  a.n = W.n; a.k = W.k; a.ktiles = p.ktiles; a.ntile16 = p.ntile16; a.nrb = p.nrb; a.splits = p.splits;
  a.m = c.m; a.epi = c.epi; a.out = c.out; a.ldo = c.ldo; a.otype = c.otype;
  a.side = c.side; a.ld_side = c.ld_side; a.side_type = c.side_type;
  a.logits = c.logits; a.ldl = c.ldl; a.row0 = c.row0;
  a.am_val = w.am_val; a.am_idx = w.am_idx; a.ws = w.ws; a.ctr = w.counters;
  hipError_t e;
  if (W.fmt == W_BF16) e = dispatch_mfma<W_BF16>(p, a, s);
  else if (W.fmt == W_W8) e = dispatch_mfma<W_W8>(p, a, s);
  else e = dispatch_mfma<W_W4>(p, a, s);
  if (e != hipSuccess || c.epi != EPI_ARGMAX) return e;
  return launch_argmax_final(w.am_val, w.am_idx, p.nrb, c.row0, c.m - c.row0, c.am_out, s);
}

}  // namespace dfl
