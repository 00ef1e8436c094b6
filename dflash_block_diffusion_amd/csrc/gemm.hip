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
// load is one fully coalesced 1 KiB read and needs no shuffling.  The
// activations come in the matching tiled layout (fm_index in common.h), so
// their operand fragments are contiguous 1 KiB reads as well: with row-major
// activations each fragment is a 16-row gather, and those gathers saturated
// the texture addresser long before HBM.
//
// Work split: a work-group (4 waves) owns R row tiles (16R rows) over the full
// K; wave w takes the w-th quarter of the K tiles and prefetches the next tile
// while it multiplies the current one.  The 4 wave partials are summed in LDS
// in a fixed order, so results are bit-reproducible.  R is chosen per shape
// so that even the narrow projections (N = 4096) launch one work-group per
// CU.  (No cross-work-group split-K: a release/acquire handoff between
// work-groups writes back the L2 and costs far more than it saves here.)
#include <cstdio>

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
// mlo = 0x000F000F, mhi = 0x00F000F0, magic = 0x64006400 (register operands).
__device__ __forceinline__ half8 deq_w4(uint32_t w, uint32_t mlo, uint32_t mhi, uint32_t magic) {
  const half2v c0 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2v s16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2v c1 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w2 = w >> 8;
  half2v a = h2((w & mlo) | magic) + c0;
  half2v b = h2((w & mhi) | magic) * s16 + c1;
  half2v c = h2((w2 & mlo) | magic) + c0;
  half2v d = h2((w2 & mhi) | magic) * s16 + c1;
  half8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// 8 int8 codes (two dwords, bytes in column order, offset binary) -> 8 halves:
// byte pairs are spread to the low bytes of two fp16 lanes over the magic 0x64.
__device__ __forceinline__ half8 deq_w8(uint32_t lo, uint32_t hi, uint32_t magic) {
  const half2v c = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  half2v a = h2(__builtin_amdgcn_perm(magic, lo, 0x05010500u)) + c;
  half2v b = h2(__builtin_amdgcn_perm(magic, lo, 0x05030502u)) + c;
  half2v d = h2(__builtin_amdgcn_perm(magic, hi, 0x05010500u)) + c;
  half2v e = h2(__builtin_amdgcn_perm(magic, hi, 0x05030502u)) + c;
  half8 r = {a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
  return r;
}

// ------------------------------------------------------------------ kernel
struct GemmArgs {
  const uint8_t* w; const uint16_t* s; const uint16_t* x; int ldx;
  int n, k, ktiles, ntile16, m;
  int epi; void* out; int ldo; int otype;
  void* side; int ld_side; int side_type; int side_col0;
  float* logits; int ldl; int row0;
  float* am_val; int* am_idx;
  // dequant bit masks, passed as arguments so that they live in registers
  // (gfx9 VOP3 encodings take no literal constants)
  uint32_t mlo, mhi, magic;
};

template <int FMT, int R, int MB>
struct Frag {          // one K tile's operands for one wave
  uint4 w[R];
  uint4 s[R];
  uint4 x[MB][tile_k(FMT) / 32];
};

// Work-group = 4 waves on R row tiles (16R weight rows) over the full K; wave
// w takes the w-th quarter of the K tiles; the quarters are summed in LDS in a
// fixed order (bit-reproducible).  Loads of the next K tile are issued before
// the current one is consumed (register double buffering).
template <int FMT, int R, int MB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_mfma_kernel(GemmArgs a) {
  constexpr int KT = tile_k(FMT);
  constexpr int SS = KT / 32;
  // ring depth (K tiles in flight per wave): as many stages as fit ~128 VGPRs
  constexpr int STAGE = 4 * R * (FMT == W_W4 ? 2 : 1) + 4 * MB * SS;
  constexpr int U = 4 * STAGE <= 128 ? 4 : (3 * STAGE <= 128 ? 3 : 2);
  constexpr int ROWS = 16 * R;          // weight rows of this work-group
  constexpr int TOK = 16 * MB;          // token rows computed
  constexpr int TS = ROWS * TOK;        // tile floats
  __shared__ float red[3][R * MB * 4][64];
  __shared__ float tileT[TOK][ROWS + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  const int rt0 = blockIdx.x * R;
  const int t0 = (int)((long long)a.ktiles * wave / 4);
  const int t1 = (int)((long long)a.ktiles * (wave + 1) / 4);
  const uint32_t mlo = a.mlo, mhi = a.mhi, magic = a.magic;

  floatx4 acc[R][MB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // activations are tiled (fm_index): the fragment of token block mb and
  // 32-column step kb is the contiguous 1 KiB at ((mb * K/32) + kb) * 512
  const uint16_t* xrow[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) xrow[mb] = a.x + (size_t)mb * (a.k >> 5) * 512 + lane * 8;
  const uint8_t* wbase[R];
  const uint16_t* sbase[R];
  bool live[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int rt = rt0 + r;
    live[r] = rt < a.ntile16;
    const int rtc = live[r] ? rt : a.ntile16 - 1;     // clamped: dead tiles re-read a valid one
    wbase[r] = a.w + (size_t)rtc * a.ktiles * 1024 + lane * 16;
    sbase[r] = (FMT == W_W4) ? a.s + (size_t)rtc * a.ktiles * 32 + g * 8 : nullptr;
  }

  auto load = [&](int t, Frag<FMT, R, MB>& f) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      f.w[r] = *(const uint4*)(wbase[r] + (size_t)t * 1024);
      if (FMT == W_W4) f.s[r] = *(const uint4*)(sbase[r] + (size_t)t * 32);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ss = 0; ss < SS; ++ss) f.x[mb][ss] = *(const uint4*)(xrow[mb] + ((size_t)t * SS + ss) * 512);
  };

  auto compute = [&](const Frag<FMT, R, MB>& f) {
    const uint4 (&xf)[MB][SS] = f.x;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (FMT == W_BF16) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, f.w[r]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              av, __builtin_bit_cast(bf16x8, xf[mb][0]), acc[r][mb], 0, 0, 0);
      } else if (FMT == W_W8) {
        const half8 a0 = deq_w8(f.w[r].x, f.w[r].y, magic);
        const half8 a1 = deq_w8(f.w[r].z, f.w[r].w, magic);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              a0, __builtin_bit_cast(half8, xf[mb][0]), acc[r][mb], 0, 0, 0);
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              a1, __builtin_bit_cast(half8, xf[mb][1]), acc[r][mb], 0, 0, 0);
        }
      } else {  // W4: two 64-wide groups per tile, sub-steps (0,1) and (2,3)
        const uint32_t wd[4] = {f.w[r].x, f.w[r].y, f.w[r].z, f.w[r].w};
        const uint32_t sd[4] = {f.s[r].x, f.s[r].y, f.s[r].z, f.s[r].w};
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
          const half8 a0 = deq_w4(wd[2 * gg], mlo, mhi, magic);
          const half8 a1 = deq_w4(wd[2 * gg + 1], mlo, mhi, magic);
          const half2v s01 = __builtin_bit_cast(half2v, sd[2 * gg]);
          const half2v s23 = __builtin_bit_cast(half2v, sd[2 * gg + 1]);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            floatx4 tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a0, __builtin_bit_cast(half8, xf[mb][2 * gg]), floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                a1, __builtin_bit_cast(half8, xf[mb][2 * gg + 1]), tmp, 0, 0, 0);
            acc[r][mb][0] += (float)s01[0] * tmp[0];
            acc[r][mb][1] += (float)s01[1] * tmp[1];
            acc[r][mb][2] += (float)s23[0] * tmp[2];
            acc[r][mb][3] += (float)s23[1] * tmp[3];
          }
        }
      }
    }
  };

  // Operands stream through a ring of U register stages: each stage holds one
  // K tile's weights (HBM), scales and activations (L2), so U tiles of loads
  // are in flight per wave while the oldest is multiplied.  The main loop is
  // branch-free (every load unconditional, the last round re-reads a clamped
  // valid tile) so the compiler can wait for one stage at a time instead of
  // draining all outstanding loads; leftover tiles run in a short tail loop.
  const int full = (t1 - t0) / U;
  if (full > 0) {
    Frag<FMT, R, MB> ring[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load(t0 + u, ring[u]);
    // keep the scheduler from sinking loads next to their uses (it would
    // trade the in-flight depth for registers)
    __builtin_amdgcn_sched_barrier(0);
    for (int rd = 0; rd < full; ++rd) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        compute(ring[u]);
        load(min(t0 + (rd + 1) * U + u, t1 - 1), ring[u]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  for (int t = t0 + full * U; t < t1; ++t) {
    Frag<FMT, R, MB> f;
    load(t, f);
    compute(f);
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
          float sum = acc[r][mb][v] + red[0][j][lane];
          sum = sum + red[1][j][lane];
          sum = sum + red[2][j][lane];
          // D layout of 16x16 MFMA: lane holds column (token) lane%16, rows 4*(lane/16)+v
          tileT[mb * 16 + lr][r * 16 + 4 * g + v] = sum;
        }
  }
  __syncthreads();
  (void)live;

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
        if (a.side)
          store_act(a.side, act_index(t, a.side_col0 + n, a.ld_side, a.side_type == T_F32 ? 0 : a.ld_side),
                    a.side_type, nv);
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
      store_act(a.out, act_index(t, n_out, a.ldo, a.otype == T_F32 ? 0 : a.n / 2), a.otype, sv * uv);
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
      a.am_val[(size_t)blockIdx.x * 64 + t] = best;
      a.am_idx[(size_t)blockIdx.x * 64 + t] = bi;
    }
  }
}

// ------------------------------------------------------------------ fp32 path
// Plain fp32 GEMM for fp32 models (the small sanity configuration): one
// thread per output column, all token rows; weights in canonical [N][K].
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ W, const float* __restrict__ X,
                                                       int ldx, int n, int k, int m, int epi, void* out,
                                                       int ldo, void* side, int ld_side, int side_type,
                                                       int side_col0, float* logits, int ldl) {
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
      if (side)
        store_act(side, act_index(t, side_col0 + col, ld_side, side_type == T_F32 ? 0 : ld_side), side_type, nv);
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
  // candidates loaded 8 at a time before merging (independent loads)
  for (int b0 = threadIdx.x; b0 < nblocks; b0 += 256 * 8) {
    float cv[8];
    int ci[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int b = b0 + 256 * u;
      cv[u] = b < nblocks ? val[(size_t)b * 64 + t] : -INFINITY;
      ci[u] = b < nblocks ? idx[(size_t)b * 64 + t] : 0x7fffffff;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) am_merge(v, i, cv[u], ci[u]);
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
// R (row tiles per work-group) is the largest that still gives every CU at
// least one work-group, bounded by the register budget R * MB <= 8 (4 for
// int4, whose dequantisation needs the most registers);
// gate/up launches need R even (tile pairs).
struct Plan { int R, MB, nwg, ktiles, ntile16; };

#ifndef DFL_GEMM_MIN_WGS
#define DFL_GEMM_MIN_WGS 256
#endif

static Plan make_plan(int fmt, int n, int k, int m, int gate_up) {
  Plan p;
  p.MB = (m + 15) / 16;
  p.ntile16 = n / 16;
  p.ktiles = k / tile_k(fmt);
  const int budget = fmt == W_W4 ? 4 : 8;      // int4 dequant needs the most registers
  int R = 8;
  while (R > 1 && (R * p.MB > budget || (p.ntile16 + R - 1) / R < DFL_GEMM_MIN_WGS)) R /= 2;
  if (gate_up && R < 2) R = 2;
  p.R = R;
  p.nwg = (p.ntile16 + R - 1) / R;
  return p;
}

size_t gemm_ws_floats(int, int, int, int) { return 0; }

int gemm_am_blocks(int fmt, int n, int m) {
  if (fmt == W_F32) return 0;
  return make_plan(fmt, n, tile_k(fmt), m, 0).nwg;
}

template <int FMT, int R>
static hipError_t dispatch_mb(int MB, dim3 grid, const GemmArgs& a, hipStream_t s) {
  if (R * MB > (FMT == W_W4 ? 4 : 8)) return hipErrorInvalidValue;
  if (FMT == W_W4 && R == 8) return hipErrorInvalidValue;
  switch (MB) {
    case 1: hipLaunchKernelGGL((gemm_mfma_kernel<FMT, R, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((gemm_mfma_kernel<FMT, R, (R <= 4 ? 2 : 1)>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((gemm_mfma_kernel<FMT, R, (R <= 2 ? 3 : 1)>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_mfma_kernel<FMT, R, (R <= 2 ? 4 : 1)>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t dispatch_mfma(const Plan& p, const GemmArgs& a, hipStream_t s) {
  dim3 grid(p.nwg);
  switch (p.R) {
    case 8: return dispatch_mb<FMT, (FMT == W_W4 ? 4 : 8)>(p.MB, grid, a, s);
    case 4: return dispatch_mb<FMT, 4>(p.MB, grid, a, s);
    case 2: return dispatch_mb<FMT, 2>(p.MB, grid, a, s);
    default: return dispatch_mb<FMT, 1>(p.MB, grid, a, s);
  }
}

static const char* variant_name(int fmt, const Plan& p) {
  static char names[4][4][9][24];
  static bool init = false;
  if (!init) {
    const char* f[4] = {"f32", "bf16", "w8", "w4"};
    for (int i = 0; i < 4; ++i)
      for (int mb = 1; mb <= 4; ++mb)
        for (int r = 1; r <= 8; ++r) snprintf(names[i][mb - 1][r], 24, "gemm_%s_r%dm%d", f[i], r, mb);
    init = true;
  }
  return names[fmt][p.MB - 1][p.R];
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
                       c.side_type, c.side_col0, lg, W.n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || c.epi != EPI_ARGMAX) return e;
    return launch_argmax_rows(w.logits_tmp, W.n, W.n, c.row0, c.m - c.row0, c.am_out, c.logits, c.ldl, s);
  }
  Plan p = make_plan(W.fmt, W.n, W.k, c.m, W.gate_up);
  if (variant) *variant = variant_name(W.fmt, p);
  GemmArgs a;
  a.w = (const uint8_t*)W.w; a.s = (const uint16_t*)W.s; a.x = (const uint16_t*)c.x; a.ldx = c.ldx;
  a.n = W.n; a.k = W.k; a.ktiles = p.ktiles; a.ntile16 = p.ntile16;
  a.m = c.m; a.epi = c.epi; a.out = c.out; a.ldo = c.ldo; a.otype = c.otype;
  a.side = c.side; a.ld_side = c.ld_side; a.side_type = c.side_type; a.side_col0 = c.side_col0;
  a.logits = c.logits; a.ldl = c.ldl; a.row0 = c.row0;
  a.am_val = w.am_val; a.am_idx = w.am_idx;
  a.mlo = 0x000F000Fu; a.mhi = 0x00F000F0u; a.magic = 0x64006400u;
  hipError_t e;
  if (W.fmt == W_BF16) e = dispatch_mfma<W_BF16>(p, a, s);
  else if (W.fmt == W_W8) e = dispatch_mfma<W_W8>(p, a, s);
  else e = dispatch_mfma<W_W4>(p, a, s);
  if (e != hipSuccess || c.epi != EPI_ARGMAX) return e;
  return launch_argmax_final(w.am_val, w.am_idx, p.nwg, c.row0, c.m - c.row0, c.am_out, s);
}

}  // namespace dfl
