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
// The W4 codes enter the MFMA in offset binary c = q + 8 as the fp16 subnormals
// c * 2^-24 (a shift and an AND per pair of codes; the MFMA multiplies fp16
// subnormal operands exactly); each group's accumulator starts at
// -8 * 2^-24 * (sum of the group's activations), itself an MFMA of the
// activation fragments against the constant operand -8 * 2^-24, so the group
// sum is 2^-24 * sum (c - 8) * x, and the factor 2^24 is applied with the
// per-row scale of the epilogue (a power of two: exact).
// X for the quantised formats is stored as the fp16 encoding of its bf16 value.
//
// Packed layout: per tile of 16 weight rows x KT columns (KT = 32/64/128 for
// BF16/W8/W4) one contiguous 1 KiB block; lane l of a wave loads bytes
// [16l, 16l+16), which hold row (l % 16) and, for each 32-wide MFMA sub-step
// ss of the tile, the 8 columns KT*t + 32*ss + 8*(l/16) + e, e = 0..7 -- one
// lane's share of a 16x32 MFMA operand.  So every wave load is one fully
// coalesced 1 KiB read and needs no shuffling.  W4 scales are packed per
// (row tile, K tile) as 16 dwords, dword r = the two group scales of row r; one
// 4-byte load per four row tiles fetches them (lane l: dword l % 16 of row tile
// l / 16 of the four), and two lane-swap steps give every lane its row's pair
// of all four.  The activations come
// in the matching tiled layout (fm_index in common.h): every operand fragment
// is a contiguous 1 KiB read as well.
//
// MFMA orientation: A = activation fragment (16 tokens x 32 K), B = weight
// fragment (32 K x 16 weight rows), so lane l accumulates weight row l % 16
// for tokens 4*(l/16)..+3 and the per-row W4 scale is one value per lane.
//
// Work split (memory-level parallelism first):
//   * a work-group (4 waves) owns RT row tiles (16*RT weight rows) and one of
//     S contiguous K ranges; wave w takes the w-th quarter of that range;
//   * each wave streams its K tiles through a ring of U register stages (U K
//     tiles of all RT row tiles in flight); every activation fragment loaded
//     feeds RT MFMAs, so activation reads are 2x (int4), 1x (int8) or 1/4x
//     (bf16) the weight bytes rather than 8x with one row tile per wave;
//   * the 4 wave partials are summed in LDS in a fixed order; with S > 1 the
//     work-group writes an fp32 partial [m][n] of its K range and the consumer
//     kernel (residual + RMSNorm, QK-norm + RoPE, GatedDeltaNet) adds the S
//     partials in a fixed order.  All sums are bit-reproducible.
//   Non-linear epilogues (fused gate/up SiLU*mul, lm-head argmax) use S = 1.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "common.h"
#include "gemm_dev.h"

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

// W4 scales: per (row tile, K tile) 16 dwords; dword r holds the scales of
// groups 2t (low half) and 2t+1 (high half) of packed row 16*rt + r.
__global__ void pack_scales_w4(int n, int k, int gate_up, const uint16_t* __restrict__ src,
                               uint16_t* __restrict__ dst) {
  const int ktiles = k / 128;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)(n / 16) * ktiles * 32;
  if (idx >= total) return;
  const int gg = idx & 1, r = (idx >> 1) & 15;
  const size_t tile = idx >> 5;
  const int t = (int)(tile % ktiles), rt = (int)(tile / ktiles);
  const int row = canon_row(rt, r, n, gate_up);
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

// ------------------------------------------------------------------ kernel

// registers of one ring stage (one K tile of all RT row tiles + its
// activation fragments) and the ring depth that fits ~140 VGPRs
__host__ __device__ constexpr int stage_regs(int fmt, int rt, int mb) {
  return 4 * rt + (fmt == W_W4 ? rt : 0) + 4 * mb * (tile_k(fmt) / 32);
}
__host__ __device__ constexpr int ring_depth(int fmt, int rt, int mb) {
  return 140 / stage_regs(fmt, rt, mb) < 2 ? 2 : (140 / stage_regs(fmt, rt, mb) > 8 ? 8 : 140 / stage_regs(fmt, rt, mb));
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// Operands are read through buffer descriptors: the base lives in SGPRs, each
// lane adds a fixed byte offset and the per-tile offset is a scalar, so no
// per-load address arithmetic runs on the vector unit.  Reads past
// num_records return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
// streamed weights are read once: non-temporal, so they do not evict the
// activations every work-group re-reads from L2
constexpr int CPOL_NT = 2;
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, bool nt) {
  const u32x4 v = __builtin_bit_cast(u32x4, nt ? __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CPOL_NT)
                                                 : __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  return uint4{v.x, v.y, v.z, v.w};
}

template <int FMT, int RT, int MB>
struct Stage {
  uint4 w[RT];
  uint32_t s[(RT + 3) / 4];       // W4: scale pairs of four row tiles, one per 16 lanes
  uint4 x[MB][tile_k(FMT) / 32];
};

// Persistent streaming GEMM.  Work-group w serves K split s = w % S and a
// contiguous, balanced range of row tiles (in units of `align` tiles, 2 for
// fused gate/up); it walks that range in chunks of RT row tiles.  Each of
// its NW waves takes 1/NW of the split's K tiles and streams the flattened
// sequence (chunk, K tile) through a ring of U register stages: loads of the
// next chunk are in flight while the previous chunk's NW wave partials are
// added in LDS (fixed order) and written out.  With NW = 8 (two waves per
// SIMD) one wave's dequantisation overlaps the other's loads.
template <int FMT, int RT, int MB, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_stream_kernel(GemmArgs a) {
  constexpr int KT = tile_k(FMT);
  constexpr int SS = KT / 32;
  constexpr int U = ring_depth(FMT, RT, MB);
  constexpr int NE = RT * MB * 4;            // accumulator floats per lane
  static_assert(NW == 4 || (NW == 8 && MB == 2), "8 waves need two token blocks");
  __shared__ float red[NW][NE][64];

  const int tid = threadIdx.x;
  // wave index as a scalar: every per-wave index and stage address below is
  // then computed on the scalar unit, and loads take an SGPR base plus the
  // lane's offset
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, g = lane >> 4;
  const int S = a.splits;
  const int sidx = blockIdx.x % S, wr = blockIdx.x / S, PR = gridDim.x / S;
  // row tiles [rtb, rte) of this work-group
  // 32-bit products: the launcher keeps units * PR and ktiles * S below 2^32
  const uint32_t units = (uint32_t)(a.ntile16 / a.align);
  const int rtb = (int)(units * (uint32_t)wr / (uint32_t)PR) * a.align;
  const int rte = (int)(units * (uint32_t)(wr + 1) / (uint32_t)PR) * a.align;
  const int nch = (rte - rtb + RT - 1) / RT;
  // K tiles [t0, t1) of this wave
  const int kt0 = (int)((uint32_t)a.ktiles * (uint32_t)sidx / (uint32_t)S);
  const int kt1 = (int)((uint32_t)a.ktiles * (uint32_t)(sidx + 1) / (uint32_t)S);
  const int nk = kt1 - kt0;
  const int t0 = kt0 + nk * wave / NW, t1 = kt0 + nk * (wave + 1) / NW;
  const int nt = t1 - t0;
  const uint32_t mlo = a.mlo, magic = a.magic;

  floatx4 acc[RT][MB];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[r][mb] = floatx4{0.f, 0.f, 0.f, 0.f};

  // activations are tiled (fm_index): the fragment of token block mb and
  // 32-column step kb is the contiguous 1 KiB at ((mb * K/32) + kb) * 1024 B;
  // weight tile (rt, t) is the 1 KiB at (rt * ktiles + t) * 1024 B and its
  // W4 scales the 64 B at (rt * ktiles + t) * 64 B
  const uint32_t xfrag = (uint32_t)(a.k >> 5);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.w, (uint32_t)a.ntile16 * a.ktiles * 1024u);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.s, FMT == W_W4 ? (uint32_t)a.ntile16 * a.ktiles * 64u : 0u);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)MB * xfrag * 1024u);
  const uint32_t vlane = lane * 16, vrow = lr * 4;

  // stage (chunk c, K tile t); row tiles past the range re-read the last one
  auto load = [&](int c, int t, Stage<FMT, RT, MB>& f) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const uint32_t tile = (uint32_t)min(rtb + c * RT + r, rte - 1) * a.ktiles + t;
      f.w[r] = buf_load16(rw, vlane, tile * 1024u, true);
      // lane (lr, g) fetches row lr's scale pair of row tile r + g
      if (FMT == W_W4 && r % 4 == 0) {
        const uint32_t rti = (uint32_t)min(rtb + c * RT + r + g, rte - 1);
        f.s[r / 4] = __builtin_amdgcn_raw_buffer_load_b32(rs, rti * a.ktiles * 64u + vrow, (uint32_t)t * 64u, 0);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int ss = 0; ss < SS; ++ss)
        f.x[mb][ss] = buf_load16(rx, vlane, ((uint32_t)mb * xfrag + (uint32_t)t * SS + ss) * 1024u, false);
  };

  auto compute = [&](const Stage<FMT, RT, MB>& f) {
    // W4: the scale pair of row tile 4q + j sits in lane lr + 16 j of f.s[q];
    // the 16-lane row swap and the 32-lane half swap put all four in every lane
    uint32_t sq[RT];
    // and the code offset of each group: -8 * 2^-24 * sum of its 64 activation columns
    // (with three or four token blocks one group at a time, below)
    constexpr int CG = MB <= 2 ? 2 : 1;
    floatx4 corr[MB][CG];
    const half8 neg8 = __builtin_bit_cast(half8, uint4{0x80088008u, 0x80088008u, 0x80088008u, 0x80088008u});
    auto offset_sum = [&](int mb, int gg, int slot) {
      const floatx4 c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f.x[mb][2 * gg]), neg8,
                                                                floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      corr[mb][slot] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f.x[mb][2 * gg + 1]),
                                                              neg8, c0, 0, 0, 0);
    };
    // group gg of row tile r: the two MFMAs over its 64 columns, then the scale
    auto w4_group = [&](int r, int gg, int slot) {
      const half8 b0 = deq_w4_sub(gg == 0 ? f.w[r].x : f.w[r].z, mlo);
      const half8 b1 = deq_w4_sub(gg == 0 ? f.w[r].y : f.w[r].w, mlo);
      const float sg = (float)h2(sq[r])[gg];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        floatx4 tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f.x[mb][2 * gg]), b0,
                                                             corr[mb][slot], 0, 0, 0);
        tmp = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f.x[mb][2 * gg + 1]), b1, tmp,
                                                     0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[r][mb][v] += sg * tmp[v];
      }
    };
    if (FMT == W_W4) {
#pragma unroll
      for (int q = 0; q < (RT + 3) / 4; ++q) {
        const auto p16 = __builtin_amdgcn_permlane16_swap(f.s[q], f.s[q], false, false);
        const auto p0 = __builtin_amdgcn_permlane32_swap(p16[0], p16[0], false, false);
        const auto p1 = __builtin_amdgcn_permlane32_swap(p16[1], p16[1], false, false);
        if (4 * q + 0 < RT) sq[4 * q + 0] = p0[0];
        if (4 * q + 1 < RT) sq[4 * q + 1] = p1[0];
        if (4 * q + 2 < RT) sq[4 * q + 2] = p0[1];
        if (4 * q + 3 < RT) sq[4 * q + 3] = p1[1];
      }
      if constexpr (MB <= 2) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          offset_sum(mb, 0, 0);
          offset_sum(mb, 1, 1);
        }
      } else {
        // group-major: each accumulator still takes group 0 before group 1
#pragma unroll
        for (int gg = 0; gg < 2; ++gg) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) offset_sum(mb, gg, 0);
#pragma unroll
          for (int r = 0; r < RT; ++r) w4_group(r, gg, 0);
        }
        return;
      }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if (FMT == W_BF16) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, f.w[r]);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.x[mb][0]), bv,
                                                               acc[r][mb], 0, 0, 0);
      } else if (FMT == W_W8) {
        const half8 b0 = deq_w8(f.w[r].x, f.w[r].y, magic);
        const half8 b1 = deq_w8(f.w[r].z, f.w[r].w, magic);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f.x[mb][0]), b0,
                                                              acc[r][mb], 0, 0, 0);
          acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, f.x[mb][1]), b1,
                                                              acc[r][mb], 0, 0, 0);
        }
      } else {  // W4: two 64-wide groups per tile, sub-steps (0,1) and (2,3)
        w4_group(r, 0, 0);
        w4_group(r, 1, CG - 1);
      }
    }
  };

  // running argmax of this thread's tokens over every chunk
  float best[MB];
  int bidx[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) { best[mb] = -INFINITY; bidx[mb] = 0x7fffffff; }
  const uint16_t* sc8 = (FMT == W_W8) ? a.s : nullptr;
  auto scale_of = [&](int n) -> float {
    // W4: the group sums carry the 2^-24 of the subnormal codes
    return FMT == W_W8 ? (float)__builtin_bit_cast(_Float16, sc8[n]) : (FMT == W_W4 ? 16777216.0f : 1.0f);
  };

  // Chunk epilogue: fixed-order reduction of the NW wave partials,
  // ((w0 + w1) + w2) + ...; thread (wave w, lane) finishes accumulator slot
  // v = w % 4 of every (r, mb) it owns (all mb with 4 waves, mb = w / 4 with
  // 8): token mb*16 + 4g + v, weight row (rt0 + r)*16 + lr.
  const int vslot = wave & 3;
  auto own = [&](int mb) { return NW == 4 || mb == (wave >> 2); };
  auto epilogue = [&](int c) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          red[wave][(r * MB + mb) * 4 + v][lane] = acc[r][mb][v];
          acc[r][mb][v] = 0.f;
        }
    __syncthreads();
    const int rt0 = rtb + c * RT;
    float val[RT][MB];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int j = (r * MB + mb) * 4 + vslot;
        float v = red[0][j][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) v = v + red[w][j][lane];
        val[r][mb] = v;
      }
    if (c + 1 < nch) __syncthreads();      // red is rewritten by the next chunk
    if (a.epi == EPI_PARTIAL) {
      float* part = a.part + (size_t)sidx * a.m * a.n;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        if (rt0 + r >= rte) continue;
        const int n = (rt0 + r) * 16 + lr;
        const float sc = scale_of(n);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int t = mb * 16 + 4 * g + vslot;
          if (own(mb) && t < a.m) part[(size_t)t * a.n + n] = val[r][mb] * sc;
        }
      }
    } else if (a.epi == EPI_SILU) {
      const int rnd = a.otype == T_F32 ? T_F32 : T_BF16;
      const int half_n = a.n >> 1;
#pragma unroll
      for (int p = 0; p < RT / 2; ++p) {
        if (rt0 + 2 * p + 1 >= rte) continue;
        const int ng = (rt0 + 2 * p) * 16 + lr, nu = ng + 16;
        const int n_out = ((rt0 >> 1) + p) * 16 + lr;
        const float sg = scale_of(ng), su = scale_of(nu);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int t = mb * 16 + 4 * g + vslot;
          if (!own(mb) || t >= a.m) continue;
          const float gv = act_round(rnd, val[2 * p][mb] * sg);
          const float uv = act_round(rnd, val[2 * p + 1][mb] * su);
          // silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal
          // (about 1 ulp each in fp32, before the bf16 rounding below);
          // e^-g = +inf for g << 0 gives g * 0 = -0
          const float sv = gv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv * 1.4426950408889634f));
          store_act(a.out, act_index(t, n_out, 0, half_n), a.otype, sv * uv, a.status);
        }
      }
    } else {  // EPI_ARGMAX: ascending n within the lane keeps the lowest index on ties
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int t = mb * 16 + 4 * g + vslot;
        if (!own(mb)) continue;
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          if (rt0 + r >= rte) continue;
          const int n = (rt0 + r) * 16 + lr;
          const float y = val[r][mb] * scale_of(n);
          if (a.logits && t >= a.row0 && t < a.m) a.logits[(size_t)(t - a.row0) * a.ldl + n] = y;
          if (y > best[mb]) { best[mb] = y; bidx[mb] = n; }
        }
      }
    }
  };

  if (nt == 0) {
    // fewer K tiles than waves: this wave only joins the reductions
    for (int c = 0; c < nch; ++c) epilogue(c);
  } else {
    // Operands stream through a ring of U register stages: U stages of loads
    // are in flight per wave while the oldest is multiplied.  Loads are
    // unconditional (past the end they re-read the last stage) so the
    // compiler waits for one stage at a time instead of draining the ring.
    const int Q = nch * nt;
    Stage<FMT, RT, MB> ring[U];
    int pc = 0, pt = t0;                       // next stage to load
    auto advance = [&](int& c, int& t) {
      if (t + 1 < t1) { ++t; } else if (c + 1 < nch) { ++c; t = t0; }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) { load(pc, pt, ring[u]); advance(pc, pt); }
    // keep the scheduler from sinking loads next to their uses (it would
    // trade the in-flight depth for registers)
    __builtin_amdgcn_sched_barrier(0);
    int cc = 0, ct = t0;                       // stage being multiplied
    int q = 0;
    for (; q + U < Q; q += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        compute(ring[u]);
        if (ct == t1 - 1) epilogue(cc);
        advance(cc, ct);
        load(pc, pt, ring[u]);
        advance(pc, pt);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // last block: the remaining 1..U stages are all in flight; no loads
    // past the end are issued, so the wave's tail carries no dead reads
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q + u < Q) {
        compute(ring[u]);
        if (ct == t1 - 1) epilogue(cc);
        advance(cc, ct);
      }
    }
  }

  if (a.epi == EPI_ARGMAX) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (!own(mb)) continue;
      float bv = best[mb];
      int bi = bidx[mb];
      // across the 16 lanes of this token (rows differ by lane): lowest index on ties
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      const int t = mb * 16 + 4 * g + vslot;
      if (lr == 0) {
        a.am_val[(size_t)blockIdx.x * 64 + t] = bv;
        a.am_idx[(size_t)blockIdx.x * 64 + t] = bi;
      }
    }
  }
}

// ------------------------------------------------------------------ fp32 path
// Plain fp32 GEMM for fp32 models (the small sanity configuration): one
// thread per output column, all token rows; weights in canonical [N][K].
// EPI_PARTIAL writes the unrounded sums to out (one split).
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ W, const float* __restrict__ X,
                                                       int ldx, int n, int k, int m, int epi, void* out,
                                                       int ldo, float* logits, int ldl) {
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
    if (epi == EPI_PARTIAL) {
      ((float*)out)[(size_t)t * ldo + col] = acc[t];
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

// Sum of the S fp32 partials of a PARTIAL launch into one fp32 matrix
// (dflash_linear's plain output); fixed split order.
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ part, int S, size_t count,
                                                        float* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (size_t)gridDim.x * blockDim.x) {
    float v = part[i];
    for (int s = 1; s < S; ++s) v = v + part[(size_t)s * count + i];
    out[i] = v;
  }
}

hipError_t launch_sum_parts(const float* part, int S, size_t count, float* out, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((count + 255) / 256, 2048);
  hipLaunchKernelGGL(sum_parts_kernel, dim3(blocks), dim3(256), 0, s, part, S, count, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------ planning
// The launch has nwg = PR * S work-groups: S K splits (partial-sum epilogue
// only) times PR work-groups per split, each owning a balanced range of row
// tiles that it walks in chunks of RT.  The rule below was fitted to a sweep
// of (RT, S, PR) on MI355X over the 4B/8B/27B-class shapes (weights rotated
// through more than the 256 MiB last-level cache) and lands within 2 % of the
// per-shape optimum summed over the shapes:
//   * RT = 2 for 64 token rows (register budget) and for bf16 partial sums,
//     6 for the fused gate/up (SiLU), 4 otherwise (3 when a work-group's
//     range is exactly three row tiles);
//   * gate/up: one work-group per CU, two when a CU would get more than one
//     chunk; lm-head: two per CU;
//   * partial sums: at most one work-group per CU; S in 1..4 minimises the
//     streamed tile slots per work-group (whole chunks, including the dead
//     row tiles of a partial chunk, times K tiles per wave) plus a small cost
//     per split for writing and re-reading the partials.
Plan make_plan(int fmt, int n, int k, int m, int epi) {
  Plan p;
  p.NW = 4;
  p.MB = (m + 15) / 16;
  p.ntile16 = n / 16;
  p.ktiles = fmt == W_F32 ? 0 : k / tile_k(fmt);
  if (p.MB >= 3) p.RT = 2;
  else if (epi == EPI_SILU) p.RT = 6;
  else if (epi == EPI_ARGMAX) p.RT = 4;
  else p.RT = fmt == W_BF16 ? 2 : 4;
  p.align = epi == EPI_SILU ? 2 : 1;
  const int units = std::max(1, p.ntile16 / p.align);
  p.S = 1;
  if (epi == EPI_PARTIAL) {
    double best = 1e30;
    for (int S = 1; S <= 4; ++S) {
      if (S > 1 && p.ktiles / S < 4) continue;
      const int PR = std::max(1, std::min(units, 256 / S));
      const int tiles = (p.ntile16 + PR - 1) / PR;
      const int chunks = (tiles + p.RT - 1) / p.RT;
      const int kw = (p.ktiles + 4 * S - 1) / (4 * S);
      const double cost = (double)chunks * p.RT * kw + 0.15 * S * p.RT;
      if (cost < best - 1e-9) { best = cost; p.S = S; p.PR = PR; }
    }
    // three row tiles per work-group (the 8B-class QKV projection: 384 tiles
    // on 128 work-groups per split): chunks of 3, so no dead fourth tile is
    // streamed and multiplied (7.7 against 8.6 us a launch)
    if (p.RT == 4 && (p.ntile16 + p.PR - 1) / p.PR == 3) p.RT = 3;
    // ... whose 12 tiles a wave split over eight waves (two per SIMD, 6 tiles
    // each) overlap one wave's dequantisation with the other's MFMAs better
    // than the wider epilogue skew costs (7.6 against 7.3 us a launch; every
    // other partial-sum shape measured slower with eight waves)
    if (p.RT == 3 && p.MB == 2) p.NW = 8;
  } else if (epi == EPI_SILU) {
    const int tiles256 = (p.ntile16 + 255) / 256;
    p.PR = std::min(units, tiles256 > p.RT ? 512 : 256);
  } else {
    p.PR = std::min(units, 512);
  }
  p.nwg = p.PR * p.S;
  p.ngroups = p.PR;
  return p;
}

int gemm_am_blocks(int fmt, int n, int m) {
  if (fmt == W_F32) return 0;
  return make_plan(fmt, n, tile_k(fmt), m, EPI_ARGMAX).nwg;
}

template <int FMT, int RT>
static hipError_t dispatch_mb(int MB, int NW, dim3 grid, const GemmArgs& a, hipStream_t s) {
  switch (MB) {
    case 1: hipLaunchKernelGGL((gemm_stream_kernel<FMT, RT, 1, 4>), grid, dim3(256), 0, s, a); break;
    case 2:
      if (NW == 8) hipLaunchKernelGGL((gemm_stream_kernel<FMT, RT, 2, 8>), grid, dim3(512), 0, s, a);
      else hipLaunchKernelGGL((gemm_stream_kernel<FMT, RT, 2, 4>), grid, dim3(256), 0, s, a);
      break;
    case 3: hipLaunchKernelGGL((gemm_stream_kernel<FMT, 2, 3, 4>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_stream_kernel<FMT, 2, 4, 4>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int FMT>
static hipError_t dispatch(const Plan& p, const GemmArgs& a, hipStream_t s) {
  dim3 grid(p.nwg);
  if (p.MB >= 3) return dispatch_mb<FMT, 2>(p.MB, 4, grid, a, s);
  switch (p.RT) {
    case 3: return dispatch_mb<FMT, 3>(p.MB, p.NW, grid, a, s);
    case 8: return dispatch_mb<FMT, 8>(p.MB, p.NW, grid, a, s);
    case 6: return dispatch_mb<FMT, 6>(p.MB, p.NW, grid, a, s);
    case 4: return dispatch_mb<FMT, 4>(p.MB, p.NW, grid, a, s);
    default: return dispatch_mb<FMT, 2>(p.MB, p.NW, grid, a, s);
  }
}

// Name of the compiled kernel and launch shape a plan runs: the template
// instance (format, row tile chunk, token row blocks) and the grid.  Launches
// that differ only in their split count run the same kernel on the same grid
// and share a name, so the name is also what a kernel trace can tell apart.
static const char* variant_name(int fmt, const Plan& p) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int>, std::string> names;
  const char* f[4] = {"f32", "bf16", "w8", "w4"};
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_tuple(fmt, p.RT, p.MB, p.NW, p.nwg);
  auto it = names.find(key);
  if (it == names.end()) {
    char buf[48];
    snprintf(buf, sizeof buf, "gemm_%s_t%dm%dw%d_g%d", f[fmt], p.RT, p.MB, p.NW, p.nwg);
    it = names.emplace(key, std::string(buf)).first;
  }
  return it->second.c_str();
}

hipError_t launch_gemm_plan(const GemmCall& c, const Workspace& w, hipStream_t s, const Plan& p) {
  const GemmW& W = *c.W;
  if (p.S < 1 || p.S > MAX_SPLITS || p.PR < 1 || p.nwg != p.PR * p.S) return hipErrorInvalidValue;
  // the kernel splits row tiles and K tiles with 32-bit products
  if (p.align < 1 || (uint64_t)(p.ntile16 / p.align) * p.PR >= (1ull << 32) ||
      (uint64_t)p.ktiles * p.S >= (1ull << 32))
    return hipErrorInvalidValue;
  if (p.RT != 2 && p.RT != 3 && p.RT != 4 && p.RT != 6 && p.RT != 8) return hipErrorInvalidValue;
  if (p.MB >= 3 && p.RT != 2) return hipErrorInvalidValue;
  if (p.NW != 4 && !(p.NW == 8 && p.MB == 2)) return hipErrorInvalidValue;
  if (c.epi == EPI_SILU && p.RT % 2) return hipErrorInvalidValue;
  if (c.epi == EPI_PARTIAL && (size_t)p.S * c.m * W.n > w.part_floats) return hipErrorInvalidValue;
  if (c.epi != EPI_PARTIAL && p.S != 1) return hipErrorInvalidValue;
  if (c.epi == EPI_ARGMAX && p.nwg > w.am_cap) return hipErrorInvalidValue;
  GemmArgs a;
  a.w = (const uint8_t*)W.w; a.s = (const uint16_t*)W.s; a.x = (const uint16_t*)c.x;
  a.n = W.n; a.k = W.k; a.ktiles = p.ktiles; a.ntile16 = p.ntile16; a.m = c.m; a.splits = p.S; a.align = p.align;
  a.epi = c.epi; a.part = c.part; a.out = c.out; a.otype = c.otype;
  a.logits = c.logits; a.ldl = c.ldl; a.row0 = c.row0;
  a.am_val = w.am_val; a.am_idx = w.am_idx; a.status = c.status;
  a.mlo = 0x000F000Fu; a.mhi = 0x00F000F0u; a.magic = 0x64006400u;
  hipError_t e;
  if (W.fmt == W_BF16) e = dispatch<W_BF16>(p, a, s);
  else if (W.fmt == W_W8) e = dispatch<W_W8>(p, a, s);
  else e = dispatch<W_W4>(p, a, s);
  if (e != hipSuccess || c.epi != EPI_ARGMAX) return e;
  return launch_argmax_final(w.am_val, w.am_idx, p.nwg, c.row0, c.m - c.row0, c.am_out, s);
}

hipError_t launch_gemm(const GemmCall& c, const Workspace& w, hipStream_t s, const char** variant,
                       double* bytes, int* splits, double* io_bytes) {
  const GemmW& W = *c.W;
  size_t wb, sb;
  packed_bytes(W.fmt, W.n, W.k, &wb, &sb);
  // algorithmic bytes: the packed weights and their scales, streamed once
  if (bytes) *bytes = (double)(wb + sb);
  // besides them: the 16-bit activations read once and the product written
  // once in its consumer's type (fp32 sums, bf16 SiLU rows, or the fp32
  // logits when they are kept)
  if (io_bytes) {
    double out_b = 0;
    if (c.epi == EPI_PARTIAL) out_b = 4.0 * c.m * W.n;
    else if (c.epi == EPI_SILU) out_b = 2.0 * c.m * (W.n / 2);
    else if (c.logits) out_b = 4.0 * c.m * W.n;
    *io_bytes = 2.0 * c.m * W.k + out_b;
  }
  if (W.fmt == W_F32) {
    if (variant) *variant = "gemm_f32";
    if (splits) *splits = 1;
    const int ncols = c.epi == EPI_SILU ? W.n / 2 : W.n;
    float* lg = c.epi == EPI_ARGMAX ? w.logits_tmp : nullptr;
    void* out = c.epi == EPI_PARTIAL ? (void*)c.part : c.out;
    const int ldo = c.epi == EPI_PARTIAL ? W.n : W.n / 2;
    hipLaunchKernelGGL(gemm_f32_kernel, dim3((ncols + 255) / 256), dim3(256), 0, s, (const float*)W.w,
                       (const float*)c.x, c.ldx, W.n, W.k, c.m, c.epi, out, ldo, lg, W.n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || c.epi != EPI_ARGMAX) return e;
    return launch_argmax_rows(w.logits_tmp, W.n, W.n, c.row0, c.m - c.row0, c.am_out, c.logits, c.ldl, s);
  }
  if (c.m > MAX_ROWS) {
    if (variant)
      *variant = W.fmt == W_W4   ? (c.epi == EPI_SILU ? "gemm_dense_w4_silu" : "gemm_dense_w4")
                 : W.fmt == W_W8 ? (c.epi == EPI_SILU ? "gemm_dense_w8_silu" : "gemm_dense_w8")
                                 : (c.epi == EPI_SILU ? "gemm_dense_bf16_silu" : "gemm_dense_bf16");
    return launch_gemm_dense(c, w, s, splits);
  }
  const Plan p = make_plan(W.fmt, W.n, W.k, c.m, c.epi);
  if (variant) *variant = variant_name(W.fmt, p);
  if (splits) *splits = p.S;
  return launch_gemm_plan(c, w, s, p);
}

}  // namespace dfl
