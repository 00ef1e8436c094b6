// Dense GEMM for prompt chunks (64 < m <= 1024 token rows): the same packed
// int4 / int8 / bf16 weights and tiled activations as the skinny GEMM,
// arranged so that MFMAs rather than the weight stream set the time.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "gemm_dev.h"

namespace dfl {

// ------------------------------------------------------- dense (prompt chunks)
// W4 / W8 / BF16 GEMM for prompt chunks of m = 16*j rows (j <= 64): enough rows
// that the MFMAs, not the weight stream, set the time, so activations are
// reused across many weight rows instead of being re-read per row tile.
// Work-group = MT token blocks (MT = 4 or 8: 64 or 128 rows) x 16 row tiles
// (256 weight rows) x one of S K ranges; wave w owns row tiles 4w..4w+3 for
// all MT token blocks.  Per K tile (128 columns) the work-group stages the
// 4*MT activation fragments (MT blocks x 4 MFMA steps, 1 KiB each) in LDS by
// direct global->LDS loads while each wave holds its four row tiles' weights
// (and group scales) in registers; both are double-buffered, so tile t+1
// loads while tile t is multiplied.  At most 256 registers a lane, so that
// two waves share each SIMD and one's MFMAs overlap the other's
// dequantisation and group-scale FMAs.  The arithmetic is the stream
// kernel's: fp16 MFMA on the raw codes, one fp32 sum per 64-wide group,
// scaled by the group's fp16 scale and accumulated in fp32 (W8: one fp32
// sum per row, times the row's fp16 scale at the end; BF16: bf16 MFMA on
// the stored weights, fp32 sums).
// MT = 8 halves the dequantisation and the weight loads per MFMA (each
// weight tile serves 128 rows) but needs 128 accumulators per lane and halves
// the grid; it is taken for the large int4 shapes of long chunks (measured on
// the 8B-class prompt pass: gate/up 11 % and down 5 % faster at 1024 rows,
// QKV and O no faster).

// The pipeline's register loads go the same way (weights non-temporal): the
// explicit per-tile wait is then the only one, and every register they write
// is read only after it (the waits are scheduling barriers).
__device__ __forceinline__ uint4 gload16_nt(const void* p) {
  uint4 r;
  asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(r) : "v"(p) : "memory");
  return r;
}
__device__ __forceinline__ uint32_t gload4(const void* p) {
  uint32_t r;
  asm volatile("global_load_dword %0, %1, off" : "=v"(r) : "v"(p) : "memory");
  return r;
}
constexpr int DENSE_MAX_ROWS = 1024;

// FMT W4: per 128-column step one 1 KiB tile and one scale dword per row
// tile; W8: two 64-column tiles per row tile and the per-row scale applied to
// the finished sum (as the stream kernel does); BF16: four 32-column tiles
// per row tile, MFMA bf16 on the weights as stored (bf16 activations).
// DENSE_RW: row tiles per wave (4; 2 for the 128-row bf16 shape)
template <int FMT, int EPI, int DENSE_MT, int DENSE_RW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_dense_kernel(GemmArgs a,
                                                                                       int kt_per) {
  static_assert(FMT == W_W4 || FMT == W_W8 || FMT == W_BF16, "dense kernel: int4, int8 or bf16 weights");
  static_assert((DENSE_MT == 4 && DENSE_RW == 4) || (DENSE_MT == 8 && DENSE_RW == 4 && FMT != W_BF16) ||
                    (DENSE_MT == 8 && DENSE_RW == 2 && FMT == W_BF16),
                "dense kernel: 64 rows x 4 row tiles, or 128 rows x 4 (int4, int8) / x 2 (bf16)");
  constexpr int WT = FMT == W_W4 ? 1 : (FMT == W_W8 ? 2 : 4);  // weight tiles per row tile and 128-column step
  constexpr int WLOADS = FMT == W_BF16 ? 4 * DENSE_RW : 2 * DENSE_RW;  // register loads per step
  __shared__ __attribute__((aligned(16))) uint8_t xs0[DENSE_MT * 4 * 1024];
  __shared__ __attribute__((aligned(16))) uint8_t xs1[DENSE_MT * 4 * 1024];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, g = lane >> 4;
  const int nblk = (a.m + 15) >> 4;
  // Work-groups are dealt to the 8 XCDs round-robin by index.  When the
  // row-tile groups come in multiples of 8, XCD x takes row-tile groups
  // x, x + 8, ... and runs all token groups of one before the next, so the
  // weights a group reads stay in that XCD's L2 for all of its token groups.
  const int ngx = (a.ntile16 + 4 * DENSE_RW - 1) / (4 * DENSE_RW), ngy = (nblk + DENSE_MT - 1) / DENSE_MT;
  const int id = blockIdx.x;
  int gx, gy;
  if (ngx % 8 == 0) {
    gx = (id / (8 * ngy)) * 8 + id % 8;
    gy = (id / 8) % ngy;
  } else {
    gx = id % ngx;
    gy = id / ngx;
  }
  const int tb0 = gy * DENSE_MT;
  const int rt0 = gx * (4 * DENSE_RW) + wave * DENSE_RW;
  const int sidx = blockIdx.z;
  const int ptiles = a.k >> 7;               // 128-column steps
  const int kt0 = sidx * kt_per, kt1 = min(ptiles, kt0 + kt_per);
  const uint32_t mlo = a.mlo, mhi = a.mhi, magic = a.magic;
  const size_t xfrag = (size_t)(a.k >> 5);
  uint32_t rtile[DENSE_RW];                  // row tiles past the end re-read the last one
#pragma unroll
  for (int i = 0; i < DENSE_RW; ++i) rtile[i] = (uint32_t)min(rt0 + i, a.ntile16 - 1);

  floatx4 acc[DENSE_MT][DENSE_RW];
#pragma unroll
  for (int tb = 0; tb < DENSE_MT; ++tb)
#pragma unroll
    for (int i = 0; i < DENSE_RW; ++i) acc[tb][i] = floatx4{0.f, 0.f, 0.f, 0.f};

  // this wave's DENSE_MT of the K tile's 4*DENSE_MT activation fragments:
  // fragment f = DENSE_MT*w + j is token block f/4 (blocks past the chunk
  // re-read its last one), MFMA step f%4
  auto stage = [&](int t, uint8_t* xs) {
#pragma unroll
    for (int j = 0; j < DENSE_MT; ++j) {
      const int f = DENSE_MT * wave + j, tb = min(tb0 + (f >> 2), nblk - 1);
      const uint16_t* src = a.x + ((size_t)tb * xfrag + (size_t)t * 4 + (f & 3)) * 512 + lane * 8;
      lds_dma16(src, (uint32_t)(uintptr_t)(lds_ptr)(xs + f * 1024));
    }
  };
  // WLOADS per step: per row tile W4 a tile and a scale dword, W8 two
  // tiles, BF16 four tiles
  auto wload = [&](int t, uint4 (&w)[DENSE_RW][WT], uint32_t (&sc)[DENSE_RW]) {
#pragma unroll
    for (int i = 0; i < DENSE_RW; ++i) {
      const size_t tile = (size_t)rtile[i] * a.ktiles + (size_t)t * WT;
#pragma unroll
      for (int j = 0; j < WT; ++j) w[i][j] = gload16_nt(a.w + (tile + j) * 1024 + lane * 16);
      if (FMT == W_W4) sc[i] = gload4(a.s + tile * 32 + lr * 2);
    }
  };
  // Per 64-wide group: its two weight steps dequantised for the 4 row tiles,
  // its two activation steps of the 4 token blocks read from LDS, then for
  // each half of the token blocks 8 independent MFMA chains (2 MFMAs each)
  // before their sums are scaled into the accumulators, so no MFMA waits on
  // the one before it and no FMA on an MFMA just issued.
  auto compute = [&](const uint8_t* xs, const uint4 (&w)[DENSE_RW][WT], const uint32_t (&sc)[DENSE_RW]) {
    if (FMT == W_BF16) {
      // step ks is tile ks of each row tile, an MFMA operand as stored
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int tb = 0; tb < DENSE_MT; ++tb) {
          const bf16x8 x = __builtin_bit_cast(bf16x8, *(const uint4*)(xs + (tb * 4 + ks) * 1024 + lane * 16));
#pragma unroll
          for (int i = 0; i < DENSE_RW; ++i)
            acc[tb][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, __builtin_bit_cast(bf16x8, w[i][ks & (WT - 1)]),
                                                                 acc[tb][i], 0, 0, 0);
        }
      return;
    }
    if (FMT == W_W8) {
      // 4 MFMA steps straight into the accumulators; step ks is dwords
      // 2(ks%2), 2(ks%2)+1 of tile ks/2
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half8 b[DENSE_RW];
#pragma unroll
        for (int i = 0; i < DENSE_RW; ++i) {
          const uint4 wt = w[i][(ks >> 1) & (WT - 1)];
          b[i] = (ks & 1) ? deq_w8(wt.z, wt.w, magic) : deq_w8(wt.x, wt.y, magic);
        }
#pragma unroll
        for (int tb = 0; tb < DENSE_MT; ++tb) {
          const half8 x = __builtin_bit_cast(half8, *(const uint4*)(xs + (tb * 4 + ks) * 1024 + lane * 16));
#pragma unroll
          for (int i = 0; i < DENSE_RW; ++i)
            acc[tb][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x, b[i], acc[tb][i], 0, 0, 0);
        }
      }
      return;
    }
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      half8 b[DENSE_RW][2];
      float sg[DENSE_RW];
#pragma unroll
      for (int i = 0; i < DENSE_RW; ++i) {
        const uint32_t wd0 = gg ? w[i][0].z : w[i][0].x, wd1 = gg ? w[i][0].w : w[i][0].y;
        b[i][0] = deq_w4(wd0, mlo, mhi, magic);
        b[i][1] = deq_w4(wd1, mlo, mhi, magic);
        sg[i] = (float)h2(sc[i])[gg];
      }
#pragma unroll
      for (int hb = 0; hb < DENSE_MT; hb += 2) {
        half8 x[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            x[j][h] = __builtin_bit_cast(half8, *(const uint4*)(xs + ((hb + j) * 4 + 2 * gg + h) * 1024 + lane * 16));
        floatx4 tmp[2][DENSE_RW];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < DENSE_RW; ++i)
            tmp[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x[j][0], b[i][0], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < DENSE_RW; ++i)
            tmp[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(x[j][1], b[i][1], tmp[j][i], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < DENSE_RW; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[hb + j][i][v] += sg[i] * tmp[j][i][v];
      }
    }
  };
  // Every tile's wait lets the next tile's loads (DENSE_MT fragment DMAs and
  // WLOADS register loads, the youngest) stay in flight; past the last
  // tile the loads re-read it, so the wait is always the same.  It is kept
  // apart from the first use so that the compiler adds none there.
  auto wait_tile = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vm_wait(DENSE_MT + WLOADS));
    asm volatile("s_nop 0");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();            // every wave's fragments of the tile are in LDS
  };
  uint4 w0[DENSE_RW][WT], w1[DENSE_RW][WT];
  uint32_t s0[DENSE_RW], s1[DENSE_RW];
  // tile t from stage (xs, w, sc); tile t + 1 goes to stage (xn, wn, sn), the
  // one tile t - 1 used: the barrier first lets every wave finish with it
  auto step = [&](int t, const uint8_t* xs, const uint4 (&w)[DENSE_RW][WT], const uint32_t (&sc)[DENSE_RW],
                  uint8_t* xn, uint4 (&wn)[DENSE_RW][WT], uint32_t (&sn)[DENSE_RW]) {
    __builtin_amdgcn_s_barrier();
    const int tn = min(t + 1, kt1 - 1);
    stage(tn, xn);
    wload(tn, wn, sn);
    wait_tile();
    compute(xs, w, sc);
  };
  if (kt0 < kt1) {
    stage(kt0, xs0);
    wload(kt0, w0, s0);
    for (int t = kt0; t < kt1; t += 2) {
      step(t, xs0, w0, s0, xs1, w1, s1);
      if (t + 1 >= kt1) break;
      step(t + 1, xs1, w1, s1, xs0, w0, s0);
    }
    // the last loads re-read a tile nobody uses: let them land before the
    // work-group (and its LDS) ends
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
  }

  // lane (lr, g) holds weight row (rt0 + i)*16 + lr for tokens
  // (tb0 + tb)*16 + 4g + v
  // W8: the row's fp16 scale on the finished sum; W4 sums are scaled already
  auto scale_of = [&](int n) -> float {
    return FMT == W_W8 ? (float)__builtin_bit_cast(_Float16, a.s[n]) : 1.0f;
  };
  if (EPI == EPI_PARTIAL) {
    float* part = a.part + (size_t)sidx * a.m * a.n;
#pragma unroll
    for (int i = 0; i < DENSE_RW; ++i) {
      if (rt0 + i >= a.ntile16) continue;
      const int n = (rt0 + i) * 16 + lr;
      const float sc = scale_of(n);
#pragma unroll
      for (int tb = 0; tb < DENSE_MT; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = (tb0 + tb) * 16 + 4 * g + v;
          if (t < a.m) part[(size_t)t * a.n + n] = acc[tb][i][v] * sc;
        }
    }
  } else {  // EPI_SILU: row tiles (2p, 2p+1) are a (gate, up) pair
    const int rnd = a.otype == T_F32 ? T_F32 : T_BF16;
    const int half_n = a.n >> 1;
#pragma unroll
    for (int p = 0; p < DENSE_RW / 2; ++p) {
      if (rt0 + 2 * p + 1 >= a.ntile16) continue;
      const int n_out = ((rt0 >> 1) + p) * 16 + lr;
      const int ng = (rt0 + 2 * p) * 16 + lr;
      const float sg = scale_of(ng), su = scale_of(ng + 16);
#pragma unroll
      for (int tb = 0; tb < DENSE_MT; ++tb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = (tb0 + tb) * 16 + 4 * g + v;
          if (t >= a.m) continue;
          const float gv = act_round(rnd, acc[tb][2 * p][v] * sg);
          const float uv = act_round(rnd, acc[tb][2 * p + 1][v] * su);
          const float sv = gv * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-gv * 1.4426950408889634f));
          store_act(a.out, act_index(t, n_out, 0, half_n), a.otype, sv * uv, a.status);
        }
    }
  }
}

// token blocks per work-group: 8 for int4 chunks of more than 512 rows with
// a wide N (gate/up) or a deep K (down), and for bf16 chunks of more than 512
// rows (whose weights, 4x the bytes of int4 ones, would otherwise load
// faster than a CU's vector-memory path moves them), else 4; row tiles per
// wave: 2 for that bf16 shape (registers), else 4
static int dense_mt(int fmt, int n, int k, int m) {
  if (fmt == W_BF16 || fmt == W_W8) return m > 512 ? 8 : 4;
  return m > 512 && (n >= 16384 || k >= 8192) ? 8 : 4;
}
static int dense_rw(int fmt, int n, int k, int m) { return fmt == W_BF16 && dense_mt(fmt, n, k, m) == 8 ? 2 : 4; }

// K splits of a dense launch: partial sums go to S slices so that the grid
// reaches the chip's 256 CUs, each split keeping at least 4 K tiles
int dense_splits(int fmt, int n, int k, int m, int epi) {
  if (epi != EPI_PARTIAL) return 1;
  const int ktiles = k / 128, mt = dense_mt(fmt, n, k, m), rw = dense_rw(fmt, n, k, m);
  const int base = ((n / 16 + 4 * rw - 1) / (4 * rw)) * ((m / 16 + mt - 1) / mt);
  int S = 1;
  while (S < MAX_SPLITS && base * S < 256 && ktiles / (2 * S) >= 4) S *= 2;
  return S;
}

bool dense_ok(int fmt, int n, int k, int m, int epi) {
  return (fmt == W_W4 || fmt == W_W8 || fmt == W_BF16) && m > MAX_ROWS && m <= DENSE_MAX_ROWS && m % 16 == 0 &&
         n % 16 == 0 && k % 128 == 0 && (epi == EPI_PARTIAL || (epi == EPI_SILU && n % 32 == 0));
}

template <int FMT, int MT, int RW = 4>
static void launch_dense(int epi, dim3 grid, hipStream_t s, const GemmArgs& a, int kt_per) {
  if (epi == EPI_PARTIAL)
    hipLaunchKernelGGL((gemm_dense_kernel<FMT, EPI_PARTIAL, MT, RW>), grid, dim3(256), 0, s, a, kt_per);
  else
    hipLaunchKernelGGL((gemm_dense_kernel<FMT, EPI_SILU, MT, RW>), grid, dim3(256), 0, s, a, kt_per);
}

hipError_t launch_gemm_dense(const GemmCall& c, const Workspace& w, hipStream_t s, int* splits) {
  const GemmW& W = *c.W;
  if (!dense_ok(W.fmt, W.n, W.k, c.m, c.epi)) return hipErrorInvalidValue;
  const int S = dense_splits(W.fmt, W.n, W.k, c.m, c.epi), mt = dense_mt(W.fmt, W.n, W.k, c.m),
            rw = dense_rw(W.fmt, W.n, W.k, c.m);
  if (c.epi == EPI_PARTIAL && (size_t)S * c.m * W.n > w.part_floats) return hipErrorInvalidValue;
  GemmArgs a{};
  a.w = (const uint8_t*)W.w; a.s = (const uint16_t*)W.s; a.x = (const uint16_t*)c.x;
  a.n = W.n; a.k = W.k; a.ktiles = W.k / tile_k(W.fmt); a.ntile16 = W.n / 16; a.m = c.m; a.splits = S; a.align = 1;
  a.epi = c.epi; a.part = c.part; a.out = c.out; a.otype = c.otype; a.status = c.status;
  a.mlo = 0x000F000Fu; a.mhi = 0x00F000F0u; a.magic = 0x64006400u;
  const int kt_per = (W.k / 128 + S - 1) / S;
  const dim3 grid(((a.ntile16 + 4 * rw - 1) / (4 * rw)) * ((c.m / 16 + mt - 1) / mt), 1, S);
  if (W.fmt == W_W4 && mt == 8) launch_dense<W_W4, 8>(c.epi, grid, s, a, kt_per);
  else if (W.fmt == W_W4) launch_dense<W_W4, 4>(c.epi, grid, s, a, kt_per);
  else if (W.fmt == W_W8 && mt == 8) launch_dense<W_W8, 8>(c.epi, grid, s, a, kt_per);
  else if (W.fmt == W_W8) launch_dense<W_W8, 4>(c.epi, grid, s, a, kt_per);
  else if (mt == 8) launch_dense<W_BF16, 8, 2>(c.epi, grid, s, a, kt_per);
  else launch_dense<W_BF16, 4>(c.epi, grid, s, a, kt_per);
  if (splits) *splits = S;
  return hipGetLastError();
}

}  // namespace dfl
