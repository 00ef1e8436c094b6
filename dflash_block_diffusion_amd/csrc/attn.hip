// Attention pieces of the draft+verify step.
//
// qk_rope_kernel: per-head RMSNorm of q and k over head_dim (the per-head form
// mirror-sd's README, "The Story", had to fix: a norm across all channels gave
// cosine ~0.5), then neox split-half RoPE (pairs (i, i+d/2), the convention of
// mx.fast.rope(traditional=False) named there), one rounding to the
// activation format, then q goes to the query buffer and k/v to the paged KV
// cache at slot(pos) = page_table[pos/64]*64 + pos%64.  A K page of one KV
// head is [64 keys][d] (row-major); a V page is stored transposed, [d][64
// keys], so that both MFMA operands of the attention (K for q.k, V^T for
// p.v) are contiguous 16-byte runs along their reduction dimension.
//
// attn_*_kernel: softmax(q k^T / sqrt(d)) v of the B block rows over the
// cache positions 0..n+B-1.  Verify (causal=1): row i (position n+i) sees
// keys 0..n+i -- the committed context plus the block causally.  Draft
// (causal=0): every block slot sees every committed context row and every
// block slot (the drafter denoises the block in one bidirectional pass,
// mlx-dspark v0.0.3 "Highlights").  Split-KV: each work-group takes 256 keys
// (128 in small states) of one KV head for all G*B query rows of that head
// (GQA) and writes an
// unnormalised partial (o, max, sum); attn_combine merges the splits -- the
// two-pass structure of the long-context verify attention in the dflash-mlx
// note ("Technical challenges", JIT SDPA 2-pass for N >= 1024), here used at
// every length so the graph of a step is length-independent.
//
// attn_prefill_kernel: the causal attention of a prompt chunk (more than 64
// rows) in one pass with an online softmax: enough query rows per KV head
// fill the chip without splitting the keys, so no partials and no combine.
#include "common.h"

namespace dfl {

static constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------------ QK norm + RoPE
// One wave per (row, head); a work-group takes R consecutive rows of one
// head: 4 when the launch has many rows (a prompt chunk), 1 otherwise.
// Work-groups are numbered so that the G q heads and the k/v head of KV head
// h come from work-groups h, h + hkv, h + 2 hkv, ...: the XCDs take
// work-groups round-robin, so with hkv = 8 (every benchmark shape) the
// outputs the attention of KV head h reads are written through XCD h's L2,
// where that attention runs too.
// S is the QKV projection's K-split count: the partial sums are loaded as
// straight-line code (a run-time count made every load conditional and let
// the compiler wait for all of them at branch boundaries).
template <int R, int S>
__global__ __launch_bounds__(64 * R) void qk_rope_kernel(RopeCall c) {
  // the committed length and the pending context count go out first (scalar loads)
  const int n = *c.dev_n;
  const int p = c.dev_p && !c.ctx_at_n ? *c.dev_p : 0;
  const int L = blockIdx.x + gridDim.x * blockIdx.y;
  const int grp = c.hkv, per = c.hq / c.hkv + 1;       // a KV head's q heads and its k/v head
  const int hk = L % grp, j = L / grp;
  const int hi = j % per, rg = j / per;
  const int head = hi < per - 1 ? hk * (per - 1) + hi : c.hq + hk;
  const int row = R == 1 ? rg : rg * R + (int)(threadIdx.x >> 6);
  const int lane = R == 1 ? (int)threadIdx.x : (int)(threadIdx.x & 63);
  if (R > 1 && row >= c.block_rows + c.ctx_rows) return;   // past the launch's rows (whole waves)
  if (row >= c.block_rows && head < c.hq) return;      // context rows only carry k/v
  const int d = c.d, half = d >> 1;
  const bool act = lane < half;
  const int i = act ? lane : 0;
  const bool kv = head >= c.hq;
  const int kh = head - c.hq;
  const int src = head * d;                 // q heads, then k heads, then v heads
  const int vs = (c.hq + c.hkv + kh) * d;
  const float* gain = kv ? c.k_norm : c.q_norm;
  // every load that does not depend on the committed length
  const float* base = c.qkv.p + (size_t)row * c.qkv.ld;
  float q1[S], q2[S], v1[S], v2[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    q1[s] = base[(size_t)s * c.qkv.stride + src + i];
    q2[s] = base[(size_t)s * c.qkv.stride + src + i + half];
  }
  if (kv) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      v1[s] = base[(size_t)s * c.qkv.stride + vs + i];
      v2[s] = base[(size_t)s * c.qkv.stride + vs + i + half];
    }
  }
  const float g1 = gain[i], g2 = gain[i + half];
  const int pos = row < c.block_rows ? n + row : (c.ctx_at_n ? n : n - p) + (row - c.block_rows);
  if ((row >= c.block_rows && !c.ctx_at_n && row - c.block_rows >= p) || pos < 0 || pos >= c.capacity) return;
  const float cs = c.cos_t[(size_t)pos * half + i];
  const float sn = c.sin_t[(size_t)pos * half + i];
  const int page = kv ? c.page_table[pos / PAGE] : 0;
  // the QKV projection is materialised in the activation format; the splits
  // are added in split order
  float y1 = q1[0], y2 = q2[0];
#pragma unroll
  for (int s = 1; s < S; ++s) { y1 = y1 + q1[s]; y2 = y2 + q2[s]; }
  const float x1 = act ? act_round(c.atype, y1) : 0.f;
  const float x2 = act ? act_round(c.atype, y2) : 0.f;
  const float ss = wave_sum_full(x1 * x1 + x2 * x2);   // every lane of the wave is active here
  const float r = 1.0f / sqrtf(ss / (float)d + c.eps);
  const float a = x1 * r * g1;
  const float b = x2 * r * g2;
  const float o1 = a * cs - b * sn;
  const float o2 = b * cs + a * sn;
  if (!act) return;
  if (!kv) {
    const size_t q = ((size_t)row * c.hq + head) * d;
    store_act(c.q_out, q + i, c.atype, o1);
    store_act(c.q_out, q + i + half, c.atype, o2);
  } else {
    float w1 = v1[0], w2 = v2[0];
#pragma unroll
    for (int s = 1; s < S; ++s) { w1 = w1 + v1[s]; w2 = w2 + v2[s]; }
    const size_t slot = (((size_t)page * c.hkv + kh) * PAGE + (pos % PAGE)) * d;
    store_act(c.kc, slot + i, c.atype, o1);
    store_act(c.kc, slot + i + half, c.atype, o2);
    const size_t vt = ((size_t)page * c.hkv + kh) * PAGE * d + (pos % PAGE);   // V^T page: [d][64]
    store_act(c.vc, vt + (size_t)i * PAGE, c.atype, w1);
    store_act(c.vc, vt + (size_t)(i + half) * PAGE, c.atype, w2);
  }
}

template <int R>
static void launch_qk_rope_r(const RopeCall& c, dim3 grid, hipStream_t s) {
  switch (c.qkv.S) {
    case 1: hipLaunchKernelGGL((qk_rope_kernel<R, 1>), grid, dim3(64 * R), 0, s, c); break;
    case 2: hipLaunchKernelGGL((qk_rope_kernel<R, 2>), grid, dim3(64 * R), 0, s, c); break;
    case 3: hipLaunchKernelGGL((qk_rope_kernel<R, 3>), grid, dim3(64 * R), 0, s, c); break;
    case 4: hipLaunchKernelGGL((qk_rope_kernel<R, 4>), grid, dim3(64 * R), 0, s, c); break;
    case 5: hipLaunchKernelGGL((qk_rope_kernel<R, 5>), grid, dim3(64 * R), 0, s, c); break;
    case 6: hipLaunchKernelGGL((qk_rope_kernel<R, 6>), grid, dim3(64 * R), 0, s, c); break;
    case 7: hipLaunchKernelGGL((qk_rope_kernel<R, 7>), grid, dim3(64 * R), 0, s, c); break;
    default: hipLaunchKernelGGL((qk_rope_kernel<R, 8>), grid, dim3(64 * R), 0, s, c); break;
  }
}

hipError_t launch_qk_rope(const RopeCall& c, hipStream_t s) {
  const int rows = c.block_rows + c.ctx_rows;
  if (c.qkv.S < 1 || c.qkv.S > MAX_SPLITS) return hipErrorInvalidValue;
  if (rows > 64)
    launch_qk_rope_r<4>(c, dim3((rows + 3) / 4, c.hq + c.hkv), s);
  else
    launch_qk_rope_r<1>(c, dim3(rows, c.hq + c.hkv), s);
  return hipGetLastError();
}

// ------------------------------------------------------------ MFMA attention
struct AttnArgs {
  const uint16_t* q; const uint16_t* kc; const uint16_t* vc; const int* pt;
  const int* dev_n; int B; int causal; int hq, hkv; float scale2;   // scale * log2(e)
  int npages;
  float* o_part; float* ml_part;
  void* out; int otype; int32_t* status;   // final rows when one split holds every key
};




// 16 bytes per lane from sbase + voff to LDS at lds + 16 * lane.  The base
// and the LDS offset are wave-uniform (page bases read with readlane, the
// work-group's LDS buffers, the scalar wave index), so they stay in SGPRs and
// a load costs no vector address arithmetic.  Issued from asm (untracked by
// the compiler's wait analysis); callers wait with explicit vmcnt waits.
__device__ __forceinline__ const void* sgpr_ptr(const void* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16_s(uint32_t voff, const void* sbase, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sgpr_ptr(sbase)),
               "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory", "m0");
}

// K page granule swizzle: key bits 0-1 and 3-4, so that the 16 keys
// {8a + 4h + b : a, b < 4} that one score tile reads (h fixed) fall in 16
// different bank groups
__device__ __forceinline__ int kswz(int key) { return (key & 3) | (((key >> 3) & 3) << 2); }

// head_dim 128, bf16 q/k/v.  Work-group = (split of 64*ATTN_PAGES keys: 256,
// or 128 for states of at most ATTN_SMALL_CAP positions, where most of a
// 256-key split would be past the keys; KV head; group of NW row blocks), one
// wave per 16-row block of the head's G*B query rows (row r = token r/G,
// query head h*G + r%G).
//  1. Every wave issues its share of the split's K pages and V^T pages as
//     direct global->LDS 16-byte loads (128 or 64 KiB in flight per
//     work-group, no registers held).  16-byte granules are XOR-swizzled inside each row so
//     that the fragment reads below hit 16 different bank groups:
//       K page  granule (key, c = d/8)    at key*16 + (c ^ kswz(key))
//       V^T page granule (d, c = key/8)   at d*8 + (c ^ ((d >> 1) & 7))
//  2. S^T = K Q^T over the whole split (a lane holds 4 keys of one row per
//     16-key tile, tiles ordered so that a lane's 8 keys of a 32-key P.V
//     step are consecutive), the row max on the raw scores, then
//     p = exp2(s * scale*log2e - m) in one fma + exp per score.  Softmax
//     weights stay fp32: each p enters the MFMA as p_hi + p_lo, two bf16
//     values whose sum carries 16 significant bits (p_hi = p truncated,
//     p_lo = the exact remainder rounded to nearest), O^T = V^T P^T.
//  3. Unnormalised partial (o, max, sum) per row; attn_combine merges the
//     splits.  While the keys fit one split (kv_len <= SPLIT) that split's
//     work-groups write the normalised rows themselves and the combine
//     leaves them alone.
// NW row-block waves per work-group (4 or 8): with 8, one staging of a
// split's K / V^T serves all 8 row blocks of a 32-token block's 128 query
// rows per KV head (G = 4), so each split is read from HBM once, not once per
// 4 row blocks.  KH = 2 gives each row block two waves, one per half of the
// split's keys (the halves' partials merged in LDS before the write): twice
// the waves on the same staging, half the dependent score / softmax / P.V
// chain per wave; a half wholly past the keys skips its work.
template <int NW, int ATTN_PAGES, int KH>
__global__ __launch_bounds__(64 * NW * KH) void attn_mfma_kernel(AttnArgs a) {
  constexpr int D = 128;
  constexpr int SPLIT = ATTN_PAGES * PAGE;     // keys per split
  constexpr int NWT = NW * KH;                 // waves per work-group
  constexpr int BPW = 16 / NWT;                // 1 KiB DMA blocks per page and wave
  constexpr int DMAS = BPW * ATTN_PAGES;       // V^T DMAs per wave (and K DMAs)
  constexpr int NT = SPLIT / 16;               // 16-key tiles per split
  constexpr int NTH = NT / KH;                 // 16-key tiles of one key part
  static_assert(KH == 1 || KH == 2, "one or two key parts");
  static_assert((NTH / 2) % 2 == 0, "a key part holds whole 64-key pages");
  static_assert(KH == 1 || NW * 8 * 64 * 16 <= ATTN_PAGES * 16384,
                "the key-part merge keeps 8 KiB of partial outputs a wave in the K staging");
  // K and V^T staging as two LDS objects, so that waiting for the K loads
  // does not also wait for the V^T loads
  __shared__ __attribute__((aligned(16))) uint8_t ldsK[ATTN_PAGES * 16384];
  __shared__ __attribute__((aligned(16))) uint8_t ldsV[ATTN_PAGES * 16384];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wt = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave of the work-group
  const int wave = wt % NW;                    // its row block in the group
  const int kh = wt / NW;                      // its key part: tiles [kh*NTH, (kh+1)*NTH)
  const int lr = lane & 15, g = lane >> 4;
  // work-group L takes KV head L mod hkv: the XCDs take work-groups
  // round-robin, so with hkv = 8 all of a KV head's splits (and both row
  // groups, which then share the staged pages through L2) run on one XCD,
  // the one whose L2 holds that head's q and new keys (qk_rope_kernel) and
  // which runs the combine of its rows
  const int Lw = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int h = Lw % a.hkv;
  const int rest = Lw / a.hkv;
  const int sidx = rest % gridDim.x, zg = rest / gridDim.x;   // split, row group
  const int key0 = sidx * SPLIT;
  const int G = a.hq / a.hkv;
  const int nrb = G * a.B / 16;

  // 1. the split's page indices (one vector load: scalar loads of them would
  //    each wait for the previous one), this wave's q fragments and the
  //    committed length go out together; a split past the keys then leaves.
  const int my_page = a.pt[min(key0 / PAGE + (lane % ATTN_PAGES), a.npages - 1)];
  const int rbi = zg * NW + wave;             // this wave's 16-row block
  const bool live = rbi < nrb;                 // wave-uniform
  const int rb = live ? rbi : nrb - 1;
  const int r = rb * 16 + lr;
  const int tok = r / G, qh = h * G + r % G;
  bf16x8 qf[4];
  {
    const uint16_t* qp = a.q + ((size_t)tok * a.hq + qh) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const uint4*)(qp + 32 * ks));
  }
  const int n = *a.dev_n;
  // 256-key splits: keep the page and q loads above the exit test (only the
  // live path uses them, so the compiler would otherwise issue them after the
  // committed length has arrived, one memory round trip later): attention +
  // combine 13.8 -> 13.6 us a layer at ctx 2048, 14.3 -> 13.9 for the 27B
  // shapes, 18.0 -> 17.8 at ctx 4096 (eight row blocks).  Small states leave
  // more of their 128-key splits dead, whose loads then cost more than the
  // earlier issue saves (10.3 -> 10.5 us).
  if (ATTN_PAGES == 4) asm volatile("" ::: "memory");
  const int kv_len = n + a.B;
  if (key0 >= kv_len) return;                 // uniform over the work-group
  // K pages first, then V^T pages (pages past the table re-read the last
  // one; their keys are masked below, and the arena holds finite values):
  // the scores and the softmax run while the V^T loads are still in flight.
  // Each wave issues DMAS K and then DMAS V^T 1 KiB blocks (16 per 16 KiB
  // page); a lane's byte offset inside a page is the same for every page.
  uint32_t koff[BPW], voff[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int q = (wt + NWT * j) * 64 + lane;   // 16-byte granule of the 16 KiB region
    const int key = q >> 4, ck = (q & 15) ^ kswz(key);
    const int d = q >> 3, cv = (q & 7) ^ ((d >> 1) & 7);
    koff[j] = (uint32_t)(key * D + ck * 8) * 2u;
    voff[j] = (uint32_t)(d * PAGE + cv * 8) * 2u;
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int p = 0; p < ATTN_PAGES; ++p) {
      const size_t pbase = ((size_t)__builtin_amdgcn_readlane(my_page, p) * a.hkv + h) * PAGE * D;
      const uint16_t* base = (half == 0 ? a.kc : a.vc) + pbase;
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        uint8_t* dst = (half == 0 ? ldsK : ldsV) + (size_t)p * 16384 + (wt + NWT * j) * 1024;
        dma16_s(half == 0 ? koff[j] : voff[j], base, lds_addr(dst));
      }
    }
  }
  // this wave's q and K loads are done once at most its V^T loads are
  // outstanding
  __builtin_amdgcn_s_waitcnt(vm_wait(DMAS));
  __builtin_amdgcn_s_barrier();

  // 2. scores of the 256 keys (tile kt holds keys 16kt + 4g + v of row lr).
  //    Splits that end at or before n are visible to every row (the whole
  //    committed context), so only the split holding the block needs the
  //    mask.
  const bool full = key0 + SPLIT <= n;         // uniform
  // a key part wholly past the keys contributes nothing (m = -inf, l = 0)
  const bool work = live && key0 + kh * (SPLIT / KH) < kv_len;   // wave-uniform
  float mx = -INFINITY;
  float lsum = 0.f;
  uint32_t ph[NTH / 2][4], pl[NTH / 2][4];
  if (work) {
    // Score tile kt = 2*ks2 + hh puts key 32*ks2 + 8*(i/4) + 4*hh + i%4 in
    // its row i, so that after the MFMA a lane (lr, g) holds keys
    // 32*ks2 + 8g + 4hh + v (v < 4): the 8 keys it feeds to the P.V step are
    // consecutive and one 16-byte V^T read matches them.  Row i = lr reads
    // key 32*(ks2%2) + 4*hh + 8*(lr/4) + lr%4 of page ks2/2, whose swizzle is
    // kswz = lr; the tile's page and row offsets are immediates.
    uint32_t kb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kb[ks] = (uint32_t)((8 * (lr >> 2) + (lr & 3)) * 256 + (((4 * ks + g) ^ lr) << 4));
    floatx4 acc[NTH];
#pragma unroll
    for (int j = 0; j < NTH; ++j) {
      const int kt = kh * NTH + j;
      const int ks2 = kt >> 1, hh = kt & 1;
      const uint8_t* kt_base = ldsK + (ks2 >> 1) * 16384 + (32 * (ks2 & 1) + 4 * hh) * 256;
      floatx4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const uint4*)(kt_base + kb[ks]));
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], c, 0, 0, 0);
      }
      acc[j] = c;
    }
    if (!full) {
      const int kmax = a.causal ? n + tok : kv_len - 1;     // last key this row sees
#pragma unroll
      for (int j = 0; j < NTH; ++j) {
        const int kt = kh * NTH + j;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (key0 + 32 * (kt >> 1) + 8 * g + 4 * (kt & 1) + v > kmax) acc[j][v] = -INFINITY;
      }
    }
    // the row max on the raw scores (scale2 > 0)
#pragma unroll
    for (int j = 0; j < NTH; ++j) mx = fmaxf(mx, fmaxf(fmaxf(acc[j][0], acc[j][1]), fmaxf(acc[j][2], acc[j][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // masked scores are -inf, so exp2 of them is 0; a row with no visible key
    // in this split subtracts 0 (no NaN) and runs the wave-wide MFMAs with p = 0
    const float ms = mx == -INFINITY ? 0.f : mx * a.scale2;
    mx = mx == -INFINITY ? -INFINITY : ms;       // the partial's max, log2 domain
#pragma unroll
    for (int ks2 = 0; ks2 < NTH / 2; ++ks2) {
      // B operand: key slots e = hh*4+v <-> key 32*(kh*NTH/2 + ks2) + 8g + e
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float pe[4], lo[4];
        uint32_t u[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          pe[v] = __builtin_amdgcn_exp2f(fmaf(acc[2 * ks2 + hh][v], a.scale2, -ms));
          lsum += pe[v];
          u[v] = __float_as_uint(pe[v]);
          lo[v] = pe[v] - __uint_as_float(u[v] & 0xffff0000u);   // exact
        }
        ph[ks2][2 * hh] = __builtin_amdgcn_perm(u[1], u[0], 0x07060302u);
        ph[ks2][2 * hh + 1] = __builtin_amdgcn_perm(u[3], u[2], 0x07060302u);
        pl[ks2][2 * hh] = pack_bf16_rne(lo[0], lo[1]);
        pl[ks2][2 * hh + 1] = pack_bf16_rne(lo[2], lo[3]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();                  // every wave's V^T loads are in LDS
  if (KH == 1 && !live) return;
  floatx4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // a lane's V^T fragment: row d = 16*dt + lr (swizzle (d/2)%8 = (lr/2)%8),
  // keys 8g..8g+7 of the 32-key step = granule 4*(ks2%2) + g; the step's page
  // and the row tile are immediates
  uint32_t vb[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) vb[k] = (uint32_t)((lr * 8 + ((4 * k + g) ^ ((lr >> 1) & 7))) * 16);
  if (work) {
#pragma unroll
    for (int ks2 = 0; ks2 < NTH / 2; ++ks2) {
      const bf16x8 pfh = __builtin_bit_cast(bf16x8, uint4{ph[ks2][0], ph[ks2][1], ph[ks2][2], ph[ks2][3]});
      const bf16x8 pfl = __builtin_bit_cast(bf16x8, uint4{pl[ks2][0], pl[ks2][1], pl[ks2][2], pl[ks2][3]});
      const uint8_t* vpage = ldsV + ((kh * NTH / 2 + ks2) >> 1) * 16384;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 vf = __builtin_bit_cast(bf16x8, *(const uint4*)(vpage + dt * 2048 + vb[ks2 & 1]));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfh, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfl, o[dt], 0, 0, 0);
      }
    }
  }

  // 3. partials: o (unnormalised), m (log2 domain) and l per query row
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (KH == 2) {
    // The second key part hands its (o, m, l) to the first through LDS (the
    // K staging, free since every wave passed the barrier after its scores);
    // the first merges them the way the combine merges splits.
    __shared__ float ml2[NW][2][16];
    floatx4* ob = (floatx4*)ldsK + (size_t)wave * 8 * 64;
    if (kh == 1 && live) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) ob[dt * 64 + lane] = o[dt];
      if (g == 0) { ml2[wave][0][lr] = mx; ml2[wave][1][lr] = lsum; }
    }
    __syncthreads();
    if (kh == 1 || !live) return;
    const float m1 = ml2[wave][0][lr], l1 = ml2[wave][1][lr];
    const float M = fmaxf(mx, m1);
    const float w0 = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - M);
    const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const floatx4 o1 = ob[dt * 64 + lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) o[dt][v] = o[dt][v] * w0 + o1[v] * w1;
    }
    lsum = lsum * w0 + l1 * w1;
    mx = M;
  }
  if (kv_len <= SPLIT) {
    // One split holds every key: the rows are final here and the combine
    // skips them.  o / l rounded to the O projection's 16-bit input format
    // (tiled, K = hq*D), the combine's arithmetic for one split; a lane's 4
    // consecutive columns go out in one 8-byte store.
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    uint16_t* outp = (uint16_t*)a.out;
    bool bad = false;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      uint32_t w[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        w[e] = pack_bf16_rne(o[dt][2 * e] * inv, o[dt][2 * e + 1] * inv);
        if (a.otype == T_F16) {
          const float fl = __uint_as_float(w[e] << 16), fh = __uint_as_float(w[e] & 0xffff0000u);
          bad = bad || !(fabsf(fl) <= 65504.0f) || !(fabsf(fh) <= 65504.0f);
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)fl) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)fh) << 16);
        }
      }
      *(uint2*)(outp + fm_index(tok, qh * D + dt * 16 + 4 * g, a.hq * D)) = uint2{w[0], w[1]};
    }
    if (a.otype == T_F16 && a.status) {
      const uint64_t b = __ballot(bad);
      if (b && lane == __builtin_ctzll(b)) atomicOr(a.status, STATUS_ACT_RANGE);
    }
    return;
  }
  const size_t row = ((size_t)sidx * a.B + tok) * a.hq + qh;
  float* op = a.o_part + row * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *(floatx4*)(op + dt * 16 + 4 * g) = o[dt];    // O^T: lane holds d = dt*16+4g+v of row lr
  if (g == 0) {
    a.ml_part[row * 2] = mx;
    a.ml_part[row * 2 + 1] = lsum;
  }
}

// ------------------------------------------------------------ fp32 attention
// Plain fp32 path (fp32 models): one thread per query row of the KV head.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kc,
                                                       const float* __restrict__ vc, const int* __restrict__ pt,
                                                       const int* dev_n, int B, int causal, int hq, int hkv,
                                                       float scale2, float* o_part, float* ml_part) {
  const int h = blockIdx.y, sidx = blockIdx.x;
  const int n = *dev_n;
  const int kv_len = n + B;
  const int key0 = sidx * ATTN_SPLIT;
  if (key0 >= kv_len) return;
  const int key1 = min(key0 + ATTN_SPLIT, kv_len);
  const int G = hq / hkv;
  const int r = threadIdx.x;
  if (r >= G * B) return;
  const int tok = r / G, qh = h * G + r % G;
  float qv[D], ov[D];
  for (int e = 0; e < D; ++e) { qv[e] = q[((size_t)tok * hq + qh) * D + e]; ov[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  for (int key = key0; key < key1; ++key) {
    if (causal && key > n + tok) break;
    const size_t slot = (((size_t)pt[key / PAGE] * hkv + h) * PAGE + key % PAGE) * D;
    float s = 0.f;
    for (int e = 0; e < D; ++e) s += qv[e] * kc[slot + e];
    s *= scale2;
    const float mn = fmaxf(m, s);
    const float al = m == -INFINITY ? 0.f : exp2f(m - mn);
    const float p = exp2f(s - mn);
    l = l * al + p;
    const size_t vt = ((size_t)pt[key / PAGE] * hkv + h) * PAGE * D + key % PAGE;   // V^T page
    for (int e = 0; e < D; ++e) ov[e] = ov[e] * al + p * vc[vt + (size_t)e * PAGE];
    m = mn;
  }
  const size_t row = ((size_t)sidx * B + tok) * hq + qh;
  for (int e = 0; e < D; ++e) o_part[row * D + e] = ov[e];
  ml_part[row * 2] = m;
  ml_part[row * 2 + 1] = l;
}

// ------------------------------------------------ prompt-chunk attention
// Causal attention of a prompt chunk (B > 64 rows at positions n..n+B-1) in
// one pass, no split-KV partials: work-group = (group of 4 row blocks, KV
// head), as in attn_mfma_kernel, and it walks the keys 0..n+t_last (t_last
// its last token) in stages of 64 keys (a page of K and one of V^T), staged
// by direct global->LDS loads into two buffers so that stage s+1 loads while
// stage s is multiplied.  64 KiB of LDS and at most 256 registers per wave
// let two work-groups share a CU, so one's MFMAs overlap the other's
// softmax.  Per stage and row: scores, the row's running max
// m, p = exp2(s - m) as bf16 hi + lo (16 significant bits), the running sum
// l and O^T rescaled by exp2(m_old - m) when the max grows (the split-KV
// combine's arithmetic applied stage by stage).  The normalised row goes
// straight to the O projection's input.
constexpr int PF_PAGES = 1;                            // pages per stage
constexpr int PF_KEYS = PF_PAGES * PAGE;               // 64 keys
constexpr int PF_DMAS = 4 * PF_PAGES;                  // K (or V^T) DMAs per wave and stage

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_prefill_kernel(AttnArgs a, void* out,
                                                                                           int otype, int ldo,
                                                                                           int32_t* status) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) uint8_t ldsK0[PF_PAGES * 16384];
  __shared__ __attribute__((aligned(16))) uint8_t ldsV0[PF_PAGES * 16384];
  __shared__ __attribute__((aligned(16))) uint8_t ldsK1[PF_PAGES * 16384];
  __shared__ __attribute__((aligned(16))) uint8_t ldsV1[PF_PAGES * 16384];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, g = lane >> 4;
  // work-group i serves KV head i mod hkv: the 8 XCDs take work-groups
  // round-robin, so with hkv = 8 each XCD's L2 only ever holds one head's
  // K/V pages (with hkv = 4, two XCDs share a head)
  const int h = blockIdx.x % a.hkv, wg = blockIdx.x / a.hkv;
  const int G = a.hq / a.hkv;
  const int nrb = G * a.B / 16;
  const int rbi = wg * 4 + wave;
  const bool live = rbi < nrb;                 // wave-uniform
  const int rb = live ? rbi : nrb - 1;
  const int r = rb * 16 + lr;
  const int tok = r / G, qh = h * G + r % G;
  bf16x8 qf[4];
  {
    const uint16_t* qp = a.q + ((size_t)tok * a.hq + qh) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const uint4*)(qp + 32 * ks));
  }
  // the page table (at most 128 pages: 8192 positions), lane l holding pages
  // l and 64 + l, read before the first stage
  const int pg0 = a.pt[min(lane, a.npages - 1)], pg1 = a.pt[min(64 + lane, a.npages - 1)];
  const int n = *a.dev_n;
  // keys 0..n+t_last of the work-group's last row
  const int t_last = (min(wg * 4 + 3, nrb - 1) * 16 + 15) / G;
  const int nst = (n + t_last + 1 + PF_KEYS - 1) / PF_KEYS;
  // the q fragments and the page table are in registers before the first
  // stage: inside the loop the only vector-memory operations are the stage
  // loads, waited for explicitly
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vm_wait(0));
  __builtin_amdgcn_sched_barrier(0);

  // stage s: K pages into kb, V^T pages into vb (wave w issues blocks w, w+4,
  // w+8, w+12 of each 16 KiB page; pages past the table re-read the last one,
  // their keys are masked)
  auto page_of = [&](int pi) {
    pi = min(pi, a.npages - 1);
    return pi < 64 ? __builtin_amdgcn_readlane(pg0, pi) : __builtin_amdgcn_readlane(pg1, pi - 64);
  };
  auto stage = [&](int st, uint8_t* kb, uint8_t* vb) {
#pragma unroll
    for (int p = 0; p < PF_PAGES; ++p) {
      const size_t pbase = ((size_t)page_of(st * PF_PAGES + p) * a.hkv + h) * PAGE * D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = wave + 4 * j;
        const int q = blk * 64 + lane;
        const int key = q >> 4, c = (q & 15) ^ (key & 15);
        lds_dma16(a.kc + pbase + key * D + c * 8, lds_addr(kb + (size_t)p * 16384 + blk * 1024));
      }
    }
#pragma unroll
    for (int p = 0; p < PF_PAGES; ++p) {
      const size_t pbase = ((size_t)page_of(st * PF_PAGES + p) * a.hkv + h) * PAGE * D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int blk = wave + 4 * j;
        const int q = blk * 64 + lane;
        const int d = q >> 3, c = (q & 7) ^ ((d >> 1) & 7);
        lds_dma16(a.vc + pbase + d * PAGE + c * 8, lds_addr(vb + (size_t)p * 16384 + blk * 1024));
      }
    }
  };

  float m_run = -INFINITY, lsum = 0.f;
  floatx4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int kmax = n + tok;                    // last key this row sees

  auto compute = [&](int st, const uint8_t* kb, const uint8_t* vb) {
    constexpr int NT = PF_KEYS / 16;
    const int key0 = st * PF_KEYS;
    // the K pages of the stage are in LDS once at most its V^T loads and the
    // next stage's loads are outstanding
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vm_wait(PF_DMAS + 2 * PF_DMAS));
    asm volatile("s_nop 0");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    uint32_t ph[NT / 2][4], pl[NT / 2][4];
    float alpha = 1.f;
    if (live) {
      float sv[NT][4];
#pragma unroll
      for (int kt = 0; kt < NT; ++kt) {
        const int p = kt >> 2, key = (kt & 3) * 16 + lr;
        const uint8_t* kpage = kb + (size_t)p * 16384 + (size_t)key * 256;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int c = (4 * ks + g) ^ (key & 15);
          const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const uint4*)(kpage + c * 16));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], acc, 0, 0, 0);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[kt][v] = acc[v] * a.scale2;
      }
      if (key0 + PF_KEYS - 1 > n) {            // the stage reaches into the chunk: causal mask
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (key0 + kt * 16 + 4 * g + v > kmax) sv[kt][v] = -INFINITY;
      }
      float mx = m_run;
#pragma unroll
      for (int kt = 0; kt < NT; ++kt) mx = fmaxf(mx, fmaxf(fmaxf(sv[kt][0], sv[kt][1]), fmaxf(sv[kt][2], sv[kt][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // a row that sees no key yet keeps m = -inf and subtracts 0 (no NaN);
      // its p are 0
      const float mref = mx == -INFINITY ? 0.f : mx;
      alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mref);
      m_run = mx;
      lsum *= alpha;
#pragma unroll
      for (int ks2 = 0; ks2 < NT / 2; ++ks2) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t hb[4], lb[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float pe = __builtin_amdgcn_exp2f(sv[2 * ks2 + hh][v] - mref);
            lsum += pe;
            const uint32_t u = __float_as_uint(pe);
            const float hv = __uint_as_float(u & 0xffff0000u);
            const uint32_t lu = __float_as_uint(pe - hv);
            hb[v] = u;
            lb[v] = lu + 0x7fffu + ((lu >> 16) & 1u);
          }
          ph[ks2][2 * hh] = __builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u);
          ph[ks2][2 * hh + 1] = __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u);
          pl[ks2][2 * hh] = __builtin_amdgcn_perm(lb[1], lb[0], 0x07060302u);
          pl[ks2][2 * hh + 1] = __builtin_amdgcn_perm(lb[3], lb[2], 0x07060302u);
        }
      }
    }
    // and its V^T pages once only the next stage's loads are outstanding
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vm_wait(2 * PF_DMAS));
    asm volatile("s_nop 0");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    if (!live) return;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int v = 0; v < 4; ++v) o[dt][v] *= alpha;
#pragma unroll
    for (int ks2 = 0; ks2 < NT / 2; ++ks2) {
      const bf16x8 pfh = __builtin_bit_cast(bf16x8, uint4{ph[ks2][0], ph[ks2][1], ph[ks2][2], ph[ks2][3]});
      const bf16x8 pfl = __builtin_bit_cast(bf16x8, uint4{pl[ks2][0], pl[ks2][1], pl[ks2][2], pl[ks2][3]});
      const int p = ks2 >> 1;
      const uint8_t* vpage = vb + (size_t)p * 16384;
      const int c0 = 4 * (ks2 & 1) + (g >> 1), hoff = (g & 1) * 8;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d = dt * 16 + lr, sw = (d >> 1) & 7;
        const uint2 lo = *(const uint2*)(vpage + (size_t)(d * 8 + (c0 ^ sw)) * 16 + hoff);
        const uint2 hi = *(const uint2*)(vpage + (size_t)(d * 8 + ((c0 + 2) ^ sw)) * 16 + hoff);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfh, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfl, o[dt], 0, 0, 0);
      }
    }
  };

  // stages 2i from buffer 0 and 2i+1 from buffer 1; the stage after the one
  // being multiplied loads into the other buffer (past the last stage the
  // last one again, so that every wait counts the same loads).  The barrier
  // at the top of each stage lets every wave finish with that buffer first.
  stage(0, ldsK0, ldsV0);
  for (int st = 0; st < nst; st += 2) {
    __builtin_amdgcn_s_barrier();
    stage(min(st + 1, nst - 1), ldsK1, ldsV1);
    compute(st, ldsK0, ldsV0);
    if (st + 1 >= nst) break;
    __builtin_amdgcn_s_barrier();
    stage(min(st + 2, nst - 1), ldsK0, ldsV0);
    compute(st + 1, ldsK1, ldsV1);
  }
  __builtin_amdgcn_s_waitcnt(vm_wait(0));      // the last (unused) loads land before the LDS is released
  if (!live) return;

  // normalised O of row (tok, qh): lane holds d = dt*16 + 4g + v
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  const int fmK = otype == T_F32 ? 0 : a.hq * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      store_act(out, act_index(tok, qh * D + dt * 16 + 4 * g + v, ldo, fmK), otype, o[dt][v] * inv, status);
}

// ------------------------------------------------------------ combine
// Merge the per-split partials of one query row: M = max m_s,
// o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, the sums in split order.
// Lane s holds split s's (m, l) and its weight; lane e's two output elements
// take the weights from lane s in turn.  All split loads of a lane are issued
// before any is consumed (no dependent load chain).

constexpr int COMBINE_MAX_SPLITS = 32;

// max over a full wave (every lane active), in every lane: DPP steps inside
// each row of 16 lanes, then the four row maxima
#define DFL_DPP_MAX(v, ctrl) \
  fmaxf((v), __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, true)))
__device__ __forceinline__ float wave_max_full(float v) {
  v = DFL_DPP_MAX(v, 0xB1);   // quad_perm [1,0,3,2]
  v = DFL_DPP_MAX(v, 0x4E);   // quad_perm [2,3,0,1]
  v = DFL_DPP_MAX(v, 0x141);  // row_half_mirror
  v = DFL_DPP_MAX(v, 0x140);  // row_mirror
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
#undef DFL_DPP_MAX

__global__ __launch_bounds__(64) void attn_combine_kernel(const float* __restrict__ o_part,
                                                          const float* __restrict__ ml_part, const int* dev_n,
                                                          int max_splits, int split, int B, int hq, int d, void* out,
                                                          int otype, int ldo, int32_t* status, int hkv,
                                                          int direct1) {
  // work-group L takes a row of KV head L mod hkv (the XCD whose L2 received
  // that head's partials from the attention)
  const int G = hq / hkv;
  const int hk = blockIdx.x % hkv, j = blockIdx.x / hkv;
  const int qh = hk * G + j % G, tok = j / G;
  const int row = tok * hq + qh;
  const size_t stride = (size_t)B * hq;
  const int lane = threadIdx.x;
  const int e = 2 * lane;                      // this lane's output elements e, e + 1 (d even, <= 128)
  const bool lv = e < d;
  // the (m, l) pairs of the state's split slots go out with the committed length
  float2 ml = {-INFINITY, 0.f};
  if (lane < max_splits) ml = *(const float2*)(ml_part + ((size_t)lane * stride + row) * 2);
  const int kv_len = *dev_n + B;
  const int ns = min((kv_len + split - 1) / split, max_splits);
  if (direct1 && ns == 1) return;             // the attention wrote these rows itself
  float2 o[COMBINE_MAX_SPLITS];
  const float* op = o_part + (size_t)row * d + (lv ? e : 0);
  const size_t sstride = stride * d;           // floats between two splits' rows
#pragma unroll
  for (int s = 0; s < COMBINE_MAX_SPLITS; ++s) {
    if (s < ns) o[s] = lv ? *(const float2*)op : float2{0.f, 0.f};
    op += sstride;
  }
  if (lane >= ns) ml = float2{-INFINITY, 0.f};
  const float M = wave_max_full(ml.x);
  const float w = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);
  const int wb = __builtin_bit_cast(int, w);
  float L = 0.f, acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int s = 0; s < COMBINE_MAX_SPLITS; ++s) {
    if (s < ns) {
      const float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wb, s));
      const float ls = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ml.y), s));
      L += ws * ls;
      acc0 += ws * o[s].x;
      acc1 += ws * o[s].y;
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  // 16-bit outputs feed the O projection: tiled layout with K = hq*d
  const int fmK = otype == T_F32 ? 0 : hq * d;
  if (lv) {
    store_act(out, act_index(tok, qh * d + e, ldo, fmK), otype, acc0 * inv, status);
    store_act(out, act_index(tok, qh * d + e + 1, ldo, fmK), otype, acc1 * inv, status);
  }
}

// compute units of the current device (looked up once per device)
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t launch_attention(const AttnCall& c, hipStream_t s) {
  // the combine takes one split a lane: checked before any launch
  if (c.max_splits < 1 || c.max_splits > COMBINE_MAX_SPLITS) return hipErrorInvalidValue;
  const float scale2 = LOG2E / sqrtf((float)c.d);
  dim3 grid(c.max_splits, c.hkv);
  if (c.atype == T_F32) {
    if (c.split != ATTN_SPLIT) return hipErrorInvalidValue;
    if (c.d == 64)
      hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, s, (const float*)c.q, (const float*)c.kc,
                         (const float*)c.vc, c.page_table, c.dev_n, c.block_rows, c.causal, c.hq, c.hkv, scale2,
                         c.o_part, c.ml_part);
    else
      hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, s, (const float*)c.q, (const float*)c.kc,
                         (const float*)c.vc, c.page_table, c.dev_n, c.block_rows, c.causal, c.hq, c.hkv, scale2,
                         c.o_part, c.ml_part);
  } else {
    AttnArgs a;
    a.q = (const uint16_t*)c.q; a.kc = (const uint16_t*)c.kc; a.vc = (const uint16_t*)c.vc;
    a.pt = c.page_table; a.dev_n = c.dev_n; a.B = c.block_rows; a.causal = c.causal;
    a.hq = c.hq; a.hkv = c.hkv; a.scale2 = scale2; a.o_part = c.o_part; a.ml_part = c.ml_part;
    a.npages = c.npages;
    a.out = c.out; a.otype = c.otype; a.status = c.status;
    const int nrb = (c.hq / c.hkv) * c.block_rows / 16;
    if (nrb < 1 || (c.hq / c.hkv) * c.block_rows % 16) return hipErrorInvalidValue;
    if (c.block_rows > 64 && c.causal && c.d == 128 && c.npages <= 128) {
      // a prompt chunk: one pass over the keys, normalised output, no combine
      hipLaunchKernelGGL(attn_prefill_kernel, dim3((nrb + 3) / 4 * c.hkv), dim3(256), 0, s, a, c.out, c.otype, c.ldo,
                         c.status);
      return hipGetLastError();
    }
    // One work-group fits a CU (128 KiB of LDS).  Eight row blocks share one
    // K / V^T staging only when the four-row-block grid would spill past the
    // device's CUs and the row blocks fill whole groups of eight: with fewer
    // splits, four-row-block work-groups spread the score and P.V work over
    // twice the CUs and are faster (8B shapes, block 32: 3.38 vs 3.53 ms a
    // step at ctx 64, 4.02 vs 3.88 ms at ctx 4096).  Four-row-block groups
    // over 256-key splits run two waves per row block, one per half of the
    // keys (attention + combine 10.5 -> 9.3 us a layer at ctx 64, 17.2 ->
    // 16.6 at ctx 2048); over 128-key splits the halves are too short to pay
    // for the merge (7.8 -> 8.1 us at ctx 64), and eight-row-block groups
    // keep one wave per row block too (with two, 1024 threads, 22.7 -> 24.3
    // us at ctx 4096).  The grid is sized by the state's capacity
    // (max_splits), not by the live context, so that one captured graph
    // serves every context length: a state whose capacity passes the
    // threshold runs the eight-row-block shape at every length.
    if (c.split != ATTN_SPLIT && (c.split != ATTN_SPLIT_SMALL || c.d != 128)) return hipErrorInvalidValue;
    if (c.otype == T_F32) return hipErrorInvalidValue;   // rows of one split are written as 16-bit here
    const bool small = c.split == ATTN_SPLIT_SMALL;
    if (nrb % 8 == 0 && c.max_splits * c.hkv * (nrb / 4) > device_cus()) {
      if (small)
        hipLaunchKernelGGL((attn_mfma_kernel<8, 2, 1>), dim3(c.max_splits, c.hkv, nrb / 8), dim3(512), 0, s, a);
      else
        hipLaunchKernelGGL((attn_mfma_kernel<8, 4, 1>), dim3(c.max_splits, c.hkv, nrb / 8), dim3(512), 0, s, a);
    } else {
      if (small)
        hipLaunchKernelGGL((attn_mfma_kernel<4, 2, 1>), dim3(c.max_splits, c.hkv, (nrb + 3) / 4), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((attn_mfma_kernel<4, 4, 2>), dim3(c.max_splits, c.hkv, (nrb + 3) / 4), dim3(512), 0, s, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(c.block_rows * c.hq), dim3(64), 0, s, c.o_part, c.ml_part,
                     c.dev_n, c.max_splits, c.split, c.block_rows, c.hq, c.d, c.out, c.otype, c.ldo, c.status,
                     c.hkv, c.atype != T_F32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace dfl
