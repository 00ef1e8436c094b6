// Attention pieces of the draft+verify step.
//
// qk_rope_kernel: per-head RMSNorm of q and k over head_dim (the per-head form
// mirror-sd's README, "The Story", had to fix: a norm across all channels gave
// cosine ~0.5), then neox split-half RoPE (pairs (i, i+d/2), the convention of
// mx.fast.rope(traditional=False) named there), one rounding to the
// activation format, then q goes to the query buffer and k/v to the paged KV
// cache at slot(pos) = page_table[pos/64]*64 + pos%64.
//
// attn_*_kernel: softmax(q k^T / sqrt(d)) v of the B block rows over the
// cache positions 0..n+B-1.  Verify (causal=1): row i (position n+i) sees
// keys 0..n+i -- the committed context plus the block causally.  Draft
// (causal=0): every block slot sees every committed context row and every
// block slot (the drafter denoises the block in one bidirectional pass,
// mlx-dspark v0.0.3 "Highlights").  Split-KV: each work-group takes 256 keys
// of one KV head for all G*B query rows of that head (GQA) and writes an
// unnormalised partial (o, max, sum); attn_combine merges the splits -- the
// two-pass structure of the long-context verify attention in the dflash-mlx
// note ("Technical challenges", JIT SDPA 2-pass for N >= 1024), here used at
// every length so the graph of a step is length-independent.
#include "common.h"

namespace dfl {

static constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------------ QK norm + RoPE
__global__ __launch_bounds__(64) void qk_rope_kernel(RopeCall c) {
  const int row = blockIdx.x, head = blockIdx.y, lane = threadIdx.x;
  const int n = *c.dev_n;
  const int p = c.dev_p ? *c.dev_p : 0;
  int pos;
  if (row < c.block_rows) {
    pos = n + row;
  } else {
    const int j = row - c.block_rows;
    if (j >= p || head < c.hq) return;      // context rows only carry k/v
    pos = n - p + j;
  }
  if (pos < 0 || pos >= c.capacity) return;
  const int d = c.d, half = d >> 1;
  const bool act = lane < half;
  const int i = act ? lane : 0;
  const size_t rbase = (size_t)row * c.ldqkv;
  const size_t src = rbase + (size_t)head * d;          // q heads, then k heads
  const float* gain = head < c.hq ? c.q_norm : c.k_norm;
  float x1 = act ? load_act(c.qkv, src + i, c.atype) : 0.f;
  float x2 = act ? load_act(c.qkv, src + i + half, c.atype) : 0.f;
  const float ss = wave_sum(x1 * x1 + x2 * x2);
  const float r = 1.0f / sqrtf(ss / (float)d + c.eps);
  const float a = x1 * r * gain[i];
  const float b = x2 * r * gain[i + half];
  const float cs = c.cos_t[(size_t)pos * half + i];
  const float sn = c.sin_t[(size_t)pos * half + i];
  const float o1 = a * cs - b * sn;
  const float o2 = b * cs + a * sn;
  if (!act) return;
  if (head < c.hq) {
    const size_t q = ((size_t)row * c.hq + head) * d;
    store_act(c.q_out, q + i, c.atype, o1);
    store_act(c.q_out, q + i + half, c.atype, o2);
  } else {
    const int kh = head - c.hq;
    const int page = c.page_table[pos / PAGE];
    const size_t slot = (((size_t)page * c.hkv + kh) * PAGE + (pos % PAGE)) * d;
    store_act(c.kc, slot + i, c.atype, o1);
    store_act(c.kc, slot + i + half, c.atype, o2);
    const size_t vs = rbase + (size_t)(c.hq + c.hkv + kh) * d;
    store_act(c.vc, slot + i, c.atype, load_act(c.qkv, vs + i, c.atype));
    store_act(c.vc, slot + i + half, c.atype, load_act(c.qkv, vs + i + half, c.atype));
  }
}

hipError_t launch_qk_rope(const RopeCall& c, hipStream_t s) {
  dim3 grid(c.block_rows + c.ctx_rows, c.hq + c.hkv);
  hipLaunchKernelGGL(qk_rope_kernel, grid, dim3(64), 0, s, c);
  return hipGetLastError();
}

// ------------------------------------------------------------ MFMA attention
struct AttnArgs {
  const uint16_t* q; const uint16_t* kc; const uint16_t* vc; const int* pt;
  const int* dev_n; int B; int causal; int hq, hkv; float scale2;   // scale * log2(e)
  float* o_part; float* ml_part;
};

constexpr int KS_LD = 128 + 8;   // padded LDS row of the K page (bf16)
constexpr int VT_LD = 64 + 8;    // padded LDS row of the transposed V page

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// head_dim 128, bf16 q/k/v.  Work-group = (split of 256 keys, KV head, group
// of 4 query row blocks); wave w handles row block 4*group + w (16 rows,
// row r = token r/G, query head h*G + r%G).  S^T = K Q^T so that a lane holds
// 4 keys of one query row; P^T then feeds O^T = V^T P^T directly as the B
// operand.  The next page's K/V are fetched into registers while the current
// page is multiplied.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma_kernel(AttnArgs a) {
  constexpr int D = 128;
  __shared__ uint16_t Ks[PAGE * KS_LD];
  __shared__ uint16_t Vt[D * VT_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, g = lane >> 4;
  const int h = blockIdx.y, sidx = blockIdx.x;
  const int n = *a.dev_n;
  const int kv_len = n + a.B;
  const int key0 = sidx * ATTN_SPLIT;
  if (key0 >= kv_len) return;
  const int key1 = min(key0 + ATTN_SPLIT, kv_len);
  const int G = a.hq / a.hkv;
  const int nrb = G * a.B / 16;
  const int rbi = blockIdx.z * 4 + wave;
  const bool live = rbi < nrb;           // wave-uniform
  const int rbc = live ? rbi : nrb - 1;  // dead waves mirror a live block (results dropped)

  bf16x8 qf[4];
  floatx4 o[8];
  float mrow = -INFINITY, lrow = 0.f;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  {
    const int r = rbc * 16 + lr;
    const int tok = r / G, qh = h * G + r % G;
    const uint16_t* qp = a.q + ((size_t)tok * a.hq + qh) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, *(const uint4*)(qp + 32 * ks));
  }
  const int tok = (rbc * 16 + lr) / G;

  const int pg0 = key0 / PAGE, pg1 = (key1 + PAGE - 1) / PAGE;
  // K/V of one page: 1024 chunks of 8 bf16 each, 4 per thread
  // named registers, not arrays: an array indexed inside the page loop is
  // left in private memory by the compiler
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
  const int fkey = tid >> 4, fdc = (tid & 15) * 8;   // chunk j: key fkey + 16 j
#define DFL_FETCH_PAGE(PG)                                                  \
  {                                                                         \
    const int page_ = a.pt[(PG)];                                           \
    const uint16_t* kp_ = a.kc + ((size_t)page_ * a.hkv + h) * PAGE * D + fkey * D + fdc; \
    const uint16_t* vp_ = a.vc + ((size_t)page_ * a.hkv + h) * PAGE * D + fkey * D + fdc; \
    k0 = *(const uint4*)(kp_);          v0 = *(const uint4*)(vp_);          \
    k1 = *(const uint4*)(kp_ + 16 * D); v1 = *(const uint4*)(vp_ + 16 * D); \
    k2 = *(const uint4*)(kp_ + 32 * D); v2 = *(const uint4*)(vp_ + 32 * D); \
    k3 = *(const uint4*)(kp_ + 48 * D); v3 = *(const uint4*)(vp_ + 48 * D); \
  }
#define DFL_STAGE(J, KR, VR)                                                \
  {                                                                         \
    const int key_ = fkey + 16 * (J);                                       \
    *(uint4*)(Ks + key_ * KS_LD + fdc) = (KR);                              \
    uint16_t* vt_ = Vt + fdc * VT_LD + key_;                                \
    vt_[0 * VT_LD] = (uint16_t)(VR).x; vt_[1 * VT_LD] = (uint16_t)((VR).x >> 16); \
    vt_[2 * VT_LD] = (uint16_t)(VR).y; vt_[3 * VT_LD] = (uint16_t)((VR).y >> 16); \
    vt_[4 * VT_LD] = (uint16_t)(VR).z; vt_[5 * VT_LD] = (uint16_t)((VR).z >> 16); \
    vt_[6 * VT_LD] = (uint16_t)(VR).w; vt_[7 * VT_LD] = (uint16_t)((VR).w >> 16); \
  }
  DFL_FETCH_PAGE(pg0)
  for (int pg = pg0; pg < pg1; ++pg) {
    __syncthreads();                             // previous page fully consumed
    DFL_STAGE(0, k0, v0)
    DFL_STAGE(1, k1, v1)
    DFL_STAGE(2, k2, v2)
    DFL_STAGE(3, k3, v3)
    __syncthreads();
    // next page (the last iteration re-reads its own page: unconditional
    // loads keep the registers out of memory) in flight during the MFMAs
    DFL_FETCH_PAGE(pg + 1 < pg1 ? pg + 1 : pg)

    float sv[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const uint4*)(Ks + (kt * 16 + lr) * KS_LD + 32 * ks + 8 * g));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], acc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kpos = pg * PAGE + kt * 16 + 4 * g + v;
        const bool vis = kpos < kv_len && (!a.causal || kpos <= n + tok);
        sv[kt][v] = vis ? acc[v] * a.scale2 : -INFINITY;
        mx = fmaxf(mx, sv[kt][v]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // No per-row branching below: the MFMAs are wave-wide, so a row whose
    // keys are all masked so far (dead) runs them too, with p = 0, alpha = 1.
    const float mnew = fmaxf(mrow, mx);
    const bool dead = mnew == -INFINITY;
    const float alpha = dead ? 1.f : (mrow == -INFINITY ? 0.f : exp2f(mrow - mnew));
    mrow = mnew;
    // softmax weights stay fp32: each p is fed to the MFMA as p_hi + p_lo,
    // two bf16 values whose sum carries 16 significant bits
    float psum = 0.f;
    uint32_t ph[4][2], pl[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float hv[4], lv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float pe = (dead || sv[kt][v] == -INFINITY) ? 0.f : exp2f(sv[kt][v] - mnew);
        hv[v] = round_bf16(pe);
        lv[v] = round_bf16(pe - hv[v]);
        psum += pe;
      }
      ph[kt][0] = bf16_pair(hv[0], hv[1]);
      ph[kt][1] = bf16_pair(hv[2], hv[3]);
      pl[kt][0] = bf16_pair(lv[0], lv[1]);
      pl[kt][1] = bf16_pair(lv[2], lv[3]);
    }
    lrow = lrow * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      // B operand: key slots e = hh*4+v <-> key (2*ks2+hh)*16 + 4g + v
      const bf16x8 pfh = __builtin_bit_cast(bf16x8, uint4{ph[2 * ks2][0], ph[2 * ks2][1], ph[2 * ks2 + 1][0], ph[2 * ks2 + 1][1]});
      const bf16x8 pfl = __builtin_bit_cast(bf16x8, uint4{pl[2 * ks2][0], pl[2 * ks2][1], pl[2 * ks2 + 1][0], pl[2 * ks2 + 1][1]});
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const uint16_t* vrow = Vt + (dt * 16 + lr) * VT_LD + (2 * ks2) * 16 + 4 * g;
        const uint2 lo = *(const uint2*)vrow;
        const uint2 hi = *(const uint2*)(vrow + 16);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfh, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pfl, o[dt], 0, 0, 0);
      }
    }
  }

#undef DFL_FETCH_PAGE
#undef DFL_STAGE
  // partials: o (unnormalised), m (log2 domain) and l per query row
  if (!live) return;
  float l = lrow;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  const int r = rbi * 16 + lr;
  const int qh = h * G + r % G;
  const size_t row = ((size_t)sidx * a.B + tok) * a.hq + qh;
  float* op = a.o_part + row * D;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *(floatx4*)(op + dt * 16 + 4 * g) = o[dt];    // O^T: lane holds d = dt*16+4g+v of row lr
  if (g == 0) {
    a.ml_part[row * 2] = mrow;
    a.ml_part[row * 2 + 1] = l;
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
    for (int e = 0; e < D; ++e) ov[e] = ov[e] * al + p * vc[slot + e];
    m = mn;
  }
  const size_t row = ((size_t)sidx * B + tok) * hq + qh;
  for (int e = 0; e < D; ++e) o_part[row * D + e] = ov[e];
  ml_part[row * 2] = m;
  ml_part[row * 2 + 1] = l;
}

// ------------------------------------------------------------ combine
// Merge the per-split partials of one query row: M = max m_s,
// o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.  All split loads of a
// thread are issued before any is consumed (no dependent load chain).
constexpr int COMBINE_MAX_SPLITS = 32;

__global__ __launch_bounds__(64) void attn_combine_kernel(const float* __restrict__ o_part,
                                                          const float* __restrict__ ml_part, const int* dev_n,
                                                          int B, int hq, int d, void* out, int otype, int ldo) {
  const int row = blockIdx.x;          // token * hq + qh
  const int tok = row / hq, qh = row % hq;
  const int kv_len = *dev_n + B;
  const int ns = min((kv_len + ATTN_SPLIT - 1) / ATTN_SPLIT, COMBINE_MAX_SPLITS);
  const size_t stride = (size_t)B * hq;
  const int e0 = threadIdx.x, e1 = threadIdx.x + 64;
  float ms[COMBINE_MAX_SPLITS], ls[COMBINE_MAX_SPLITS], o0[COMBINE_MAX_SPLITS], o1[COMBINE_MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < COMBINE_MAX_SPLITS; ++s) {
    if (s < ns) {
      const size_t r = s * stride + row;
      ms[s] = ml_part[r * 2];
      ls[s] = ml_part[r * 2 + 1];
      o0[s] = e0 < d ? o_part[r * d + e0] : 0.f;
      o1[s] = e1 < d ? o_part[r * d + e1] : 0.f;
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < COMBINE_MAX_SPLITS; ++s)
    if (s < ns) M = fmaxf(M, ms[s]);
  float L = 0.f, acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int s = 0; s < COMBINE_MAX_SPLITS; ++s) {
    if (s < ns && ms[s] != -INFINITY) {
      const float w = exp2f(ms[s] - M);
      L += w * ls[s];
      acc0 += w * o0[s];
      acc1 += w * o1[s];
    }
  }
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  // 16-bit outputs feed the O projection: tiled layout with K = hq*d
  const int fmK = otype == T_F32 ? 0 : hq * d;
  if (e0 < d) store_act(out, act_index(tok, qh * d + e0, ldo, fmK), otype, acc0 * inv);
  if (e1 < d) store_act(out, act_index(tok, qh * d + e1, ldo, fmK), otype, acc1 * inv);
}

hipError_t launch_attention(const AttnCall& c, hipStream_t s) {
  const float scale2 = LOG2E / sqrtf((float)c.d);
  dim3 grid(c.max_splits, c.hkv);
  if (c.atype == T_F32) {
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
    const int nrb = (c.hq / c.hkv) * c.block_rows / 16;
    dim3 g3(c.max_splits, c.hkv, (nrb + 3) / 4);
    hipLaunchKernelGGL(attn_mfma_kernel, g3, dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(c.block_rows * c.hq), dim3(64), 0, s, c.o_part, c.ml_part,
                     c.dev_n, c.block_rows, c.hq, c.d, c.out, c.otype, c.ldo);
  return hipGetLastError();
}

}  // namespace dfl
