// Temperature sampling in the speculative loop.
//
// The mlx-dspark v0.0.3 release notes ("Highlights") make sampling at a
// temperature T > 0 lossless with respect to the target: the output is an
// exact sample of the target at T.  The rule that does this is speculative
// sampling: slot j draws d_j from the drafter's q_j = softmax(z_j / T); the
// target's row j-1 gives p_{j-1} = softmax(y_{j-1} / T); d_j is kept while
// u_j < p_{j-1}(d_j) / q_j(d_j); at the first rejection the correction is
// drawn from max(0, p_a - q_{a+1}) renormalised, and when every verified
// draft is kept a bonus token is drawn from p_N.
//
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011), counter (n, row, stream, 0) and key
// (seed low, seed high), with n the committed length at the start of the
// step; stream 0 = draft samples, 1 = acceptance tests, 2 = correction or
// bonus, 3 = the first token after the prompt.  u = (x0 / 2^8 + 1/2) / 2^24.
//
// A categorical draw over a vocabulary row is one work-group of 1024
// threads: the row is cut into tiles of 1024 consecutive entries, the tile
// sums are formed with coalesced loads and prefixed in index order, and the
// work-group scans the tile that holds u * sum; the drawn index is the
// smallest v whose running sum exceeds u * sum.  Every sum has a fixed
// order, so a draw is bit-reproducible.
#include "common.h"

namespace dfl {

namespace {

constexpr int SAMPLE_THREADS = 1024;
constexpr float LOG2E_F = 1.4426950408889634f;

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint2 k) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = c.x * 0xD2511F53u, hi0 = __umulhi(c.x, 0xD2511F53u);
    const uint32_t lo1 = c.z * 0xCD9E8D57u, hi1 = __umulhi(c.z, 0xCD9E8D57u);
    c = make_uint4(hi1 ^ c.y ^ k.x, lo1, hi0 ^ c.w ^ k.y, lo0);
    k.x += 0x9E3779B9u;
    k.y += 0xBB67AE85u;
  }
  return c;
}

__device__ __forceinline__ float uniform01(uint64_t seed, uint32_t n, uint32_t row, uint32_t stream) {
  const uint4 o = philox4x32_10(make_uint4(n, row, stream, 0u), make_uint2((uint32_t)seed, (uint32_t)(seed >> 32)));
  return ((float)(o.x >> 8) + 0.5f) * 5.9604644775390625e-8f;     // exact: 24-bit integer + 1/2, times 2^-24
}

__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * LOG2E_F); }

// fixed-order reductions over the 1024 threads (tree in LDS)
__device__ float wg_max(float v, float* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int o = SAMPLE_THREADS / 2; o > 0; o >>= 1) {
    if (t < o) red[t] = fmaxf(red[t], red[t + o]);
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

// Smallest v in [0, vocab) whose running sum of w exceeds u * sum(w); -1 when
// sum(w) is 0.  Every thread returns the same index.  The row is cut into
// tiles of 1024 consecutive entries: the 16 waves form the tile sums with
// coalesced loads (wave w takes tiles w, w+16, ...; fixed reduction order),
// one thread turns them into exclusive prefixes, and the work-group scans
// the one tile that holds u * sum.
constexpr int CAT_TILE = SAMPLE_THREADS;
constexpr int CAT_MAX_TILES = 256;            // vocab up to 262144
template <class W>
__device__ int wg_categorical(const W& w, int vocab, float u, float* scan, float* tile, int* pick, float* total) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int ntiles = (vocab + CAT_TILE - 1) / CAT_TILE;
  for (int k = wave; k < ntiles; k += SAMPLE_THREADS / 64) {
    float s = 0.f;
#pragma unroll 4
    for (int e = 0; e < CAT_TILE / 64; ++e) {
      const int v = k * CAT_TILE + e * 64 + lane;
      if (v < vocab) s += w(v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if (lane == 0) tile[k] = s;
  }
  __syncthreads();
  if (t == 0) {
    float acc = 0.f;
    for (int k = 0; k < ntiles; ++k) {
      const float x = tile[k];
      tile[k] = acc;                           // exclusive prefix
      acc += x;
    }
    tile[ntiles] = acc;
    *total = acc;
    pick[0] = 0x7fffffff;
    pick[1] = -1;
    pick[2] = -1;
  }
  __syncthreads();
  const float S = *total;
  int r = -1;
  if (S > 0.f) {
    float target = u * S;
    if (target >= S) target = S * 0.99999994f;    // u * S rounded up to the total
    if (t < ntiles && tile[t] <= target && target < tile[t + 1]) pick[2] = t;
    __syncthreads();
    const int k = pick[2] < 0 ? ntiles - 1 : pick[2];
    const int v = k * CAT_TILE + t;
    const float x = v < vocab ? w(v) : 0.f;
    // inclusive scan of the tile, Hillis-Steele (fixed order)
    scan[t] = x;
    __syncthreads();
    for (int o = 1; o < SAMPLE_THREADS; o <<= 1) {
      const float add = t >= o ? scan[t - o] : 0.f;
      __syncthreads();
      scan[t] += add;
      __syncthreads();
    }
    if (x > 0.f) {
      if (tile[k] + scan[t] > target) atomicMin(&pick[0], v);
      atomicMax(&pick[1], v);                    // last entry of the tile with weight
    }
    __syncthreads();
    r = pick[0] != 0x7fffffff ? pick[0] : pick[1];
  }
  __syncthreads();
  return r;
}

// One work-group per row: log-normaliser lse = log sum exp(z / T) of the row
// and, when stream >= 0, a draw from softmax(z / T) with counter
// (n, row0 + r, stream), n = *dev_n + n_add (or n_add when dev_n is null).
__global__ __launch_bounds__(SAMPLE_THREADS) void sample_rows_kernel(const float* __restrict__ logits, int ld,
                                                                    int vocab, float invT, uint64_t seed,
                                                                    const int* dev_n, int n_add, int row0,
                                                                    int stream, int32_t* out_tok,
                                                                    float* out_lse) {
  __shared__ float red[SAMPLE_THREADS];
  __shared__ float tile[CAT_MAX_TILES + 1];
  __shared__ int pick[3];
  __shared__ float total;
  const int r = blockIdx.x, t = threadIdx.x;
  const float* z = logits + (size_t)r * ld;
  float m = -INFINITY;
  for (int v = t; v < vocab; v += SAMPLE_THREADS) m = fmaxf(m, z[v]);
  const float M = wg_max(m, red);
  const float scale = invT;
  auto w = [&](int v) { return exp_f((z[v] - M) * scale); };
  if (stream < 0) {
    // normaliser only: strided (coalesced) sums, then a fixed-order tree
    float sum = 0.f;
    for (int v = t; v < vocab; v += SAMPLE_THREADS) sum += w(v);
    red[t] = sum;
    __syncthreads();
    for (int o = SAMPLE_THREADS / 2; o > 0; o >>= 1) {
      if (t < o) red[t] += red[t + o];
      __syncthreads();
    }
    if (t == 0 && out_lse) out_lse[r] = M * invT + logf(red[0]);
    return;
  }
  const int n = (dev_n ? *dev_n : 0) + n_add;
  const float u = uniform01(seed, (uint32_t)n, (uint32_t)(row0 + r), (uint32_t)stream);
  const int tok = wg_categorical(w, vocab, u, red, tile, pick, &total);
  if (t == 0) {
    if (out_lse) out_lse[r] = M * invT + logf(total);
    if (out_tok) out_tok[r] = tok;
  }
}

// Acceptance over N verified drafts and the correction/bonus draw (one
// work-group).  block[0] is the anchor, block[j] = d_j; dlog row j-1 holds
// the drafter's logits of slot j, vlog row i the target's logits of row i;
// lse_q / lse_p their log-normalisers at T.  Writes acc[0] = a, emit[0..a-1]
// = d_1..d_a, emit[a] = the drawn token, emit[a+1..B-1] = -1 and the token
// to next_anchor[0] (which may alias block[0]).
__global__ __launch_bounds__(SAMPLE_THREADS) void spec_accept_kernel(
    const int32_t* block, const float* __restrict__ dlog, const float* __restrict__ vlog, int vocab, int N,
    const float* __restrict__ lse_q, const float* __restrict__ lse_p, float invT, uint64_t seed, const int* dev_n,
    int n_add, int B, int32_t* acc, int32_t* emit, int32_t* next_anchor) {
  __shared__ float scan[SAMPLE_THREADS];
  __shared__ float tile[CAT_MAX_TILES + 1];
  __shared__ int pick[3];
  __shared__ float total;
  __shared__ int s_fail;
  __shared__ int32_t drafts[64];
  const int t = threadIdx.x;
  const uint32_t n = (uint32_t)((dev_n ? *dev_n : 0) + n_add);
  if (t < B) drafts[t] = block[t];
  if (t == 0) s_fail = N + 1;
  __syncthreads();
  // thread j tests draft j (all N tests at once); a = first rejected j - 1
  if (t >= 1 && t <= N) {
    const int d = drafts[t];
    bool keep = d >= 0 && d < vocab;           // not a token: rejected (q(d) undefined)
    if (keep) {
      const float lp = vlog[(size_t)(t - 1) * vocab + d] * invT - lse_p[t - 1];
      const float lq = dlog[(size_t)(t - 1) * vocab + d] * invT - lse_q[t - 1];
      const float u = uniform01(seed, n, (uint32_t)t, 1u);
      keep = u < exp_f(lp - lq);
    }
    if (!keep) atomicMin(&s_fail, t);
  }
  __syncthreads();
  const int a = s_fail - 1;
  const float* y = vlog + (size_t)a * vocab;
  const float ly = lse_p[a];
  const float u = uniform01(seed, n, (uint32_t)a, 2u);
  auto wp = [&](int v) { return exp_f(y[v] * invT - ly); };
  int tok = -1;
  if (a < N) {
    const float* z = dlog + (size_t)a * vocab;      // slot a+1
    const float lz = lse_q[a];
    auto wr = [&](int v) { return fmaxf(exp_f(y[v] * invT - ly) - exp_f(z[v] * invT - lz), 0.f); };
    tok = wg_categorical(wr, vocab, u, scan, tile, pick, &total);
  }
  if (tok < 0) tok = wg_categorical(wp, vocab, u, scan, tile, pick, &total);
  for (int i = t; i < B; i += SAMPLE_THREADS) emit[i] = i < a ? drafts[i + 1] : (i == a ? tok : -1);
  if (t == 0) {
    acc[0] = a;
    if (next_anchor) next_anchor[0] = tok;
  }
}

}  // namespace

hipError_t launch_sample_rows(const float* logits, int ld, int vocab, int rows, float temperature, uint64_t seed,
                              const int* dev_n, int n_add, int row0, int stream, int32_t* out_tok, float* out_lse,
                              hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (!(temperature > 0.f) || vocab < 1 || vocab > CAT_TILE * CAT_MAX_TILES) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_rows_kernel, dim3(rows), dim3(SAMPLE_THREADS), 0, s, logits, ld, vocab,
                     1.0f / temperature, seed, dev_n, n_add, row0, stream, out_tok, out_lse);
  return hipGetLastError();
}

hipError_t launch_spec_accept(const int32_t* block, const float* dlog, const float* vlog, int vocab, int N,
                              const float* lse_q, const float* lse_p, float temperature, uint64_t seed,
                              const int* dev_n, int n_add, int B, int32_t* acc, int32_t* emit,
                              int32_t* next_anchor, hipStream_t s) {
  if (N < 1 || N >= B || B > 64 || vocab < 1 || vocab > CAT_TILE * CAT_MAX_TILES || !(temperature > 0.f))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(spec_accept_kernel, dim3(1), dim3(SAMPLE_THREADS), 0, s, block, dlog, vlog, vocab, N, lse_q,
                     lse_p, 1.0f / temperature, seed, dev_n, n_add, B, acc, emit, next_anchor);
  return hipGetLastError();
}

}  // namespace dfl
