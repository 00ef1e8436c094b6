// GatedDeltaNet layers of the hybrid target: verify recurrence + tape, and
// the tape replay that commits the accepted tokens.
//
// The dflash-mlx note ("Technical challenges") and the agentlens summary of
// bstnxbt/dflash-mlx ("How it works") roll GatedDeltaNet state back by
// replaying a tape recorded during verify instead of snapshotting it.  Per
// head, with state S [dv][dk] (fp32):
//   r = v - alpha * (S k);  u = beta * r;  S <- alpha * S + u k^T;  o = S q
// q, k L2-normalised (q also scaled by 1/sqrt(dk)); alpha = sigmoid(-a) (the
// same as exp(-softplus(a))), beta = sigmoid(b).
//
// Both kernels apply a token in the SAME pinned fp32 order, so the committed
// state is bit-reproducible (and equals a from-scratch recompute over the
// recorded tape):
//   acc = halving-tree sum over j of (S[i][j] * k[j])   (each product rounded)
//   p = alpha*acc; r = v[i] - p; u = beta*r; S[i][j] = (alpha*S[i][j]) + (u*k[j])
// Thread layout: 4 consecutive lanes own value row i; lane r holds columns
// j = r + 4m (m < dk/4).  The halving tree's strides dk/2 .. 4 stay inside a
// lane; strides 2 and 1 are the xor-2 / xor-1 lane exchanges.
// This file is compiled with -ffp-contract=off: no multiply-add fusion, except
// in the verify's chunk-form outputs (steps 3-5 of verify_block), which feed
// no state.
#include "common.h"

#pragma clang fp contract(off)

namespace dfl {

// Column j = r + 4m of a k (or q) row sits at kv[r + 4m] in the tape's
// layout, or at kv[r * (dk/4 + 4) + m] in the lane-major LDS layout of the
// verify (each lane's columns contiguous, the 4 lanes' runs 4 banks apart);
// both give the same values, so the same results.
template <int DK>
constexpr int KRUN = DK / 4 + 4;

// x of lane l ^ X (X = 1 or 2) within each quad of lanes, by a DPP quad
// permutation (the 4 lanes of a row are a quad)
template <int X>
__device__ __forceinline__ float quad_xor(float x) {
  constexpr int sel = X == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), sel, 0xF, 0xF, true));
}
// x of the lane R places further round its DPP row of 16 lanes
template <int R>
__device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + R, 0xF, 0xF, true));
}
// the sum over each row of 16 lanes, in every lane of the row
__device__ __forceinline__ float row16_sum(float x) {
  x = x + quad_xor<1>(x);
  x = x + quad_xor<2>(x);
  x = x + row_ror<4>(x);
  x = x + row_ror<8>(x);
  return x;
}
template <int DK, bool LANE_MAJOR>
__device__ __forceinline__ int kcol(int r, int m) { return LANE_MAJOR ? r * KRUN<DK> + m : r + 4 * m; }

template <int DK, bool LANE_MAJOR = false>
__device__ __forceinline__ float tree_dot(const float (&S)[DK / 4], const float* kv_lds, int r) {
  float p[DK / 4];
#pragma unroll
  for (int m = 0; m < DK / 4; ++m) p[m] = S[m] * kv_lds[kcol<DK, LANE_MAJOR>(r, m)];
#pragma unroll
  for (int w = DK / 8; w >= 1; w >>= 1)
#pragma unroll
    for (int m = 0; m < w; ++m) p[m] = p[m] + p[m + w];
  float x = p[0];
  x = x + quad_xor<2>(x);
  x = x + quad_xor<1>(x);
  return x;
}

template <int DK, bool LANE_MAJOR = false>
__device__ __forceinline__ void apply_token(float (&S)[DK / 4], const float* k_lds, float v_i, float alpha,
                                            float beta, int r) {
  const float acc = tree_dot<DK, LANE_MAJOR>(S, k_lds, r);
  const float p = alpha * acc;
  const float rr = v_i - p;
  const float u = beta * rr;
#pragma unroll
  for (int m = 0; m < DK / 4; ++m) {
    const float a = alpha * S[m];
    const float b = u * k_lds[kcol<DK, LANE_MAJOR>(r, m)];
    S[m] = a + b;
  }
}

// Verify: the T = rows tokens of a block in the chunk (UT / WY) form of the
// rule.  With gamma_t = alpha_1..alpha_t (kept as log gamma, cumulative sums
// of log alpha = -softplus(a)), per head:
//   KS = K S0^T, QS = Q S0^T            (one pass over the committed state)
//   A[s][r] = beta_s gamma_s/gamma_r k_s.k_r (r < s),
//   (I + A) U = diag(beta)(V - diag(gamma) KS)   (forward substitution)
//   O = diag(gamma) QS + (M o Q K^T) U,  M[t][s] = gamma_t/gamma_s (s <= t).
// The committed state is only read; the tape records (k_hat, v, alpha, beta)
// per token for the commit's pinned replay.  dv / GDN_RW work-groups of 4*dv
// threads per head, each for GDN_RW value rows; in the state's register
// layout thread (i, r) holds value row i, key columns r + 4m.
constexpr int GDN_MAXT = 32;
// Value rows per work-group: a head's dv rows go to dv / GDN_RW work-groups
// (rows are independent in the rule), so the per-row work (K S0^T, Q S0^T,
// O, the replay), which is VALU-bound, spreads over more CUs; every
// work-group of a head repeats the per-token and T x T work.  Eight rows
// (16 work-groups a head: 256 for 16 heads of dv = 128) against 32: hybrid
// step 3.265 -> 3.218 ms, its 2048-token prompt pass 85.7 -> 81.0 ms.
template <int DV>
constexpr int GDN_RW = DV < 8 ? DV : 8;

template <int DK, int DV>
struct GdnSmem {
  // per token: k_hat at [0, KB) and q_hat at [KB, 2 KB) (lane-major), v at
  // [VO, VO + DV), alpha at AO, beta at BO
  // (rows padded to 16 bytes, so that a lane's k or q run is read 16 bytes
  // at a time)
  static constexpr int KB = 4 * KRUN<DK>, VO = 2 * KB, AO = VO + DV, BO = AO + 1, ROW = (BO + 1 + 3) / 4 * 4;
  float kq[GDN_MAXT][ROW] __attribute__((aligned(16)));
  // the work-group's GDN_RW rows of the state S0, lane-major like k and q
  float Sl[GDN_RW<DV>][4 * KRUN<DK>] __attribute__((aligned(16)));
  float lga[GDN_MAXT];                   // log alpha, then log gamma
  float ga[GDN_MAXT];                    // gamma = exp(log gamma)
  float KS[GDN_MAXT][DV + 1], QS[GDN_MAXT][DV + 1], U[GDN_MAXT][DV + 1];
  float Am[GDN_MAXT][GDN_MAXT + 1], Mq[GDN_MAXT][GDN_MAXT + 1];
};


// The projections of the T tokens at rows row0.. of a block (materialised in
// the activation format later, at the LDS store): thread e takes column e of
// the head's k, q, v, a, b (NCOL <= threads) for every token, raw[t] for
// token t, so its address is one base plus t rows and every load of the
// block goes out before any is used.  The K splits are added in their fixed
// order.
template <int DK, int DV, int TM>
__device__ __forceinline__ void gdn_load_block(const GdnCall& c, int row0, int T, float (&raw)[TM]) {
  constexpr int NT = 4 * DV, NCOL = 2 * DK + DV + 2;
  static_assert(NCOL <= NT, "one projection column per thread");
  const int h = blockIdx.x, e = threadIdx.x, gh = c.gh;
  const size_t qo = (size_t)h * DK, ko = (size_t)gh * DK + (size_t)h * DK;
  const size_t vo = (size_t)2 * gh * DK + (size_t)h * DV;
  const size_t ao = (size_t)2 * gh * DK + (size_t)gh * DV + h, bo = ao + gh;
  const bool live = e < NCOL;
  const size_t col = e < DK ? ko + e : e < 2 * DK ? qo + (e - DK) : e < 2 * DK + DV ? vo + (e - 2 * DK)
                                                                                   : (e == 2 * DK + DV ? ao : bo);
  const float* p = c.proj.p + (size_t)row0 * c.proj.ld + (live ? col : 0);
  // unconditional loads (rows past the block re-read its last row, idle
  // threads column 0), zeroed after: no branch between the loads
#pragma unroll
  for (int t = 0; t < TM; ++t) raw[t] = p[(size_t)min(t, T - 1) * c.proj.ld];
  for (int sp = 1; sp < c.proj.S; ++sp) {
    const float* ps = p + (size_t)sp * c.proj.stride;
#pragma unroll
    for (int t = 0; t < TM; ++t) raw[t] = raw[t] + ps[(size_t)min(t, T - 1) * c.proj.ld];
  }
#pragma unroll
  for (int t = 0; t < TM; ++t) raw[t] = live && t < T ? raw[t] : 0.f;
}

// The block of T tokens at projection / output rows row0..row0+T-1 against
// the work-group's rows i0..i0+GDN_RW-1 of the state S0 in sm.Sl (i0 =
// blockIdx.y GDN_RW; written by the caller before the call).  raw holds the block's
// projections (gdn_load_block); once they are in LDS, the loads of the
// block at next_row0 (if >= 0, next_T tokens) go into raw, in flight during
// the rest.  Writes the block's outputs of the work-group's rows and, if
// tape, its tape records.  Leaves the block's k_hat, v, alpha, beta in sm.kq
// for a replay.  (TM: the most tokens a call passes, T <= TM <= GDN_MAXT)
template <int DK, int DV, int TM>
__device__ __forceinline__ void verify_block(const GdnCall& c, int row0, int T, float* tape_base,
                                             GdnSmem<DK, DV>& sm,
                                             float (&raw)[TM],
                                             int next_row0, int next_T) {
  constexpr int NT = 4 * DV;
  constexpr int RW = GDN_RW<DV>;
  constexpr int REC = DK + DV + 2;
  constexpr int KB = GdnSmem<DK, DV>::KB, VO = GdnSmem<DK, DV>::VO, AO = GdnSmem<DK, DV>::AO,
                BO = GdnSmem<DK, DV>::BO;
  const int h = blockIdx.x, i0 = blockIdx.y * RW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = tid & 3;
  const int gh = c.gh;

  // 1a. the block's projections, materialised in the activation format:
  //     row t of kq takes k, q (lane-major), v, a, b; thread e holds column e
  constexpr int NCOL = 2 * DK + DV + 2;
  if (tid < NCOL) {
    const int e = tid;
    const int pos = e < DK ? kcol<DK, true>(e & 3, e >> 2)
                           : e < 2 * DK ? KB + kcol<DK, true>((e - DK) & 3, (e - DK) >> 2) : VO + (e - 2 * DK);
#pragma unroll
    for (int t = 0; t < TM; ++t)
      if (t < T) sm.kq[t][pos] = act_round(c.atype, raw[t]);
  }
  if (next_row0 >= 0) gdn_load_block<DK, DV, TM>(c, next_row0, next_T, raw);
  __syncthreads();
  // 1b. per token, 16 lanes per token (4 tokens per wave): L2 norms (sums
  //     over the 16 lanes by DPP), gates, tape
  for (int t0 = 0; t0 < T; t0 += 4 * (NT / 64)) {
    const int t = t0 + 4 * wave + (lane >> 4), l16 = lane & 15;
    const bool tok = t < T;
    float qs = 0.f, ks = 0.f;
    if (tok)
      for (int e = l16; e < DK; e += 16) {
        const int pe = kcol<DK, true>(e & 3, e >> 2);
        const float qv = sm.kq[t][KB + pe];
        const float kv = sm.kq[t][pe];
        qs += qv * qv;
        ks += kv * kv;
      }
    qs = row16_sum(qs);                        // every lane takes part in the exchanges
    ks = row16_sum(ks);
    if (!tok) continue;
    const float qn = 1.0f / sqrtf(qs + 1e-6f) * (1.0f / sqrtf((float)DK));
    const float kn = 1.0f / sqrtf(ks + 1e-6f);
    float* tape = tape_base ? tape_base + ((size_t)t * gh + h) * REC : nullptr;
    for (int e = l16; e < DK; e += 16) {
      const int pe = kcol<DK, true>(e & 3, e >> 2);
      const float kh = sm.kq[t][pe] * kn;
      sm.kq[t][pe] = kh;
      sm.kq[t][KB + pe] = sm.kq[t][KB + pe] * qn;
      if (tape) tape[e] = kh;
    }
    if (tape)
      for (int e = l16; e < DV; e += 16) tape[DK + e] = sm.kq[t][VO + e];
    if (l16 == 0) {
      const float av = sm.kq[t][AO];
      const float bv = sm.kq[t][BO];
      const float alpha = 1.0f / (1.0f + expf(av));
      const float beta = 1.0f / (1.0f + expf(-bv));
      sm.kq[t][AO] = alpha;
      sm.kq[t][BO] = beta;
      if (tape) {
        tape[DK + DV] = alpha;
        tape[DK + DV + 1] = beta;
      }
      sm.lga[t] = -(fmaxf(av, 0.f) + log1pf(expf(-fabsf(av))));   // log alpha = -softplus(a)
    }
  }
  __syncthreads();
  if (tid == 0)
    for (int t = 1; t < T; ++t) sm.lga[t] = sm.lga[t - 1] + sm.lga[t];   // log gamma_t
  // 2. KS, QS: row i of S0 against every k_hat_t, q_hat_t (4 lanes per row,
  //    halving-tree partial dots over the lane's columns, then the xor-2 /
  //    xor-1 exchanges)
  //    every thread group of 4 GDN_RW threads takes every G-th token
  {
    constexpr int G = NT / (4 * RW);
    const int lt = tid % (4 * RW), il = lt >> 2;
    float Sr[DK / 4];
#pragma unroll
    for (int m = 0; m < DK / 4; ++m) Sr[m] = sm.Sl[il][kcol<DK, true>(r, m)];
    for (int t = tid / (4 * RW); t < T; t += G) {
      const float dk_ = tree_dot<DK, true>(Sr, &sm.kq[t][0], r);
      const float dq_ = tree_dot<DK, true>(Sr, &sm.kq[t][KB], r);
      if (r == 0) { sm.KS[t][i0 + il] = dk_; sm.QS[t][i0 + il] = dq_; }
    }
  }
  __syncthreads();
  {
  // Steps 3-5 feed only the block's outputs O (the tape and the state are
  // set above and by the pinned replay), so their products and sums may fuse
  // into multiply-adds: the forward substitution's dependent chain halves.
#pragma clang fp contract(fast)
  // 3. A and M o QK^T (T x T each); gamma_t once per token
  if (tid < T) sm.ga[tid] = expf(sm.lga[tid]);
  for (int e = tid; e < 2 * T * T; e += NT) {
    const int which = e / (T * T), t = (e / T) % T, s2 = e % T;
    float v = 0.f;
    if (which == 0 ? s2 < t : s2 <= t) {
      const float* x = which == 0 ? &sm.kq[t][0] : &sm.kq[t][KB];
      float d = 0.f;
#pragma unroll 1
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll 8
        for (int m = 0; m < DK / 4; ++m) d = d + x[rr * KRUN<DK> + m] * sm.kq[s2][rr * KRUN<DK> + m];
      const float ratio = expf(sm.lga[t] - sm.lga[s2]);
      v = which == 0 ? sm.kq[t][BO] * ratio * d : ratio * d;
    }
    if (which == 0) sm.Am[t][s2] = v; else sm.Mq[t][s2] = v;
  }
  __syncthreads();
  // 4. U by forward substitution, one thread per value column of the
  //    work-group's rows (the column's U values also kept in registers for
  //    the chain)
  if (tid < RW) {
    const int col = i0 + tid;
    float uu[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < T) {
        const float beta = sm.kq[t][BO];
        float u = beta * (sm.kq[t][VO + col] - sm.ga[t] * sm.KS[t][col]);
#pragma unroll
        for (int s2 = 0; s2 < t; ++s2) u = u - sm.Am[t][s2] * uu[s2];
        uu[t] = u;
        sm.U[t][col] = u;
      }
    }
  }
  __syncthreads();
  // 5. O = diag(gamma) QS + (M o QK^T) U over the work-group's rows; every
  //    thread takes (token, row) pairs
  for (int e = tid; e < T * RW; e += NT) {
    const int t = e / RW, il = i0 + e % RW;
    float o = sm.ga[t] * sm.QS[t][il];
    for (int s2 = 0; s2 <= t; ++s2) o = o + sm.Mq[t][s2] * sm.U[s2][il];
    store_act(c.out, act_index(row0 + t, h * DV + il, c.ldo, c.otype == T_F32 ? 0 : c.gh * DV), c.otype, o,
              c.status);
  }
  }
}

template <int DK, int DV, int TM>
__global__ __launch_bounds__(4 * DV) void gdn_verify_kernel(GdnCall c) {
  __shared__ GdnSmem<DK, DV> sm;
  const int h = blockIdx.x, tid = threadIdx.x, r = tid & 3;
  const int i = blockIdx.y * GDN_RW<DV> + (tid >> 2);
  // the block's projections go out first and the state rows after them, so
  // both are in flight together (the state's LDS stores wait for its loads)
  // TM: the most tokens of the instance (16 for 16-token blocks: no loads of
  // rows past the block)
  float raw[TM];
  gdn_load_block<DK, DV, TM>(c, 0, c.rows, raw);
  if (tid < 4 * GDN_RW<DV>) {
    const float* Sg = c.S + ((size_t)h * DV + i) * DK;
#pragma unroll
    for (int m = 0; m < DK / 4; ++m) sm.Sl[tid >> 2][kcol<DK, true>(r, m)] = Sg[r + 4 * m];
  }
  // (verify_block's first barrier orders these stores before their reads);
  // the head's first work-group records the tape
  verify_block<DK, DV, TM>(c, 0, c.rows, blockIdx.y == 0 ? c.tape : nullptr, sm, raw, -1, 0);
}

// A prompt chunk of nblk blocks of B tokens, all committed: per block the
// verify above from the state in registers, then the commit's pinned replay
// of the block's B tokens into that state (the tape records are the block's
// sm.kq rows, bit for bit), so outputs and state are the ones separate verify
// and replay launches per block give.  The state is written back at the end.
template <int DK, int DV, int TM>
__global__ __launch_bounds__(4 * DV) void gdn_prompt_kernel(GdnCall c, int nblk, int B) {
  __shared__ GdnSmem<DK, DV> sm;
  const int h = blockIdx.x, tid = threadIdx.x, r = tid & 3;
  const int i = blockIdx.y * GDN_RW<DV> + (tid >> 2);
  const bool owner = tid < 4 * GDN_RW<DV>;
  float* Sg = const_cast<float*>(c.S) + ((size_t)h * DV + i) * DK;
  float S[DK / 4];
  if (owner)
#pragma unroll
    for (int m = 0; m < DK / 4; ++m) S[m] = Sg[r + 4 * m];
  // block j + 1's projections load while block j is worked on
  float raw[TM];
  gdn_load_block<DK, DV, TM>(c, 0, B, raw);
  for (int j = 0; j < nblk; ++j) {
    if (owner)
#pragma unroll
      for (int m = 0; m < DK / 4; ++m) sm.Sl[tid >> 2][kcol<DK, true>(r, m)] = S[m];
    verify_block<DK, DV, TM>(c, j * B, B, nullptr, sm, raw, j + 1 < nblk ? (j + 1) * B : -1, B);
    __syncthreads();
    if (owner)
      for (int t = 0; t < B; ++t)
        apply_token<DK, true>(S, &sm.kq[t][0], sm.kq[t][GdnSmem<DK, DV>::VO + i], sm.kq[t][GdnSmem<DK, DV>::AO],
                              sm.kq[t][GdnSmem<DK, DV>::BO], r);
    __syncthreads();                            // the next block overwrites sm
  }
  if (owner)
#pragma unroll
    for (int m = 0; m < DK / 4; ++m) Sg[r + 4 * m] = S[m];
}

hipError_t launch_gdn_verify(const GdnCall& c, hipStream_t s) {
  if (c.rows < 1 || c.rows > 32) return hipErrorInvalidValue;    // one chunk of at most 32 tokens
  const bool t16 = c.rows <= 16;
  if (c.dk == 128 && c.dv == 128) {
    const dim3 grid(c.gh, 128 / GDN_RW<128>);
    if (t16) hipLaunchKernelGGL((gdn_verify_kernel<128, 128, 16>), grid, dim3(512), 0, s, c);
    else hipLaunchKernelGGL((gdn_verify_kernel<128, 128, GDN_MAXT>), grid, dim3(512), 0, s, c);
  } else if (c.dk == 32 && c.dv == 32) {
    const dim3 grid(c.gh, 32 / GDN_RW<32>);
    if (t16) hipLaunchKernelGGL((gdn_verify_kernel<32, 32, 16>), grid, dim3(128), 0, s, c);
    else hipLaunchKernelGGL((gdn_verify_kernel<32, 32, GDN_MAXT>), grid, dim3(128), 0, s, c);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gdn_prompt(const GdnCall& c, int B, hipStream_t s) {
  if (B < 1 || B > GDN_MAXT || c.rows < B || c.rows % B) return hipErrorInvalidValue;
  const int nblk = c.rows / B;
  if (c.dk == 128 && c.dv == 128) {
    const dim3 grid(c.gh, 128 / GDN_RW<128>);
    if (B <= 16) hipLaunchKernelGGL((gdn_prompt_kernel<128, 128, 16>), grid, dim3(512), 0, s, c, nblk, B);
    else hipLaunchKernelGGL((gdn_prompt_kernel<128, 128, GDN_MAXT>), grid, dim3(512), 0, s, c, nblk, B);
  } else if (c.dk == 32 && c.dv == 32) {
    const dim3 grid(c.gh, 32 / GDN_RW<32>);
    if (B <= 16) hipLaunchKernelGGL((gdn_prompt_kernel<32, 32, 16>), grid, dim3(128), 0, s, c, nblk, B);
    else hipLaunchKernelGGL((gdn_prompt_kernel<32, 32, GDN_MAXT>), grid, dim3(128), 0, s, c, nblk, B);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Commit: every (layer, head) replays the first cnt tape records into its
// committed state, in place.
template <int DK, int DV>
__global__ __launch_bounds__(4 * DV) void gdn_replay_kernel(float* S_all, const float* tape_all, int B, int gh,
                                                            const int32_t* d_acc, int host_count,
                                                            const int32_t* scal, int capacity) {
  constexpr int REC = DK + DV + 2;
  constexpr int NT = 4 * DV;
  constexpr int PERT = (GDN_MAXT * REC + NT - 1) / NT;
  __shared__ float recs[GDN_MAXT][REC];
  const int cnt = d_acc ? d_acc[0] + 1 : host_count;
  if (scal[SC_N] + cnt + B > capacity) return;      // the commit will be refused
  if (cnt > GDN_MAXT) return;                       // (B <= GDN_MAXT: not reached)
  const int h = blockIdx.x, l = blockIdx.y;
  const int tid = threadIdx.x, i = tid >> 2, r = tid & 3;
  float* Sg = S_all + (((size_t)l * gh + h) * DV + i) * DK;
  const float* tape = tape_all + (size_t)l * B * gh * REC;
  // every committed token's record in one round of loads, issued together
  // with the state row's, then into LDS: the token loop below reads no
  // global memory
  float v[PERT];
#pragma unroll
  for (int u = 0; u < PERT; ++u) {
    const int e = tid + u * NT;
    v[u] = e < cnt * REC ? tape[((size_t)(e / REC) * gh + h) * REC + e % REC] : 0.f;
  }
  float S[DK / 4];
#pragma unroll
  for (int m = 0; m < DK / 4; ++m) S[m] = Sg[r + 4 * m];
#pragma unroll
  for (int u = 0; u < PERT; ++u) {
    const int e = tid + u * NT;
    if (e < cnt * REC) recs[e / REC][e % REC] = v[u];
  }
  __syncthreads();
  for (int t = 0; t < cnt; ++t) {
    const float* rec = recs[t];
    apply_token<DK>(S, rec, rec[DK + i], rec[DK + DV], rec[DK + DV + 1], r);
  }
#pragma unroll
  for (int m = 0; m < DK / 4; ++m) Sg[r + 4 * m] = S[m];
}

hipError_t launch_gdn_replay(float* S_all, const float* tape_all, int n_layers, int B, int gh, int dk, int dv,
                             const int32_t* d_acc, int host_count, const int32_t* scal, int capacity,
                             hipStream_t s) {
  if (n_layers <= 0) return hipSuccess;
  dim3 grid(gh, n_layers);
  if (dk == 128 && dv == 128)
    hipLaunchKernelGGL((gdn_replay_kernel<128, 128>), grid, dim3(512), 0, s, S_all, tape_all, B, gh, d_acc,
                       host_count, scal, capacity);
  else if (dk == 32 && dv == 32)
    hipLaunchKernelGGL((gdn_replay_kernel<32, 32>), grid, dim3(128), 0, s, S_all, tape_all, B, gh, d_acc,
                       host_count, scal, capacity);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dfl
