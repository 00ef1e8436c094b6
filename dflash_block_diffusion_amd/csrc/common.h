// Internal declarations shared by the HIP translation units of libdflash.
// gfx950 only: wave64, MFMA f32_16x16x32_{f16,bf16}.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

// element types of activation buffers
enum ElemType { T_F32 = 0, T_BF16 = 1, T_F16 = 2 };

// weight formats (same values as DFLASH_FMT_*)
enum WFmt { W_F32 = 0, W_BF16 = 1, W_W8 = 2, W_W4 = 3 };

constexpr int PAGE = 64;         // tokens per KV page
constexpr int ATTN_SPLIT = 256;  // keys per attention work-group (4 pages) ...
constexpr int ATTN_SPLIT_SMALL = 128;  // ... or 2 pages, for states of at most ATTN_SMALL_CAP positions
constexpr int ATTN_SMALL_CAP = 1792;
constexpr int MAX_ROWS = 64;     // max GEMM rows (tokens) per call

inline int elem_bytes(int t) { return t == T_F32 ? 4 : 2; }

// K elements covered by one 1 KiB tile of 16 rows (each lane holds 16 bytes)
inline __host__ __device__ constexpr int tile_k(int fmt) {
  return fmt == W_BF16 ? 32 : (fmt == W_W8 ? 64 : 128);
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet); both results
// are formed and one selected, so no divergent branch is emitted
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rn = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t qnan = (u >> 16) | 0x40u;
  return (u & 0x7fffffffu) > 0x7f800000u ? qnan : rn;
}
__device__ __forceinline__ float round_bf16(float f) { return bf16_bits_to_f32(f32_to_bf16_bits(f)); }
// two fp32 values rounded to nearest-even bf16 and packed, low half first: one
// v_cvt_pk_bf16_f32, equal to f32_to_bf16_bits on every non-NaN input
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float floatx2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2v){lo, hi}, bf16x2v));
}

// Load one activation element as fp32.
__device__ __forceinline__ float load_act(const void* p, size_t i, int t) {
  if (t == T_F32) return ((const float*)p)[i];
  uint16_t h = ((const uint16_t*)p)[i];
  if (t == T_BF16) return bf16_bits_to_f32(h);
  return (float)__builtin_bit_cast(_Float16, h);
}

// Store an activation element.  bf16 is the materialisation format of all
// 16-bit activations; T_F16 buffers hold the fp16 encoding of the same
// bf16-rounded value (exact for |v| in [2^-17, 65504]), which is what the
// fp16 MFMA of the quantised GEMMs consumes.  T_F32 stores v unrounded.
__device__ __forceinline__ void store_act(void* p, size_t i, int t, float v) {
  if (t == T_F32) { ((float*)p)[i] = v; return; }
  uint32_t b = f32_to_bf16_bits(v);
  if (t == T_BF16) { ((uint16_t*)p)[i] = (uint16_t)b; return; }
  _Float16 h = (_Float16)bf16_bits_to_f32(b);
  ((uint16_t*)p)[i] = __builtin_bit_cast(uint16_t, h);
}
// value the stored element will read back as
__device__ __forceinline__ float act_round(int t, float v) { return t == T_F32 ? v : round_bf16(v); }

// Status word bit (DFLASH_STATUS_ACT_RANGE): a bf16 activation feeding an
// fp16 GEMM input lay outside the finite fp16 range (|v| > 65504, where the
// fp16 encoding reads back as inf) or was NaN.  bf16 values at or below
// 65280 are finite in fp16; the next bf16 value, 65536, is not.
constexpr int STATUS_ACT_RANGE = 4;
__device__ __forceinline__ void flag_f16_range(int t, float v, int32_t* status) {
  if (t == T_F16 && status && !(fabsf(v) <= 65504.0f)) atomicOr(status, STATUS_ACT_RANGE);
}
// store_act that also reports an fp16 range violation to *status (if not null)
__device__ __forceinline__ void store_act(void* p, size_t i, int t, float v, int32_t* status) {
  if (t == T_F16) flag_f16_range(t, round_bf16(v), status);
  store_act(p, i, t, v);
}

// Fragment-major ("tiled") layout of 16-bit GEMM inputs X[t][k] with K
// columns: 16-token blocks are outermost and contiguous; inside a block,
// every 32-column step is one 1 KiB MFMA operand fragment in lane order
// (lane = t%16 + 16*((k%32)/8), 8 consecutive k per lane).  A wave then
// loads each operand fragment with one contiguous 1 KiB read.
__host__ __device__ __forceinline__ size_t fm_index(int t, int k, int K) {
  return ((size_t)(t >> 4) * (K >> 5) + (k >> 5)) * 512 + (size_t)(((t & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7));
}
// index of element (t, k) of a GEMM input: tiled when fmK > 0 (fmK = K),
// row-major with leading dimension ld otherwise (fp32 inputs)
__device__ __forceinline__ size_t act_index(int t, int k, int ld, int fmK) {
  return fmK ? fm_index(t, k, fmK) : (size_t)t * ld + k;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Sum over a full wave (every lane active), left in every lane: DPP steps
// inside each row of 16 lanes (quad swaps, then the 8- and 16-lane mirrors,
// after which all 16 lanes hold the row's sum bit for bit), then the four
// row sums in a fixed order.  No LDS round trip.
#define DFL_DPP_ADD(v, ctrl) \
  ((v) + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (v)), (ctrl), 0xF, 0xF, true)))
__device__ __forceinline__ float wave_sum_full(float v) {
  v = DFL_DPP_ADD(v, 0xB1);   // quad_perm [1,0,3,2]
  v = DFL_DPP_ADD(v, 0x4E);   // quad_perm [2,3,0,1]
  v = DFL_DPP_ADD(v, 0x141);  // row_half_mirror
  v = DFL_DPP_ADD(v, 0x140);  // row_mirror
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}
#undef DFL_DPP_ADD

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ------------------------------------------------------------ GEMM interface
struct GemmW {
  int fmt, n, k, gate_up;
  const void* w;      // packed
  const void* s;      // packed scales (W8/W4) or null
};

// EPI_PARTIAL: fp32 partial sums [S][m][n] of S K ranges (one range for fp32
//              models), added up by the consuming kernel (see Parts);
// EPI_SILU:    fused gate/up -> silu(gate) * up, 16-bit tiled output (K = n/2);
// EPI_ARGMAX:  per-row argmax over n (lowest index on ties), optional logits.
enum Epi { EPI_PARTIAL = 0, EPI_SILU = 2, EPI_ARGMAX = 3 };

struct GemmCall {
  const GemmW* W;
  const void* x; int ldx;        // activations: F32 row-major [rows][ldx] for W_F32; tiled
                                 // (fm_index with K) BF16 for W_BF16, F16 for W8/W4
  int m;                         // valid rows (<= 64); kernels compute ceil(m/16)*16 rows
  int epi;
  float* part;                   // PARTIAL: [S][m][n]
  void* out; int otype;          // SILU output
  // ARGMAX
  float* logits; int ldl; int row0;         // optional fp32 logits of rows row0..m-1
  int32_t* am_out;                          // argmax of rows row0..m-1 -> am_out[0..]
  int32_t* status;                          // SILU: range flag of fp16 outputs (or null)
};

struct Workspace {
  float* part; size_t part_floats;          // split-K partials
  float* am_val; int* am_idx; int am_cap;   // argmax partials [am_cap][64]
  float* logits_tmp;                        // F32 path: [64][V] logits scratch
};

// RT row tiles per chunk, MB 16-token blocks, S K splits, PR work-groups per
// split (nwg = PR * S), align = row tiles per balancing unit (2 for gate/up)
struct Plan { int RT, MB, S, PR, ngroups, nwg, ktiles, ntile16, align, NW; };
Plan make_plan(int fmt, int n, int k, int m, int epi);
// prompt chunks: m in (64, 1024], m % 16 == 0, W4 or W8 weights (K % 128 == 0), partial-sum or
// SiLU epilogue (launch_gemm takes this path for m > 64)
bool dense_ok(int fmt, int n, int k, int m, int epi);
int dense_splits(int fmt, int n, int k, int m, int epi);
struct Workspace;

hipError_t launch_gemm(const GemmCall& c, const Workspace& w, hipStream_t s, const char** variant,
                       double* bytes, int* splits, double* io_bytes = nullptr);
hipError_t launch_gemm_plan(const GemmCall& c, const Workspace& w, hipStream_t s, const Plan& p);
hipError_t launch_pack(int fmt, int n, int k, int gate_up, const void* src, const void* src_scales,
                       void* dst, void* dst_scales, hipStream_t s);
hipError_t launch_sum_parts(const float* part, int S, size_t count, float* out, hipStream_t s);
void packed_bytes(int fmt, int n, int k, size_t* wb, size_t* sb);
int gemm_am_blocks(int fmt, int n, int m);

// The S fp32 partials of one PARTIAL launch as seen by a consumer: element
// (t, n) is the sum over s of p[s*stride + t*ld + n], added in split order.
struct Parts {
  const float* p;
  int S;
  size_t stride;   // floats between splits (m * n of the launch)
  int ld;          // row stride (n of the launch)
};
// LDS pointer, the destination of direct global->LDS loads
typedef __attribute__((address_space(3))) void* lds_ptr;
// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (vmcnt in bits 3:0 and 15:14; expcnt 7 and lgkmcnt 15: not waited on)
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// 16 bytes per lane from src to LDS at lds + 16 * lane (lds wave-uniform).
// Issued from asm so that the compiler does not track it: its wait analysis
// would otherwise drain every such load before unrelated register reads.
// Callers wait for it with explicit vmcnt waits (a vector-memory load, in
// issue order with the others).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_ptr)p; }

constexpr int MAX_SPLITS = 8;
// All S loads are issued before the first add (S <= MAX_SPLITS), so the
// partials cost one memory round trip, not S.  parts_fetch only issues the
// loads, so that a kernel can put other loads in flight before parts_add.
__device__ __forceinline__ void parts_fetch(const Parts& P, int t, int n, float (&x)[MAX_SPLITS]) {
  const float* q = P.p + (size_t)t * P.ld + n;
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s) x[s] = s < P.S ? q[(size_t)s * P.stride] : 0.f;
}
__device__ __forceinline__ float parts_add(const Parts& P, const float (&x)[MAX_SPLITS]) {
  float v = x[0];
#pragma unroll
  for (int s = 1; s < MAX_SPLITS; ++s)
    if (s < P.S) v = v + x[s];
  return v;
}
__device__ __forceinline__ float parts_sum(const Parts& P, int t, int n) {
  float x[MAX_SPLITS];
  parts_fetch(P, t, n, x);
  return parts_add(P, x);
}

// ------------------------------------------------------------ other kernels
struct RopeCall {
  Parts qkv; int atype;                     // QKV GEMM partials [rows][n_qkv]; rounded to atype
  int block_rows;                           // B: rows 0..B-1 at positions n+i
  int ctx_rows;                             // drafter: rows B..B+ctx_rows-1 are context rows
  const int* dev_n; const int* dev_p;       // committed length, pending context rows
  const float* q_norm; const float* k_norm; float eps;
  const float* cos_t; const float* sin_t;   // [capacity][d/2]
  void* q_out;                              // [B][hq][d] act
  void* kc; void* vc; const int* page_table; int capacity;
  int hq, hkv, d;
  int ctx_at_n = 0;                         // 1: context row j sits at position n+j and every
                                            //    row is kept (dev_p unused; no block rows)
};
hipError_t launch_qk_rope(const RopeCall& c, hipStream_t s);

struct AttnCall {
  const void* q; int atype;                  // [B][hq][d] act (bf16 or f32)
  const void* kc; const void* vc; const int* page_table;
  const int* dev_n; int block_rows; int causal;
  int hq, hkv, d; int max_splits; int npages;  // key splits of the state; pages in the table
  int split = ATTN_SPLIT;                     // keys per split (ATTN_SPLIT or ATTN_SPLIT_SMALL)
  float* o_part; float* ml_part;              // [max_splits][B*hq][d], [max_splits][B*hq][2]
  void* out; int otype; int ldo;              // [B][hq*d]
  int32_t* status;                            // range flag of fp16 outputs (or null)
};
hipError_t launch_attention(const AttnCall& c, hipStream_t s);

// Temperature sampling (csrc/sample.hip).  launch_sample_rows: per row of
// logits ([rows][ld] fp32) the log-normaliser log sum exp(z/T) -> out_lse[r]
// (if not null) and, for stream >= 0, a draw from softmax(z/T) with Philox
// counter (n, row0 + r, stream), n = *dev_n + n_add (n_add when dev_n is
// null) -> out_tok[r].  launch_spec_accept: speculative-sampling acceptance
// over N verified drafts plus the correction/bonus draw (accept/emit/next
// anchor as dflash_accept).
hipError_t launch_sample_rows(const float* logits, int ld, int vocab, int rows, float temperature, uint64_t seed,
                              const int* dev_n, int n_add, int row0, int stream, int32_t* out_tok, float* out_lse,
                              hipStream_t s);
hipError_t launch_spec_accept(const int32_t* block, const float* dlog, const float* vlog, int vocab, int N,
                              const float* lse_q, const float* lse_p, float temperature, uint64_t seed,
                              const int* dev_n, int n_add, int B, int32_t* acc, int32_t* emit,
                              int32_t* next_anchor, hipStream_t s);

// Residual update + RMSNorm of `rows` rows of width h, one work-group per row:
//   NORM_ONLY  v = x
//   NORM_RESID v = round(x + round(sum of in)); x <- v; side copy of v (optional)
//   NORM_PROJ  v = round(sum of in)            (x untouched)
// then out = round(v * (mean(v^2) + eps)^-1/2 * gain).  out is tiled (K = h)
// when otype is 16-bit and tiled != 0, else row-major [rows][ldo].
enum NormMode { NORM_ONLY = 0, NORM_RESID = 1, NORM_PROJ = 2 };
struct NormCall {
  int mode;
  Parts in;
  void* x; int xtype; int ldx;              // residual stream (row-major)
  void* side; int side_type; int ld_side; int side_col0;   // tiled (K = ld_side) when 16-bit
  const float* gain; float eps; int h; int rows;
  void* out; int otype; int ldo; int tiled;
  int32_t* status;                          // range flag of fp16 outputs (or null)
};
hipError_t launch_norm(const NormCall& c, hipStream_t s);
hipError_t launch_embed(const void* table, int ttype, int h, int vocab, const int32_t* tokens,
                        int mask_mode, int mask_token, int rows, void* out, int ldo,
                        int32_t* status, hipStream_t s);
hipError_t launch_argmax_final(const float* am_val, const int* am_idx, int nblocks, int row0,
                               int rows, int32_t* out, hipStream_t s);
hipError_t launch_argmax_rows(const float* logits, int ld, int vocab, int row0, int rows,
                              int32_t* out, float* logits_copy, int ldc, hipStream_t s);
hipError_t launch_accept(const int32_t* block, const int32_t* y, int B, int32_t* acc,
                         int32_t* emit, int32_t* next_anchor, hipStream_t s);
hipError_t launch_commit(int32_t* scal, const int32_t* d_acc, int host_count, const int32_t* emit,
                         int32_t* tokens, int32_t* acc_log, int acc_log_len, int capacity, int B,
                         hipStream_t s);
hipError_t launch_set_scalars(int32_t* scal, int n, int p, int clear_status, hipStream_t s);
hipError_t launch_copy_tokens(const int32_t* src, int32_t* dst, int count, hipStream_t s);
hipError_t launch_rollback(int32_t* scal, int new_len, const int32_t* tokens, int32_t* block,
                           hipStream_t s);
hipError_t launch_inject(const int32_t* scal, int32_t* block, int B, const int32_t* ref, int ref_len,
                         const int32_t* sched, int n_sched, const int32_t* filler, int vocab,
                         hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, size_t count, int32_t v, hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, size_t count, hipStream_t s);

// GatedDeltaNet
struct GdnCall {
  Parts proj; int atype;                    // [B][gh*(2dk+dv)+2gh] GEMM partials, rounded to atype
  int rows; int gh, dk, dv;
  const float* S;                            // committed state [gh][dv][dk]
  float* tape;                               // [B][gh][dk+dv+2]
  void* out; int otype; int ldo;             // o [B][gh*dv]
  int32_t* status;                           // range flag of fp16 outputs (or null)
};
hipError_t launch_gdn_verify(const GdnCall& c, hipStream_t s);
// a prompt chunk of c.rows = nblk * B committed tokens: verify and replay
// block by block into c.S (updated in place); no tape
hipError_t launch_gdn_prompt(const GdnCall& c, int B, hipStream_t s);
// replays cnt = a+1 (or host_count) tape tokens into every GDN layer's state;
// skipped when the matching commit will be refused for capacity
hipError_t launch_gdn_replay(float* S_all, const float* tape_all, int n_layers, int B, int gh, int dk,
                             int dv, const int32_t* d_acc, int host_count, const int32_t* scal,
                             int capacity, hipStream_t s);

// scalar slots in the arena
enum Scalar { SC_N = 0, SC_P = 1, SC_STEP = 2, SC_STATUS = 3, SC_SNAP_N = 4,
              SC_VBASE = 5,    // n when the last verify was enqueued (its row 0's position)
              SC_STATUS2 = 6,  // status bits of work on the overlap stream
              SC_COUNT = 16 };

}  // namespace dfl
