// Host side of libdflash: the C ABI declared in include/dflash.h.
//
// Orchestrates the kernels of one draft+verify step on a caller's stream:
//   draft   context projection (fc + RMSNorm) of the rows the previous verify
//           committed, embedding of [anchor, mask x (B-1)], drafter layers
//           (block queries over committed-context + block keys, bidirectional),
//           final norm, the TARGET's lm-head + argmax (drafts d_1..d_{B-1});
//   verify  embedding of the block, target layers (causal over context and
//           block; GatedDeltaNet layers record their tape), conditioning-layer
//           outputs copied to the drafter's context buffer, lm-head + argmax;
//   accept  longest matching prefix + correction;
//   commit  GDN tape replay, n += a+1, token log, pending context rows.
// Every length that changes per step is read by the kernels from device
// memory, so one step can be captured once as a hipGraph and replayed.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "dflash.h"

using namespace dfl;

static thread_local std::string g_err;

static int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPCHK(x)                                                                          \
  do {                                                                                     \
    hipError_t e_ = (x);                                                                   \
    if (e_ != hipSuccess) return fail(DFLASH_E_DEVICE, std::string(#x) + ": " + hipGetErrorString(e_)); \
  } while (0)

extern "C" const char* dflash_last_error(void) { return g_err.c_str(); }

extern "C" int dflash_device_count(int* h_count) {
  if (!h_count) return fail(DFLASH_E_INVALID, "h_count is null");
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess) { *h_count = 0; return fail(DFLASH_E_DEVICE, hipGetErrorString(e)); }
  *h_count = n;
  return DFLASH_OK;
}

// ------------------------------------------------------------------ weights
static bool fmt_ok(int fmt) { return fmt >= DFLASH_FMT_F32 && fmt <= DFLASH_FMT_W4A16; }

static int check_gemm_shape(int fmt, int n, int k, int gate_up) {
  if (n <= 0 || k <= 0) return fail(DFLASH_E_SHAPE, "GEMM dims must be positive");
  if (n % (gate_up ? 32 : 16)) return fail(DFLASH_E_SHAPE, "GEMM N must be a multiple of 16 (32 for gate/up)");
  if (fmt != DFLASH_FMT_F32 && k % tile_k(fmt))
    return fail(DFLASH_E_SHAPE, "GEMM K must be a multiple of " + std::to_string(tile_k(fmt)) + " for this format");
  return DFLASH_OK;
}

extern "C" int dflash_packed_bytes(int fmt, int n, int k, size_t* wb, size_t* sb) {
  if (!fmt_ok(fmt) || !wb || !sb) return fail(DFLASH_E_INVALID, "bad format or null output");
  int rc = check_gemm_shape(fmt, n, k, 0);
  if (rc) return rc;
  packed_bytes(fmt, n, k, wb, sb);
  return DFLASH_OK;
}

extern "C" int dflash_pack_weight(int fmt, int n, int k, int gate_up, const void* src, const void* src_scales,
                                  void* dst, void* dst_scales, void* stream) {
  if (!fmt_ok(fmt)) return fail(DFLASH_E_INVALID, "unknown weight format");
  if (!src || !dst) return fail(DFLASH_E_INVALID, "null source or destination");
  if ((fmt == DFLASH_FMT_W8A16 || fmt == DFLASH_FMT_W4A16) && (!src_scales || !dst_scales))
    return fail(DFLASH_E_INVALID, "quantised formats need scales");
  int rc = check_gemm_shape(fmt, n, k, gate_up);
  if (rc) return rc;
  HIPCHK(launch_pack(fmt, n, k, gate_up, src, src_scales, dst, dst_scales, (hipStream_t)stream));
  return DFLASH_OK;
}

static GemmW mkw(int fmt, int n, int k, int gu, const void* w, const void* s);

// ------------------------------------------------------------------ one linear
struct LinearWs {
  size_t part_off, amv_off, ami_off, lg_off, total;
  size_t part_floats;
};

static LinearWs linear_ws_layout(int fmt, int n, int k, int m) {
  LinearWs L;
  size_t off = 0;
  auto take = [&](size_t bytes) { off = (off + 255) & ~(size_t)255; size_t o = off; off += bytes; return o; };
  const int S = m > MAX_ROWS ? dense_splits(fmt, n, k, m, EPI_PARTIAL) : make_plan(fmt, n, k, m, EPI_PARTIAL).S;
  L.part_floats = (size_t)S * m * n;
  L.part_off = take(L.part_floats * 4);
  const int am = m > MAX_ROWS ? 1 : std::max(1, gemm_am_blocks(fmt, n, m));
  L.amv_off = take((size_t)am * 64 * 4);
  L.ami_off = take((size_t)am * 64 * 4);
  L.lg_off = take(fmt == DFLASH_FMT_F32 ? (size_t)MAX_ROWS * n * 4 : 4);
  L.total = off;
  return L;
}

// rows a dflash_linear call takes: up to 64 for every format, and prompt
// chunks (multiples of 16 up to 1024) for W4A16 / W8A16 with the fp32 output
static bool linear_rows_ok(int fmt, int n, int k, int m, int epilogue) {
  if (m >= 1 && m <= MAX_ROWS) return true;
  return epilogue == 0 && dense_ok(fmt, n, k, m, EPI_PARTIAL);
}

extern "C" size_t dflash_linear_workspace_bytes(int fmt, int n, int k, int m) {
  if (!fmt_ok(fmt) || check_gemm_shape(fmt, n, k, 0) || !linear_rows_ok(fmt, n, k, m, 0)) return 0;
  return linear_ws_layout(fmt, n, k, m).total;
}

// argument checks shared by dflash_linear and dflash_linear_noalloc (the
// workspace is checked by the caller)
static int linear_check(int fmt, int n, int k, const void* w, const void* sc, const void* x, int ldx, int m,
                        int epilogue, float* out, int32_t* am) {
  if (!fmt_ok(fmt)) return fail(DFLASH_E_INVALID, "unknown weight format");
  int rc = check_gemm_shape(fmt, n, k, 0);
  if (rc) return rc;
  if (!linear_rows_ok(fmt, n, k, m, epilogue))
    return fail(DFLASH_E_SHAPE, "m must be in [1, 64] (or, BF16/W8A16/W4A16 with epilogue 0, a multiple of 16 up to 1024)");
  if (fmt == DFLASH_FMT_F32 && ldx < k) return fail(DFLASH_E_SHAPE, "ldx must be >= k");
  if (!w || !x || (fmt >= DFLASH_FMT_W8A16 && !sc)) return fail(DFLASH_E_INVALID, "null argument");
  if (epilogue == 0 && !out) return fail(DFLASH_E_INVALID, "epilogue 0 needs d_out");
  if (epilogue == 1 && !am) return fail(DFLASH_E_INVALID, "epilogue 1 needs d_argmax");
  if (epilogue != 0 && epilogue != 1) return fail(DFLASH_E_INVALID, "unknown epilogue");
  return DFLASH_OK;
}

// enqueue one checked linear with its workspace at ws (device memory of at
// least linear_ws_layout(...).total bytes)
static int linear_run(int fmt, int n, int k, const void* w, const void* sc, const void* x, int ldx, int m,
                      int epilogue, float* out, int32_t* am, void* ws, void* stream) {
  const LinearWs L = linear_ws_layout(fmt, n, k, m);
  char* b = (char*)ws;
  Workspace W;
  W.part = (float*)(b + L.part_off); W.part_floats = L.part_floats;
  W.am_val = (float*)(b + L.amv_off); W.am_idx = (int*)(b + L.ami_off);
  W.am_cap = std::max(1, gemm_am_blocks(fmt, n, m));
  W.logits_tmp = (float*)(b + L.lg_off);
  GemmW g = mkw(fmt, n, k, 0, w, sc);
  GemmCall c{};
  c.W = &g; c.x = x; c.ldx = ldx; c.m = m;
  c.epi = epilogue == 0 ? EPI_PARTIAL : EPI_ARGMAX;
  c.part = W.part; c.out = nullptr; c.otype = T_F32;
  c.logits = epilogue == 1 ? out : nullptr; c.ldl = n; c.row0 = 0; c.am_out = am;
  int S = 1;
  HIPCHK(launch_gemm(c, W, (hipStream_t)stream, nullptr, nullptr, &S));
  if (epilogue == 0) HIPCHK(launch_sum_parts(W.part, S, (size_t)m * n, out, (hipStream_t)stream));
  return DFLASH_OK;
}

extern "C" int dflash_linear(int fmt, int n, int k, const void* w, const void* sc, const void* x, int ldx, int m,
                             int epilogue, float* out, int32_t* am, void* ws, size_t ws_bytes, void* stream) {
  int rc = linear_check(fmt, n, k, w, sc, x, ldx, m, epilogue, out, am);
  if (rc) return rc;
  if (!ws) return fail(DFLASH_E_INVALID, "null workspace");
  if (ws_bytes < linear_ws_layout(fmt, n, k, m).total) return fail(DFLASH_E_INVALID, "workspace too small");
  return linear_run(fmt, n, k, w, sc, x, ldx, m, epilogue, out, am, ws, stream);
}

// ------------------------------------------------------------ static scratch
// Workspace of dflash_linear_noalloc: a file-scope device array, one copy per
// device, resident until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: its device address is looked up
// once per device (with that device current) by hipGetSymbolAddress and only
// that address is handed to kernels.  Nothing in it has to start at zero:
// every call writes the split partials and argmax partials it then reads.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

static int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[NOALLOC_MAX_DEVICES] = {nullptr};
  int dev = -1;
  HIPCHK(hipGetDevice(&dev));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(DFLASH_E_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DFLASH_E_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return DFLASH_OK;
}

extern "C" size_t dflash_linear_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

extern "C" int dflash_linear_noalloc(int fmt, int n, int k, const void* w, const void* sc, const void* x, int ldx,
                                     int m, int epilogue, float* out, int32_t* am, void* stream) {
  int rc = linear_check(fmt, n, k, w, sc, x, ldx, m, epilogue, out, am);
  if (rc) return rc;
  const size_t need = linear_ws_layout(fmt, n, k, m).total;
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(DFLASH_E_CAPACITY, "this linear needs " + std::to_string(need) + " bytes of workspace; the static "
                "scratch holds " + std::to_string(NOALLOC_SCRATCH_BYTES) + " (use dflash_linear with a workspace)");
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return linear_run(fmt, n, k, w, sc, x, ldx, m, epilogue, out, am, ws, stream);
}

// ------------------------------------------------------------------ models
struct Layer {
  int kind;
  const float *in_norm, *post_norm, *q_norm, *k_norm;
  GemmW qkv, o, gu, down;
};

struct dflash_model {
  dflash_model_desc d;
  std::vector<Layer> layers;
  GemmW lm{}, fc{};
  const dflash_model* target = nullptr;   // drafter: bound target
  bool drafter = false;
  int act = T_F32;                        // residual / KV / q type
  int gin = T_F32;                        // GEMM input type
  int n_gdn = 0;
};

static GemmW mkw(int fmt, int n, int k, int gu, const void* w, const void* s) {
  GemmW g;
  g.fmt = fmt; g.n = n; g.k = k; g.gate_up = gu; g.w = w; g.s = s;
  return g;
}

extern "C" int dflash_model_create(const dflash_model_desc* desc, dflash_model** out) {
  if (!desc || !out) return fail(DFLASH_E_INVALID, "null desc or out");
  *out = nullptr;
  const dflash_model_desc& d = *desc;
  if (!fmt_ok(d.fmt)) return fail(DFLASH_E_INVALID, "unknown weight format");
  if (d.n_layers <= 0 || !d.layers) return fail(DFLASH_E_INVALID, "no layers");
  if (d.hidden <= 0 || d.n_q_heads <= 0 || d.n_kv_heads <= 0 || d.ffn <= 0 || d.vocab <= 1)
    return fail(DFLASH_E_SHAPE, "non-positive dimension");
  if (d.head_dim != 64 && d.head_dim != 128) return fail(DFLASH_E_SHAPE, "head_dim must be 64 or 128");
  if (d.fmt != DFLASH_FMT_F32 && d.head_dim != 128)
    return fail(DFLASH_E_SHAPE, "16-bit attention needs head_dim 128");
  if (d.n_q_heads % d.n_kv_heads) return fail(DFLASH_E_SHAPE, "n_q_heads must be a multiple of n_kv_heads");
  if (d.hidden % 16) return fail(DFLASH_E_SHAPE, "hidden must be a multiple of 16");
  const bool drafter = d.w_fc != nullptr;
  if (!drafter && (!d.embed || !d.w_lm || !d.final_norm))
    return fail(DFLASH_E_INVALID, "a target needs embed, w_lm and final_norm");
  if (drafter && (!d.hidden_norm || !d.final_norm || d.n_sel <= 0 || d.n_sel > 8))
    return fail(DFLASH_E_INVALID, "a drafter needs w_fc, hidden_norm, final_norm and 1..8 sel_layers");
  if (drafter && (d.mask_token < 0 || d.mask_token >= d.vocab)) return fail(DFLASH_E_INVALID, "mask_token out of range");
  auto* m = new dflash_model();
  m->d = d;
  m->drafter = drafter;
  m->act = d.fmt == DFLASH_FMT_F32 ? T_F32 : T_BF16;
  m->gin = d.fmt == DFLASH_FMT_F32 ? T_F32 : d.fmt == DFLASH_FMT_BF16 ? T_BF16 : T_F16;
  const int H = d.hidden, F = d.ffn, hq = d.n_q_heads, hkv = d.n_kv_heads, hd = d.head_dim;
  int rc = DFLASH_OK;
  for (int l = 0; l < d.n_layers && rc == DFLASH_OK; ++l) {
    const dflash_layer_desc& L = d.layers[l];
    Layer y;
    y.kind = L.kind;
    y.in_norm = L.in_norm; y.post_norm = L.post_norm; y.q_norm = L.q_norm; y.k_norm = L.k_norm;
    if (!L.in_norm || !L.post_norm || !L.w_qkv || !L.w_o || !L.w_gu || !L.w_down) {
      rc = fail(DFLASH_E_INVALID, "layer " + std::to_string(l) + " is missing a tensor");
      break;
    }
    if (L.kind == DFLASH_LAYER_ATTN) {
      if (!L.q_norm || !L.k_norm) { rc = fail(DFLASH_E_INVALID, "attention layer needs q/k norms"); break; }
      y.qkv = mkw(d.fmt, (hq + 2 * hkv) * hd, H, 0, L.w_qkv, L.s_qkv);
      y.o = mkw(d.fmt, H, hq * hd, 0, L.w_o, L.s_o);
    } else if (L.kind == DFLASH_LAYER_GDN) {
      if (drafter) { rc = fail(DFLASH_E_UNSUPPORTED, "GatedDeltaNet layers are supported in targets only"); break; }
      const int gh = d.gdn_heads, dk = d.gdn_dk, dv = d.gdn_dv;
      if (!((dk == 128 && dv == 128) || (dk == 32 && dv == 32)) || gh <= 0) {
        rc = fail(DFLASH_E_SHAPE, "GatedDeltaNet needs dk == dv in {32, 128}");
        break;
      }
      y.qkv = mkw(d.fmt, gh * (2 * dk + dv) + 2 * gh, H, 0, L.w_qkv, L.s_qkv);
      y.o = mkw(d.fmt, H, gh * dv, 0, L.w_o, L.s_o);
      m->n_gdn++;
    } else {
      rc = fail(DFLASH_E_INVALID, "unknown layer kind");
      break;
    }
    y.gu = mkw(d.fmt, 2 * F, H, 1, L.w_gu, L.s_gu);
    y.down = mkw(d.fmt, H, F, 0, L.w_down, L.s_down);
    for (const GemmW* g : {&y.qkv, &y.o, &y.gu, &y.down}) {
      if (rc == DFLASH_OK) rc = check_gemm_shape(g->fmt, g->n, g->k, g->gate_up);
      if (rc == DFLASH_OK && g->fmt >= DFLASH_FMT_W8A16 && !g->s) rc = fail(DFLASH_E_INVALID, "missing scales");
    }
    m->layers.push_back(y);
  }
  if (rc == DFLASH_OK && !drafter) {
    m->lm = mkw(d.fmt, d.vocab, H, 0, d.w_lm, d.s_lm);
    rc = check_gemm_shape(d.fmt, d.vocab, H, 0);
  }
  if (rc == DFLASH_OK && drafter) {
    m->fc = mkw(d.fmt, H, d.n_sel * H, 0, d.w_fc, d.s_fc);
    rc = check_gemm_shape(d.fmt, H, d.n_sel * H, 0);
  }
  if (rc != DFLASH_OK) { delete m; return rc; }
  m->d.layers = nullptr;   // the caller's array is not kept
  *out = m;
  return DFLASH_OK;
}

extern "C" void dflash_model_destroy(dflash_model* m) { delete m; }

extern "C" int dflash_drafter_bind(dflash_model* drafter, const dflash_model* target) {
  if (!drafter || !target) return fail(DFLASH_E_INVALID, "null model");
  if (!drafter->drafter || target->drafter) return fail(DFLASH_E_INVALID, "bind(drafter, target) arguments swapped");
  if (drafter->d.hidden != target->d.hidden || drafter->d.vocab != target->d.vocab)
    return fail(DFLASH_E_SHAPE, "drafter and target must share hidden size and vocab");
  if (drafter->act != target->act) return fail(DFLASH_E_SHAPE, "drafter and target activation types differ");
  for (int i = 0; i < drafter->d.n_sel; ++i) {
    const int l = drafter->d.sel_layers[i];
    if (l < 0 || l >= target->d.n_layers || (i > 0 && l <= drafter->d.sel_layers[i - 1]))
      return fail(DFLASH_E_SHAPE, "conditioning layers must be ascending target layer indices");
  }
  drafter->target = target;
  return DFLASH_OK;
}

// ------------------------------------------------------------------ state
struct ProfRec { const char* name; double bytes, io_bytes; hipEvent_t a, b; GemmCall call; };

// Partial sums a GEMM left for the next residual/norm kernel, and where the
// new residual is to be copied (conditioning layers feed the drafter).
struct Pending {
  Parts in{nullptr, 0, 0, 0};
  void* side = nullptr; int side_type = 0; int ld_side = 0; int side_col0 = 0;
};

struct dflash_state {
  const dflash_model* t = nullptr;
  const dflash_model* dr = nullptr;
  int B = 0, max_ctx = 0, capacity = 0, pages = 0, max_splits = 0;
  int split = ATTN_SPLIT;   // keys per block-attention split
  int vrows = 0;          // rows a verify runs (B, or fewer under a draft cap)
  int pm = 0;             // rows of a dense prompt chunk (0: prompts run in blocks of B)
  bool pm_draft = false;  // the drafter's context pass of a chunk runs dense as well
  int max_draft = 0;      // drafts verified per step (0 = the whole block)
  float temp = 0.f;       // sampling temperature (0 = greedy)
  uint64_t seed = 0;
  float* dlog = nullptr;  // [B][vocab] drafter logits of slots 1..B-1 (sampling)
  float* vlog = nullptr;  // [B][vocab] target logits of the verify rows (sampling)
  float* lse = nullptr;   // [2][B] log-normalisers at T: drafter slots, target rows
  char* base = nullptr;
  size_t bytes = 0;
  int32_t* scal = nullptr;
  int32_t* tokens = nullptr;
  int32_t* acc_log = nullptr;
  int acc_log_len = 4096;
  float* cos_t = nullptr;
  float* sin_t = nullptr;
  int32_t* pt = nullptr;
  std::vector<void*> tk, tv, dk, dv;
  void* x = nullptr;      // residual [64][H] act
  void* bu = nullptr;     // norm outputs / QKV input [64][H] gin
  void* ba = nullptr;     // attention or GDN output [64][max(hq*d, gh*dv)] gin
  void* bf = nullptr;     // SiLU*mul output [64][F] gin
  void* bqkv = nullptr;   // QKV / GDN projection [64][Nqkv] act
  void* bq = nullptr;     // q after norm+rope [B][hq][d] act
  void* side = nullptr;   // drafter context input [64][n_sel*H] drafter gin
  float* o_part = nullptr;
  float* ml_part = nullptr;
  Workspace ws{};
  int32_t* ybuf = nullptr;   // [64] prefill argmax scratch
  float* gdn_S = nullptr;
  float* gdn_snap = nullptr;
  float* gdn_tape = nullptr;
  int snap_n = -1;
  bool prof = false;
  std::vector<ProfRec> prof_recs;
  std::vector<hipEvent_t> ev_pool;
  // Draft/verify overlap: a second stream takes the next draft's context rows
  // while the verify finishes (dflash_set_overlap)
  bool ov_on = false;
  hipStream_t ov_stream = nullptr;
  hipEvent_t ov_fork = nullptr, ov_join = nullptr;
  bool ov_pending = false;   // overlap work enqueued and not yet joined
  bool ctx_ready = false;    // the last verify's context rows are in the drafter cache
  Workspace ws2{};           // GEMM workspace of the overlap stream
  void* bu2 = nullptr;       // context features of the overlap stream [B][H] drafter gin
  std::vector<GemmW> dkv;    // each drafter layer's k/v rows of its QKV weight
};

struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(char* b) : base(b) {}
  template <class T>
  T* take(size_t count) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

static int gdn_rec(const dflash_model* t) { return t->d.gdn_dk + t->d.gdn_dv + 2; }

// rows of a dense prompt chunk (a multiple of both block sizes)
constexpr int DENSE_PROMPT_ROWS = 1024;

// The k and v output rows of a QKV projection (rows hq*d .. (hq+2*hkv)*d)
// as a weight of their own: packed weights are stored row tile by row tile
// (16 output rows, all K tiles), so a whole-tile row range is contiguous, and
// so are its scales.
static GemmW kv_rows(const GemmW& W, const dflash_model* m) {
  const int r0 = m->d.n_q_heads * m->d.head_dim, rows = 2 * m->d.n_kv_heads * m->d.head_dim;
  GemmW v = W;
  v.n = rows;
  if (W.fmt == W_F32) {
    v.w = (const char*)W.w + (size_t)r0 * W.k * 4;
    return v;
  }
  const int ktiles = W.k / tile_k(W.fmt);
  v.w = (const char*)W.w + (size_t)(r0 / 16) * ktiles * 1024;
  if (W.fmt == W_W8) v.s = (const char*)W.s + (size_t)r0 * 2;
  if (W.fmt == W_W4) v.s = (const char*)W.s + (size_t)(r0 / 16) * ktiles * 64;
  return v;
}

static void carve(dflash_state* s, Carver& c) {
  const dflash_model *t = s->t, *d = s->dr;
  const int H = t->d.hidden, B = s->B;
  const int eb = t->act == T_F32 ? 4 : 2;
  s->scal = c.take<int32_t>(SC_COUNT);
  s->tokens = c.take<int32_t>(s->capacity + 64);
  s->acc_log = c.take<int32_t>(s->acc_log_len);
  s->cos_t = c.take<float>((size_t)s->capacity * (t->d.head_dim / 2));
  s->sin_t = c.take<float>((size_t)s->capacity * (t->d.head_dim / 2));
  s->pt = c.take<int32_t>(s->pages);
  const size_t tkv = (size_t)s->pages * t->d.n_kv_heads * PAGE * t->d.head_dim * eb;
  s->tk.assign(t->d.n_layers, nullptr);
  s->tv.assign(t->d.n_layers, nullptr);
  for (int l = 0; l < t->d.n_layers; ++l)
    if (t->layers[l].kind == DFLASH_LAYER_ATTN) { s->tk[l] = c.take<char>(tkv); s->tv[l] = c.take<char>(tkv); }
  const size_t dkv = (size_t)s->pages * d->d.n_kv_heads * PAGE * d->d.head_dim * eb;
  s->dk.assign(d->d.n_layers, nullptr);
  s->dv.assign(d->d.n_layers, nullptr);
  for (int l = 0; l < d->d.n_layers; ++l) { s->dk[l] = c.take<char>(dkv); s->dv[l] = c.take<char>(dkv); }
  int qkv_n = 0, att_w = 0, F = 0;
  for (const dflash_model* m : {t, d}) {
    for (const Layer& L : m->layers) {
      qkv_n = std::max(qkv_n, L.qkv.n);
      att_w = std::max(att_w, L.o.k);
    }
    F = std::max(F, m->d.ffn);
  }
  // row buffers: a block (+ its context rows), or a dense prompt chunk
  const size_t R = std::max(MAX_ROWS, s->pm), RB = std::max(B, s->pm);
  s->x = c.take<char>(R * H * 4);
  // (the drafter's context rows sit after the B block rows)
  s->bu = c.take<char>(std::max(R, (size_t)B + (s->pm_draft ? s->pm : 0)) * H * 4);
  s->ba = c.take<char>(R * att_w * 4);
  s->bf = c.take<char>(R * F * 4);
  s->bqkv = c.take<char>(R * qkv_n * 4);
  s->bq = c.take<char>(RB * t->d.n_q_heads * t->d.head_dim * 4 + (size_t)B * d->d.n_q_heads * d->d.head_dim * 4);
  s->side = c.take<char>(R * d->d.n_sel * H * 4);
  const int hq = std::max(t->d.n_q_heads, d->d.n_q_heads), hd = std::max(t->d.head_dim, d->d.head_dim);
  s->o_part = c.take<float>((size_t)s->max_splits * RB * hq * hd);
  s->ml_part = c.take<float>((size_t)s->max_splits * RB * hq * 2);
  // GEMM workspaces: the largest need over every weight of both stacks
  size_t pf = 1;
  int am = 0;
  auto need = [&](const GemmW& g, int m) {
    const Plan p = make_plan(g.fmt, g.n, g.k, m, EPI_PARTIAL);
    pf = std::max(pf, (size_t)p.S * m * g.n);
  };
  for (const Layer& L : t->layers) { need(L.qkv, B); need(L.o, B); need(L.down, B); }
  // a prompt chunk is any multiple of B up to pm rows; fewer rows can take
  // more K splits
  if (s->pm)
    for (int m = B; m <= s->pm; m += B)
      if (m > MAX_ROWS)
        for (const Layer& L : t->layers)
          for (const GemmW* g : {&L.qkv, &L.o, &L.down})
            pf = std::max(pf, (size_t)dense_splits(g->fmt, g->n, g->k, m, EPI_PARTIAL) * m * g->n);
  if (s->pm_draft)
    for (int m = B; m <= s->pm; m += B)
      if (m > MAX_ROWS) {
        pf = std::max(pf, (size_t)dense_splits(d->fc.fmt, d->fc.n, d->fc.k, m, EPI_PARTIAL) * m * d->fc.n);
        for (const Layer& L : d->layers)
          pf = std::max(pf, (size_t)dense_splits(L.qkv.fmt, L.qkv.n, L.qkv.k, m, EPI_PARTIAL) * m * L.qkv.n);
      }
  for (const Layer& L : d->layers) { need(L.qkv, 2 * B); need(L.o, B); need(L.down, B); }
  need(d->fc, B);
  am = std::max(1, gemm_am_blocks(t->lm.fmt, t->lm.n, B));
  s->ws.part = c.take<float>(pf);
  s->ws.part_floats = pf;
  s->ws.am_val = c.take<float>((size_t)am * 64);
  s->ws.am_idx = c.take<int>((size_t)am * 64);
  s->ws.am_cap = am;
  s->ws.logits_tmp = t->d.fmt == DFLASH_FMT_F32 ? c.take<float>((size_t)MAX_ROWS * t->d.vocab) : nullptr;
  // the overlap stream's GEMMs: the fc projection and every drafter layer's
  // k/v rows, B rows each
  {
    size_t pf2 = 1;
    auto need2 = [&](const GemmW& g) {
      const Plan p = make_plan(g.fmt, g.n, g.k, B, EPI_PARTIAL);
      pf2 = std::max(pf2, (size_t)p.S * B * g.n);
    };
    need2(d->fc);
    for (const Layer& L : d->layers) need2(kv_rows(L.qkv, d));
    s->ws2.part = c.take<float>(pf2);
    s->ws2.part_floats = pf2;
    s->ws2.am_val = nullptr; s->ws2.am_idx = nullptr; s->ws2.am_cap = 0; s->ws2.logits_tmp = nullptr;
    s->bu2 = c.take<char>((size_t)B * d->d.hidden * 4);
  }
  s->ybuf = c.take<int32_t>(64);
  const size_t sf = (size_t)t->n_gdn * t->d.gdn_heads * t->d.gdn_dv * t->d.gdn_dk;
  s->gdn_S = t->n_gdn ? c.take<float>(sf) : nullptr;
  s->gdn_snap = t->n_gdn ? c.take<float>(sf) : nullptr;
  s->gdn_tape = t->n_gdn ? c.take<float>((size_t)t->n_gdn * B * t->d.gdn_heads * gdn_rec(t)) : nullptr;
  s->dlog = c.take<float>((size_t)B * t->d.vocab);
  s->vlog = c.take<float>((size_t)B * t->d.vocab);
  s->lse = c.take<float>((size_t)2 * B);
}

static int setup_dims(dflash_state* s, const dflash_model* t, const dflash_model* d, int max_ctx, int block) {
  if (!t || !d) return fail(DFLASH_E_INVALID, "null model");
  if (d->target != t) return fail(DFLASH_E_INVALID, "the drafter is not bound to this target");
  if (block != 16 && block != 32) return fail(DFLASH_E_SHAPE, "block must be 16 or 32");
  if (max_ctx < 1) return fail(DFLASH_E_SHAPE, "max_ctx must be positive");
  s->t = t; s->dr = d; s->B = block; s->max_ctx = max_ctx;
  s->vrows = block; s->max_draft = 0;
  const int need = max_ctx + 2 * block;
  s->pages = (need + PAGE - 1) / PAGE;
  s->capacity = s->pages * PAGE;
  // 128-key splits in small states: there a 256-key split holds mostly
  // positions past the keys, and the halved staging and scores outweigh the
  // combine's extra partials (8B shapes, attention + combine a layer: 11.1
  // against 13.4 us at ctx 256, 13.2 against 15.1 at ctx 1024; 16.5 against
  // 15.8 at ctx 1536, where 256-key splits stay); and in block-16 states of
  // up to 32 such splits, whose query rows make a single row group a KV
  // head, so 256-key splits would leave most CUs idle (4B shapes at ctx
  // 2048: 11.4 against 13.0 us; block 32 keeps 256: 13.6 against 14.0 us)
  const bool small = s->capacity <= ATTN_SMALL_CAP || (block == 16 && s->capacity <= 32 * ATTN_SPLIT_SMALL);
  s->split = t->act != T_F32 && t->d.head_dim == 128 && small ? ATTN_SPLIT_SMALL : ATTN_SPLIT;
  s->max_splits = (s->capacity + s->split - 1) / s->split;
  if (s->max_splits > 32) return fail(DFLASH_E_CAPACITY, "max_ctx too large (at most 32 attention splits)");
  // dense prompt chunks: an int4 or bf16 target (the projections have the
  // dense kernel; GatedDeltaNet layers run the chunk's recurrence B tokens
  // at a time)
  s->pm = 0;
  if ((t->d.fmt == DFLASH_FMT_W4A16 || t->d.fmt == DFLASH_FMT_BF16) && t->act == T_BF16 && max_ctx > 2 * block) {
    bool ok = true;
    for (const Layer& L : t->layers)
      ok = ok && dense_ok(L.qkv.fmt, L.qkv.n, L.qkv.k, DENSE_PROMPT_ROWS, EPI_PARTIAL) &&
           dense_ok(L.o.fmt, L.o.n, L.o.k, DENSE_PROMPT_ROWS, EPI_PARTIAL) &&
           dense_ok(L.gu.fmt, L.gu.n, L.gu.k, DENSE_PROMPT_ROWS, EPI_SILU) &&
           dense_ok(L.down.fmt, L.down.n, L.down.k, DENSE_PROMPT_ROWS, EPI_PARTIAL);
    if (ok) s->pm = DENSE_PROMPT_ROWS;
  }
  // and the drafter's context pass of a chunk, if its projections have the
  // dense kernel too (else it runs B rows at a time)
  s->pm_draft = false;
  if (s->pm) {
    bool ok = dense_ok(d->fc.fmt, d->fc.n, d->fc.k, s->pm, EPI_PARTIAL);
    for (const Layer& L : d->layers) ok = ok && dense_ok(L.qkv.fmt, L.qkv.n, L.qkv.k, s->pm, EPI_PARTIAL);
    s->pm_draft = ok;
  }
  return DFLASH_OK;
}

extern "C" size_t dflash_state_bytes(const dflash_model* t, const dflash_model* d, int max_ctx, int block) {
  dflash_state s;
  if (setup_dims(&s, t, d, max_ctx, block) != DFLASH_OK) return 0;
  Carver c(nullptr);
  carve(&s, c);
  return c.off + 256;
}

extern "C" int dflash_state_init(dflash_state** out, const dflash_model* t, const dflash_model* d, void* arena,
                                 size_t arena_bytes, int max_ctx, int block) {
  if (!out || !arena) return fail(DFLASH_E_INVALID, "null out or arena");
  *out = nullptr;
  auto* s = new dflash_state();
  int rc = setup_dims(s, t, d, max_ctx, block);
  if (rc) { delete s; return rc; }
  Carver probe(nullptr);
  carve(s, probe);
  if (probe.off + 256 > arena_bytes) {
    delete s;
    return fail(DFLASH_E_CAPACITY, "arena too small: need " + std::to_string(probe.off + 256) + " bytes");
  }
  char* base = (char*)(((uintptr_t)arena + 255) & ~(uintptr_t)255);
  Carver c(base);
  carve(s, c);
  s->base = base;
  s->bytes = c.off;
  for (const Layer& L : d->layers) s->dkv.push_back(kv_rows(L.qkv, d));
  // zero the whole arena (KV pages are read whole: unwritten slots must be finite)
  hipError_t e = launch_fill_i32((int32_t*)base, c.off / 4, 0, nullptr);
  // RoPE table: angle pos * base^(-2i/d) in double, cos/sin rounded to fp32
  const int half = t->d.head_dim / 2;
  std::vector<float> cs((size_t)s->capacity * half), sn((size_t)s->capacity * half);
  for (int p = 0; p < s->capacity; ++p)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow(t->d.rope_base, -2.0 * i / t->d.head_dim);
      const double ang = (double)p * inv;
      cs[(size_t)p * half + i] = (float)std::cos(ang);
      sn[(size_t)p * half + i] = (float)std::sin(ang);
    }
  std::vector<int32_t> pt(s->pages);
  for (int i = 0; i < s->pages; ++i) pt[i] = i;     // pages handed out in order
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(s->cos_t, cs.data(), cs.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(s->sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(s->pt, pt.data(), pt.size() * 4, hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    delete s;
    return fail(DFLASH_E_DEVICE, std::string("state init: ") + hipGetErrorString(e));
  }
  *out = s;
  return DFLASH_OK;
}

extern "C" void dflash_state_destroy(dflash_state* s) {
  if (!s) return;
  for (auto& r : s->prof_recs) { hipEventDestroy(r.a); hipEventDestroy(r.b); }
  for (auto ev : s->ev_pool) hipEventDestroy(ev);
  if (s->ov_stream) {
    hipStreamSynchronize(s->ov_stream);
    hipStreamDestroy(s->ov_stream);
    hipEventDestroy(s->ov_fork);
    hipEventDestroy(s->ov_join);
  }
  delete s;
}

// ------------------------------------------------------------------ helpers
static hipEvent_t take_event(dflash_state* s) {
  if (!s->ev_pool.empty()) { hipEvent_t e = s->ev_pool.back(); s->ev_pool.pop_back(); return e; }
  hipEvent_t e = nullptr;
  hipEventCreate(&e);
  return e;
}

// Enqueue one GEMM.  PARTIAL launches return (in *parts) the partial sums
// the consuming kernel adds up.
static int gemm_ws(dflash_state* s, const Workspace& ws, int32_t* status, const GemmW& W, const void* x, int ldx,
                   int m, int epi, hipStream_t st, Parts* parts = nullptr, void* out = nullptr, int otype = 0,
                   float* logits = nullptr, int ldl = 0, int row0 = 0, int32_t* am_out = nullptr) {
  GemmCall c{};
  c.W = &W; c.x = x; c.ldx = ldx; c.m = m; c.epi = epi;
  c.part = ws.part; c.out = out; c.otype = otype;
  c.logits = logits; c.ldl = ldl; c.row0 = row0; c.am_out = am_out;
  c.status = status;
  const char* name = nullptr;
  double bytes = 0, io = 0;
  int S = 1;
  hipEvent_t ea = nullptr, eb = nullptr;
  if (s->prof) { ea = take_event(s); eb = take_event(s); hipEventRecord(ea, st); }
  hipError_t e = launch_gemm(c, ws, st, &name, &bytes, &S, &io);
  if (s->prof) { hipEventRecord(eb, st); s->prof_recs.push_back({name, bytes, io, ea, eb, c}); }
  if (e != hipSuccess) return fail(DFLASH_E_DEVICE, std::string("gemm: ") + hipGetErrorString(e));
  if (parts) *parts = Parts{ws.part, S, (size_t)m * W.n, W.n};
  return DFLASH_OK;
}

static int gemm(dflash_state* s, const GemmW& W, const void* x, int ldx, int m, int epi, hipStream_t st,
                Parts* parts = nullptr, void* out = nullptr, int otype = 0, float* logits = nullptr,
                int ldl = 0, int row0 = 0, int32_t* am_out = nullptr) {
  return gemm_ws(s, s->ws, s->scal + SC_STATUS, W, x, ldx, m, epi, st, parts, out, otype, logits, ldl, row0,
                 am_out);
}

#define RC(x) do { int rc_ = (x); if (rc_) return rc_; } while (0)

// Residual update with the pending partials (if any), then RMSNorm into out.
static int norm(dflash_state* s, const dflash_model* m, Pending& pend, const float* gain, void* out, int otype,
                int rows, hipStream_t st) {
  NormCall c{};
  c.mode = pend.in.p ? NORM_RESID : NORM_ONLY;
  c.in = pend.in;
  c.x = s->x; c.xtype = m->act; c.ldx = m->d.hidden;
  c.side = pend.side; c.side_type = pend.side_type; c.ld_side = pend.ld_side; c.side_col0 = pend.side_col0;
  c.gain = gain; c.eps = m->d.eps; c.h = m->d.hidden; c.rows = rows;
  c.out = out; c.otype = otype; c.ldo = m->d.hidden; c.tiled = 1;
  c.status = s->scal + SC_STATUS;
  HIPCHK(launch_norm(c, st));
  pend = Pending{};
  return DFLASH_OK;
}

// B = block rows of this pass: the whole block for a draft (plus as many
// context rows), the verify rows for a verify.
// ctx: a draft pass also projects the pending context rows (rows B..2B-1 of
// the QKV input); after_norm (if set) runs once the layer's first norm -- which
// completes the previous layer's residual and conditioning rows -- is enqueued.
static int attn_layer(dflash_state* s, const dflash_model* m, int l, const Layer& L, bool draft, Pending& pend,
                      int B, hipStream_t st, bool ctx = true, const std::function<int()>* after_norm = nullptr) {
  const int H = m->d.hidden, hq = m->d.n_q_heads, hkv = m->d.n_kv_heads, hd = m->d.head_dim;
  const bool with_ctx = draft && ctx;
  const int rows = with_ctx ? 2 * B : B;
  RC(norm(s, m, pend, L.in_norm, s->bu, m->gin, B, st));
  if (after_norm) RC((*after_norm)());
  Parts qkv;
  RC(gemm(s, L.qkv, s->bu, H, rows, EPI_PARTIAL, st, &qkv));
  RopeCall rc;
  rc.qkv = qkv; rc.atype = m->act;
  rc.block_rows = B; rc.ctx_rows = with_ctx ? B : 0;
  rc.dev_n = s->scal + SC_N; rc.dev_p = draft ? s->scal + SC_P : nullptr;
  rc.q_norm = L.q_norm; rc.k_norm = L.k_norm; rc.eps = m->d.eps;
  rc.cos_t = s->cos_t; rc.sin_t = s->sin_t; rc.q_out = s->bq;
  rc.kc = draft ? s->dk[l] : s->tk[l]; rc.vc = draft ? s->dv[l] : s->tv[l];
  rc.page_table = s->pt; rc.capacity = s->capacity; rc.hq = hq; rc.hkv = hkv; rc.d = hd;
  HIPCHK(launch_qk_rope(rc, st));
  AttnCall ac;
  ac.q = s->bq; ac.atype = m->act; ac.kc = rc.kc; ac.vc = rc.vc; ac.page_table = s->pt;
  ac.dev_n = s->scal + SC_N; ac.block_rows = B; ac.causal = draft ? 0 : 1;
  ac.hq = hq; ac.hkv = hkv; ac.d = hd; ac.max_splits = s->max_splits; ac.npages = s->pages; ac.split = s->split;
  ac.o_part = s->o_part; ac.ml_part = s->ml_part; ac.out = s->ba; ac.otype = m->gin; ac.ldo = hq * hd;
  ac.status = s->scal + SC_STATUS;
  HIPCHK(launch_attention(ac, st));
  RC(gemm(s, L.o, s->ba, hq * hd, B, EPI_PARTIAL, st, &pend.in));
  return DFLASH_OK;
}

// FFN block; the down projection's partials stay pending (with the side copy
// of the new residual for a conditioning layer) for the next norm.
static int ffn(dflash_state* s, const dflash_model* m, const Layer& L, Pending& pend, int B, hipStream_t st,
               void* side, int ld_side, int side_type, int side_col0) {
  const int H = m->d.hidden, F = m->d.ffn;
  RC(norm(s, m, pend, L.post_norm, s->bu, m->gin, B, st));
  RC(gemm(s, L.gu, s->bu, H, B, EPI_SILU, st, nullptr, s->bf, m->gin));
  RC(gemm(s, L.down, s->bf, F, B, EPI_PARTIAL, st, &pend.in));
  pend.side = side; pend.ld_side = ld_side; pend.side_type = side_type; pend.side_col0 = side_col0;
  return DFLASH_OK;
}

// Context projection of the rows the last verify committed -> QKV input rows
// B..2B-1 (whole 16-row blocks after the block rows of the tiled input).
static int draft_context(dflash_state* s, hipStream_t st, int side_row0 = 0, int rows = 0) {
  const dflash_model* d = s->dr;
  const int H = d->d.hidden, B = s->B;
  if (rows == 0) rows = B;
  // conditioning rows side_row0.. (whole 16-row blocks of the tiled input)
  const void* side = (const char*)s->side + (size_t)side_row0 * d->d.n_sel * H * elem_bytes(d->gin);
  Parts fc;
  RC(gemm(s, d->fc, side, d->d.n_sel * H, rows, EPI_PARTIAL, st, &fc));
  NormCall c{};
  c.mode = NORM_PROJ; c.in = fc; c.x = nullptr; c.xtype = d->act; c.ldx = H;
  c.gain = d->d.hidden_norm; c.eps = d->d.eps; c.h = H; c.rows = rows;
  c.out = (char*)s->bu + (size_t)B * H * elem_bytes(d->gin); c.otype = d->gin; c.ldo = H; c.tiled = 1;
  c.status = s->scal + SC_STATUS;
  HIPCHK(launch_norm(c, st));
  return DFLASH_OK;
}

// The part of a draft a prompt chunk needs: every drafter layer's K/V of the
// pending context rows, written to the drafter cache.  Each layer projects
// the same context rows (they do not pass through the layers), so the block
// rows, the attention, the FFNs and the lm-head are not run.  The block rows'
// cache slots the full draft would write are transient (the next context rows
// take them before any read).
// rows = the pending context rows (B, or a whole dense prompt chunk).
static int draft_context_kv(dflash_state* s, hipStream_t st, int side_row0 = 0, int rows = 0) {
  const dflash_model* d = s->dr;
  const int H = d->d.hidden, B = s->B;
  if (rows == 0) rows = B;
  RC(draft_context(s, st, side_row0, rows));
  const void* ctx_in = (const char*)s->bu + (size_t)B * H * elem_bytes(d->gin);
  for (int l = 0; l < d->d.n_layers; ++l) {
    const Layer& L = d->layers[l];
    Parts qkv;
    RC(gemm(s, L.qkv, ctx_in, H, rows, EPI_PARTIAL, st, &qkv));
    RopeCall rc;
    rc.qkv = qkv; rc.atype = d->act;
    rc.block_rows = 0; rc.ctx_rows = rows;   // partial row j = context row j
    rc.dev_n = s->scal + SC_N; rc.dev_p = s->scal + SC_P;
    rc.q_norm = L.q_norm; rc.k_norm = L.k_norm; rc.eps = d->d.eps;
    rc.cos_t = s->cos_t; rc.sin_t = s->sin_t; rc.q_out = s->bq;
    rc.kc = s->dk[l]; rc.vc = s->dv[l];
    rc.page_table = s->pt; rc.capacity = s->capacity;
    rc.hq = d->d.n_q_heads; rc.hkv = d->d.n_kv_heads; rc.d = d->d.head_dim;
    HIPCHK(launch_qk_rope(rc, st));
  }
  return DFLASH_OK;
}

// Draft/verify overlap (mirror-sd README, "How It Works": the drafter runs
// while the target verifies).  The part of the next draft that depends on the
// verify alone -- the drafter's context rows: the fc projection and hidden
// norm of every verify row's conditioning features, then each drafter
// layer's k/v of them with QK-norm and RoPE, written to the drafter cache at
// the rows' positions -- goes to the overlap stream as soon as the last
// conditioning layer's rows are complete, and runs while the target's last
// layers, the lm-head, the acceptance and the commit run on the caller's
// stream.  Rows past the accepted prefix land at positions that the next
// draft's block rows overwrite before any read, so the drafter cache the draft
// reads equals the sequential path's, and the draft then skips those rows.
static int overlap_ctx(dflash_state* s, int rows, hipStream_t st) {
  const dflash_model* d = s->dr;
  const int H = d->d.hidden;
  hipStream_t os = s->ov_stream;
  HIPCHK(hipEventRecord(s->ov_fork, st));
  HIPCHK(hipStreamWaitEvent(os, s->ov_fork, 0));
  s->ov_pending = true;
  int32_t* status = s->scal + SC_STATUS2;
  Parts fc;
  RC(gemm_ws(s, s->ws2, status, d->fc, s->side, d->d.n_sel * H, rows, EPI_PARTIAL, os, &fc));
  NormCall c{};
  c.mode = NORM_PROJ; c.in = fc; c.x = nullptr; c.xtype = d->act; c.ldx = H;
  c.gain = d->d.hidden_norm; c.eps = d->d.eps; c.h = H; c.rows = rows;
  c.out = s->bu2; c.otype = d->gin; c.ldo = H; c.tiled = 1;
  c.status = status;
  HIPCHK(launch_norm(c, os));
  for (int l = 0; l < d->d.n_layers; ++l) {
    const Layer& L = d->layers[l];
    Parts kv;
    RC(gemm_ws(s, s->ws2, status, s->dkv[l], s->bu2, H, rows, EPI_PARTIAL, os, &kv));
    RopeCall rc;
    rc.qkv = kv; rc.atype = d->act;
    rc.block_rows = 0; rc.ctx_rows = rows; rc.ctx_at_n = 1;   // row j at the verify's n + j
    rc.dev_n = s->scal + SC_VBASE; rc.dev_p = nullptr;
    rc.q_norm = L.q_norm; rc.k_norm = L.k_norm; rc.eps = d->d.eps;
    rc.cos_t = s->cos_t; rc.sin_t = s->sin_t; rc.q_out = nullptr;
    rc.kc = s->dk[l]; rc.vc = s->dv[l];
    rc.page_table = s->pt; rc.capacity = s->capacity;
    rc.hq = 0; rc.hkv = d->d.n_kv_heads; rc.d = d->d.head_dim;   // the k/v columns only
    HIPCHK(launch_qk_rope(rc, os));
  }
  HIPCHK(hipEventRecord(s->ov_join, os));
  s->ctx_ready = true;
  return DFLASH_OK;
}

// The caller's stream waits for the overlap work (if any is outstanding).
static int overlap_join(dflash_state* s, hipStream_t st) {
  if (!s->ov_pending) return DFLASH_OK;
  HIPCHK(hipStreamWaitEvent(st, s->ov_join, 0));
  s->ov_pending = false;
  return DFLASH_OK;
}

static int do_draft(dflash_state* s, int32_t* block, float* logits, hipStream_t st) {
  const dflash_model *t = s->t, *d = s->dr;
  const int H = d->d.hidden, B = s->B;
  RC(overlap_join(s, st));
  // the pending context rows, unless the overlap stream already wrote them
  const bool ctx = !(s->ov_on && s->ctx_ready);
  if (ctx) RC(draft_context(s, st));
  HIPCHK(launch_embed(t->d.embed, t->act, H, t->d.vocab, block, 1, d->d.mask_token, B, s->x, H,
                      s->scal + SC_STATUS, st));
  Pending pend;
  for (int l = 0; l < d->d.n_layers; ++l) {
    RC(attn_layer(s, d, l, d->layers[l], true, pend, B, st, ctx));
    RC(ffn(s, d, d->layers[l], pend, B, st, nullptr, 0, 0, 0));
  }
  RC(norm(s, d, pend, d->d.final_norm, s->bu, t->gin, B, st));
  const int V = t->d.vocab;
  if (s->temp > 0.f) {
    // slots 1..B-1 draw from softmax(z / T); their logits stay for the acceptance
    RC(gemm(s, t->lm, s->bu, H, B, EPI_ARGMAX, st, nullptr, nullptr, 0, s->dlog, V, 1, block + 1));
    HIPCHK(launch_sample_rows(s->dlog, V, V, B - 1, s->temp, s->seed, s->scal + SC_N, 0, 1, 0, block + 1, s->lse,
                              st));
    if (logits) HIPCHK(hipMemcpyAsync(logits, s->dlog, (size_t)(B - 1) * V * 4, hipMemcpyDeviceToDevice, st));
    return DFLASH_OK;
  }
  RC(gemm(s, t->lm, s->bu, H, B, EPI_ARGMAX, st, nullptr, nullptr, 0, logits, V, 1, block + 1));
  return DFLASH_OK;
}

// Target forward of rows 0..B-1 of block (B = s->B for prefill chunks, the
// verify rows otherwise).
// overlap: a block verify whose next draft's context rows go to the overlap
// stream (once the last conditioning layer's rows are complete)
static int do_verify(dflash_state* s, const int32_t* block, int32_t* argmax, float* logits, int B, hipStream_t st,
                     bool head = true, bool overlap = false) {
  const dflash_model *t = s->t, *d = s->dr;
  const int H = t->d.hidden;
  const int sel_last = d->d.n_sel ? d->d.sel_layers[d->d.n_sel - 1] : -1;
  const bool ov = overlap && sel_last >= 0;
  const std::function<int()> fork = [&]() { return overlap_ctx(s, B, st); };
  if (ov) HIPCHK(launch_copy_tokens(s->scal + SC_N, s->scal + SC_VBASE, 1, st));
  HIPCHK(launch_embed(t->d.embed, t->act, H, t->d.vocab, block, 0, 0, B, s->x, H, s->scal + SC_STATUS, st));
  Pending pend;
  int sel = 0, g = 0;
  for (int l = 0; l < t->d.n_layers; ++l) {
    const Layer& L = t->layers[l];
    // the first norm of the layer after the last conditioning layer completes
    // that layer's conditioning rows
    const std::function<int()>* hook = ov && l == sel_last + 1 ? &fork : nullptr;
    if (L.kind == DFLASH_LAYER_ATTN) {
      RC(attn_layer(s, t, l, L, false, pend, B, st, true, hook));
    } else {
      const int gh = t->d.gdn_heads, dkk = t->d.gdn_dk, dvv = t->d.gdn_dv;
      RC(norm(s, t, pend, L.in_norm, s->bu, t->gin, B, st));
      if (hook) RC((*hook)());
      GdnCall gc;
      RC(gemm(s, L.qkv, s->bu, H, B, EPI_PARTIAL, st, &gc.proj));
      gc.atype = t->act; gc.rows = B; gc.gh = gh; gc.dk = dkk; gc.dv = dvv;
      gc.S = s->gdn_S + (size_t)g * gh * dvv * dkk;
      gc.tape = s->gdn_tape + (size_t)g * s->B * gh * gdn_rec(t);   // tape rows are laid out per B
      gc.out = s->ba; gc.otype = t->gin; gc.ldo = gh * dvv;
      gc.status = s->scal + SC_STATUS;
      if (B <= s->B) {
        HIPCHK(launch_gdn_verify(gc, st));
      } else {
        // a prompt chunk (whole blocks, all committed): block after block,
        // the block-path verify from the layer's state, then the pinned
        // replay of all of the block's tokens into it, so that the state and
        // outputs are the ones B-row prefill chunks give; the chunk's commit
        // then skips the replay
        HIPCHK(launch_gdn_prompt(gc, s->B, st));
      }
      RC(gemm(s, L.o, s->ba, gh * dvv, B, EPI_PARTIAL, st, &pend.in));
      ++g;
    }
    void* side = nullptr;
    int col0 = 0;
    if (sel < d->d.n_sel && d->d.sel_layers[sel] == l) {
      side = s->side;                  // conditioning rows: columns sel*H.. of the fc input
      col0 = sel * H;
      ++sel;
    }
    RC(ffn(s, t, L, pend, B, st, side, d->d.n_sel * H, d->gin, col0));
  }
  // (this norm also completes the last layer's residual update, which writes
  // its conditioning rows when that layer is a selected one)
  RC(norm(s, t, pend, t->d.final_norm, s->bu, t->gin, B, st));
  if (ov && sel_last == t->d.n_layers - 1) RC(fork());
  // a prompt chunk before the last needs only the caches, the GatedDeltaNet
  // state and the conditioning rows: no logits
  if (!head) return DFLASH_OK;
  const int V = t->d.vocab;
  if (s->temp > 0.f) {
    // the acceptance reads the target's tempered distributions of these rows
    RC(gemm(s, t->lm, s->bu, H, B, EPI_ARGMAX, st, nullptr, nullptr, 0, s->vlog, V, 0, argmax));
    if (logits) HIPCHK(hipMemcpyAsync(logits, s->vlog, (size_t)B * V * 4, hipMemcpyDeviceToDevice, st));
    return DFLASH_OK;
  }
  RC(gemm(s, t->lm, s->bu, H, B, EPI_ARGMAX, st, nullptr, nullptr, 0, logits, V, 0, argmax));
  return DFLASH_OK;
}

// gdn_done: the GatedDeltaNet states already hold the committed tokens (a
// prompt chunk replays them block by block in its forward pass)
static int do_commit(dflash_state* s, const int32_t* d_acc, int host_count, const int32_t* emit, hipStream_t st,
                     bool gdn_done = false) {
  const dflash_model* t = s->t;
  if (t->n_gdn && !gdn_done)
    HIPCHK(launch_gdn_replay(s->gdn_S, s->gdn_tape, t->n_gdn, s->B, t->d.gdn_heads, t->d.gdn_dk, t->d.gdn_dv,
                             d_acc, host_count, s->scal, s->capacity, st));
  HIPCHK(launch_commit(s->scal, d_acc, host_count, emit, s->tokens, s->acc_log, s->acc_log_len, s->capacity,
                       s->B, st));
  return DFLASH_OK;
}

// ------------------------------------------------------------------ ABI
extern "C" int dflash_prefill(dflash_state* s, const int32_t* d_tokens, int n_tokens, int32_t* d_first,
                              void* stream) {
  if (!s || !d_tokens || !d_first) return fail(DFLASH_E_INVALID, "null argument");
  if (n_tokens < 1) return fail(DFLASH_E_SHAPE, "empty prompt");
  if (n_tokens + 2 * s->B > s->capacity || n_tokens > s->max_ctx)
    return fail(DFLASH_E_CAPACITY, "prompt longer than the state's max_ctx");
  hipStream_t st = (hipStream_t)stream;
  const dflash_model* t = s->t;
  RC(overlap_join(s, st));
  HIPCHK(launch_set_scalars(s->scal, 0, 0, 1, st));
  HIPCHK(launch_copy_tokens(d_tokens, s->tokens, n_tokens, st));
  if (t->n_gdn)
    HIPCHK(launch_fill_i32((int32_t*)s->gdn_S,
                           (size_t)t->n_gdn * t->d.gdn_heads * t->d.gdn_dv * t->d.gdn_dk, 0, st));
  int last = 0, c0 = 0;
  // Without GatedDeltaNet layers and with a dense drafter pass, the whole
  // prompt runs as chunks (the last one padded to a whole 16-row group); the
  // first token is the argmax of the last row, from the lm-head over its
  // 16-row group, and the drafter's context rows are committed in two parts
  // (up to that group, then the group's valid rows), as B-row chunks would.
  // Otherwise the whole blocks before the one holding the last token run as
  // chunks and that block takes the block path.
  const bool fold = s->pm > 0 && s->pm_draft && t->n_gdn == 0;
  if (fold) {
    const int H = t->d.hidden;
    while (c0 < n_tokens) {
      const int valid = std::min(s->pm, n_tokens - c0);
      if (c0 + valid < n_tokens) {           // a full chunk (pm rows, a multiple of B)
        RC(do_verify(s, s->tokens + c0, s->ybuf, nullptr, valid, st, false));
        RC(do_commit(s, nullptr, valid, nullptr, st));
        RC(draft_context_kv(s, st, 0, valid));
        c0 += valid;
        continue;
      }
      const int rows = (valid + 15) / 16 * 16, tail0 = (valid - 1) / 16 * 16;
      last = valid - tail0;
      RC(do_verify(s, s->tokens + c0, s->ybuf, nullptr, rows, st, false));
      // the last row's logits: lm-head over its 16-row group of the final norm
      const void* xh = (const char*)s->bu + (size_t)tail0 * H * elem_bytes(t->gin);
      RC(gemm(s, t->lm, xh, H, 16, EPI_ARGMAX, st, nullptr, nullptr, 0, s->temp > 0.f ? s->vlog : nullptr,
              t->d.vocab, 0, s->ybuf));
      if (tail0 > 0) {
        RC(do_commit(s, nullptr, tail0, nullptr, st));
        RC(draft_context_kv(s, st, 0, tail0));
      }
      RC(do_commit(s, nullptr, last, nullptr, st));
      // the group's context rows (rows past the prompt go to slots past n,
      // which the next rows overwrite before any read)
      RC(draft_context_kv(s, st, tail0, 16));
      c0 = n_tokens;
    }
  } else if (s->pm > 0) {
    // the whole blocks before the one holding the last token run as dense
    // chunks of up to pm rows; their drafter context rows then go in B at a
    // time (the commit of each block makes it the pending context)
    const int dense_end = ((n_tokens - 1) / s->B) * s->B;
    while (c0 < dense_end) {
      const int rows = std::min(s->pm, dense_end - c0);
      RC(do_verify(s, s->tokens + c0, s->ybuf, nullptr, rows, st, false));
      const bool gdn_done = rows > s->B;
      if (s->pm_draft) {
        RC(do_commit(s, nullptr, rows, nullptr, st, gdn_done));
        RC(draft_context_kv(s, st, 0, rows));
      } else {
        for (int j = 0; j < rows; j += s->B) {
          RC(do_commit(s, nullptr, s->B, nullptr, st, gdn_done));
          RC(draft_context_kv(s, st, j));
        }
      }
      c0 += rows;
    }
  }
  for (; c0 < n_tokens; c0 += s->B) {
    const int len = std::min(s->B, n_tokens - c0);
    // only the last chunk's last row is read: the first token (logits land in
    // vlog when sampling)
    const bool final_chunk = c0 + s->B >= n_tokens;
    RC(do_verify(s, s->tokens + c0, s->ybuf, nullptr, s->B, st, final_chunk));
    RC(do_commit(s, nullptr, len, nullptr, st));
    RC(draft_context_kv(s, st));                   // the chunk's drafter context rows
    last = len;
  }
  if (s->temp > 0.f)   // the first token is a draw from the last prompt row at T (stream 3, counter (P, 0))
    HIPCHK(launch_sample_rows(s->vlog + (size_t)(last - 1) * t->d.vocab, t->d.vocab, t->d.vocab, 1, s->temp,
                              s->seed, nullptr, n_tokens, 0, 3, s->ybuf + last - 1, nullptr, st));
  HIPCHK(launch_copy_tokens(s->ybuf + last - 1, s->tokens + n_tokens, 1, st));
  HIPCHK(launch_copy_tokens(s->ybuf + last - 1, d_first, 1, st));
  HIPCHK(launch_set_scalars(s->scal, -1, 0, 0, st));
  s->snap_n = -1;
  s->ctx_ready = true;            // every prompt row's context is in the drafter cache
  return DFLASH_OK;
}

extern "C" int dflash_draft_block(dflash_state* s, int32_t* d_block, float* d_logits, void* stream) {
  if (!s || !d_block) return fail(DFLASH_E_INVALID, "null argument");
  return do_draft(s, d_block, d_logits, (hipStream_t)stream);
}

extern "C" int dflash_verify_block(dflash_state* s, const int32_t* d_block, int32_t* d_argmax, float* d_logits,
                                   void* stream) {
  if (!s || !d_block || !d_argmax) return fail(DFLASH_E_INVALID, "null argument");
  hipStream_t st = (hipStream_t)stream;
  RC(overlap_join(s, st));
  s->ctx_ready = false;
  return do_verify(s, d_block, d_argmax, d_logits, s->vrows, st, true, s->ov_on);
}

extern "C" int dflash_set_overlap(dflash_state* s, int on) {
  if (!s) return fail(DFLASH_E_INVALID, "null state");
  if (on && !s->ov_stream) {
    hipStream_t os = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&os, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (os) hipStreamDestroy(os);
      if (f) hipEventDestroy(f);
      return fail(DFLASH_E_DEVICE, std::string("overlap stream: ") + hipGetErrorString(e));
    }
    s->ov_stream = os; s->ov_fork = f; s->ov_join = j;
  }
  s->ov_on = on != 0;
  return DFLASH_OK;
}

// Draft cap (mlx-dspark v0.0.3 "Highlights" and "API", --max-draft): verify
// only the first N = min(max_draft, B-1) drafts (0 = the whole block).  The
// verify then runs V >= N+1 rows, V the smallest multiple of the attention
// row quantum (16 query rows of one KV head per MFMA block) not below N+1;
// the caller accepts over N+1 rows.
extern "C" int dflash_set_max_draft(dflash_state* s, int max_draft, int* h_verify_rows, int* h_accept_block) {
  if (!s) return fail(DFLASH_E_INVALID, "null state");
  if (max_draft < 0) return fail(DFLASH_E_SHAPE, "max_draft must be >= 0");
  const int N = max_draft == 0 ? s->B - 1 : std::min(max_draft, s->B - 1);
  // the target's MFMA attention takes G*V query rows per KV head in 16-row
  // blocks (G query heads per KV head); the fp32 attention has no quantum
  int q = 1;
  if (s->t->act != T_F32) {
    const int G = s->t->d.n_q_heads / s->t->d.n_kv_heads;
    while ((G * q) % 16) ++q;
  }
  const int V = std::min(s->B, (N + 1 + q - 1) / q * q);
  s->max_draft = max_draft;
  s->vrows = V;
  if (h_verify_rows) *h_verify_rows = V;
  if (h_accept_block) *h_accept_block = N + 1;
  return DFLASH_OK;
}

// Temperature sampling (mlx-dspark v0.0.3 "Highlights": --temperature T > 0
// is an exact sample of the target at T).
extern "C" int dflash_set_sampling(dflash_state* s, float temperature, uint64_t seed) {
  if (!s) return fail(DFLASH_E_INVALID, "null state");
  if (!(temperature >= 0.f) || !std::isfinite(temperature))
    return fail(DFLASH_E_SHAPE, "temperature must be finite and >= 0");
  s->temp = temperature;
  s->seed = seed;
  return DFLASH_OK;
}

extern "C" int dflash_accept_sampled(dflash_state* s, const int32_t* d_block, int32_t* d_accept, int32_t* d_emit,
                                     int32_t* d_next_anchor, void* stream) {
  if (!s || !d_block || !d_accept || !d_emit) return fail(DFLASH_E_INVALID, "null argument");
  if (!(s->temp > 0.f)) return fail(DFLASH_E_UNSUPPORTED, "sampling is off (temperature 0): use dflash_accept");
  hipStream_t st = (hipStream_t)stream;
  const int V = s->t->d.vocab;
  const int N = s->max_draft == 0 ? s->B - 1 : std::min(s->max_draft, s->B - 1);
  HIPCHK(launch_sample_rows(s->vlog, V, V, N + 1, s->temp, s->seed, s->scal + SC_N, 0, 0, -1, nullptr,
                            s->lse + s->B, st));
  HIPCHK(launch_spec_accept(d_block, s->dlog, s->vlog, V, N, s->lse, s->lse + s->B, s->temp, s->seed,
                            s->scal + SC_N, 0, s->B, d_accept, d_emit, d_next_anchor, st));
  return DFLASH_OK;
}

extern "C" int dflash_sample_logits(const float* d_logits, int ld, int rows, int vocab, float temperature,
                                    uint64_t seed, int n, int row0, int stream_id, int32_t* d_tokens, float* d_lse,
                                    void* stream) {
  if (!d_logits || (!d_tokens && stream_id >= 0)) return fail(DFLASH_E_INVALID, "null argument");
  if (rows < 0 || vocab < 1 || ld < vocab || n < 0 || row0 < 0 || stream_id > 3)
    return fail(DFLASH_E_SHAPE, "bad shape or counter");
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return fail(DFLASH_E_SHAPE, "temperature must be > 0");
  HIPCHK(launch_sample_rows(d_logits, ld, vocab, rows, temperature, seed, nullptr, n, row0, stream_id, d_tokens,
                            d_lse, (hipStream_t)stream));
  return DFLASH_OK;
}

extern "C" int dflash_accept_logits(const int32_t* d_block, const float* d_dlog, const float* d_vlog, int vocab,
                                    int n_drafts, int block, float temperature, uint64_t seed, int n,
                                    float* d_lse, int32_t* d_accept, int32_t* d_emit, int32_t* d_next_anchor,
                                    void* stream) {
  if (!d_block || !d_dlog || !d_vlog || !d_lse || !d_accept || !d_emit) return fail(DFLASH_E_INVALID, "null argument");
  if (vocab < 1 || n < 0 || block < 2 || block > 64 || n_drafts < 1 || n_drafts >= block)
    return fail(DFLASH_E_SHAPE, "need 1 <= n_drafts < block <= 64");
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return fail(DFLASH_E_SHAPE, "temperature must be > 0");
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(launch_sample_rows(d_dlog, vocab, vocab, n_drafts, temperature, seed, nullptr, n, 1, -1, nullptr, d_lse, st));
  HIPCHK(launch_sample_rows(d_vlog, vocab, vocab, n_drafts + 1, temperature, seed, nullptr, n, 0, -1, nullptr,
                            d_lse + block, st));
  HIPCHK(launch_spec_accept(d_block, d_dlog, d_vlog, vocab, n_drafts, d_lse, d_lse + block, temperature, seed,
                            nullptr, n, block, d_accept, d_emit, d_next_anchor, st));
  return DFLASH_OK;
}

extern "C" int dflash_accept(const int32_t* d_block, const int32_t* d_argmax, int block, int32_t* d_accept,
                             int32_t* d_emit, int32_t* d_next_anchor, void* stream) {
  if (!d_block || !d_argmax || !d_accept || !d_emit) return fail(DFLASH_E_INVALID, "null argument");
  if (block < 2 || block > 64) return fail(DFLASH_E_SHAPE, "block must be in [2, 64]");
  HIPCHK(launch_accept(d_block, d_argmax, block, d_accept, d_emit, d_next_anchor, (hipStream_t)stream));
  return DFLASH_OK;
}

extern "C" int dflash_kv_commit(dflash_state* s, const int32_t* d_accept, const int32_t* d_emit, void* stream) {
  if (!s || !d_accept) return fail(DFLASH_E_INVALID, "null argument");
  hipStream_t st = (hipStream_t)stream;
  RC(do_commit(s, d_accept, 0, d_emit, st));
  // the step ends with the overlap work joined, so that a captured step is
  // self-contained
  return overlap_join(s, st);
}

static int read_scalars(dflash_state* s, int32_t* h, hipStream_t st) {
  HIPCHK(hipStreamSynchronize(st));
  if (s->ov_stream) HIPCHK(hipStreamSynchronize(s->ov_stream));
  HIPCHK(hipMemcpy(h, s->scal, SC_COUNT * sizeof(int32_t), hipMemcpyDeviceToHost));
  h[SC_STATUS] |= h[SC_STATUS2];
  return DFLASH_OK;
}

extern "C" int dflash_kv_rollback(dflash_state* s, int new_len, int32_t* d_block, void* stream) {
  if (!s) return fail(DFLASH_E_INVALID, "null state");
  hipStream_t st = (hipStream_t)stream;
  RC(overlap_join(s, st));
  int32_t h[SC_COUNT];
  RC(read_scalars(s, h, st));
  if (new_len < 1 || new_len > h[SC_N]) return fail(DFLASH_E_SHAPE, "rollback length outside [1, n]");
  if (s->t->n_gdn) {
    if (s->snap_n != new_len)
      return fail(DFLASH_E_UNSUPPORTED, "GatedDeltaNet rollback needs a snapshot taken at that length");
    const size_t sf = (size_t)s->t->n_gdn * s->t->d.gdn_heads * s->t->d.gdn_dv * s->t->d.gdn_dk;
    HIPCHK(launch_copy_f32(s->gdn_snap, s->gdn_S, sf, st));
  }
  HIPCHK(launch_rollback(s->scal, new_len, s->tokens, d_block, st));
  s->ctx_ready = true;            // no pending context rows: positions < new_len are in the cache
  return DFLASH_OK;
}

extern "C" int dflash_gdn_snapshot(dflash_state* s, void* stream) {
  if (!s) return fail(DFLASH_E_INVALID, "null state");
  hipStream_t st = (hipStream_t)stream;
  int32_t h[SC_COUNT];
  RC(read_scalars(s, h, st));
  if (s->t->n_gdn) {
    const size_t sf = (size_t)s->t->n_gdn * s->t->d.gdn_heads * s->t->d.gdn_dv * s->t->d.gdn_dk;
    HIPCHK(launch_copy_f32(s->gdn_S, s->gdn_snap, sf, st));
  }
  s->snap_n = h[SC_N];
  return DFLASH_OK;
}

extern "C" int dflash_inject(dflash_state* s, int32_t* d_block, const int32_t* d_ref, int ref_len,
                             const int32_t* d_sched, int n_sched, const int32_t* d_filler, void* stream) {
  if (!s || !d_block || !d_ref || !d_sched || !d_filler) return fail(DFLASH_E_INVALID, "null argument");
  if (n_sched < 1 || ref_len < 1) return fail(DFLASH_E_SHAPE, "empty schedule or reference");
  HIPCHK(launch_inject(s->scal, d_block, s->B, d_ref, ref_len, d_sched, n_sched, d_filler, s->t->d.vocab,
                       (hipStream_t)stream));
  return DFLASH_OK;
}

extern "C" int dflash_state_query(dflash_state* s, int32_t* h_out, void* stream) {
  if (!s || !h_out) return fail(DFLASH_E_INVALID, "null argument");
  int32_t h[SC_COUNT];
  RC(read_scalars(s, h, (hipStream_t)stream));
  h_out[0] = h[SC_N];
  h_out[1] = h[SC_STEP];
  h_out[2] = h[SC_STATUS];
  h_out[3] = h[SC_P];
  return DFLASH_OK;
}

extern "C" int dflash_state_buffers(dflash_state* s, dflash_state_view* v) {
  if (!s || !v) return fail(DFLASH_E_INVALID, "null argument");
  v->tokens = s->tokens;
  v->acc_log = s->acc_log;
  v->acc_log_len = s->acc_log_len;
  v->side = s->side;
  v->ctx_feat = (char*)s->bu + (size_t)s->B * s->dr->d.hidden * elem_bytes(s->dr->gin);
  v->gdn_state = s->gdn_S;
  v->gdn_tape = s->gdn_tape;
  v->tape_stride = gdn_rec(s->t);
  v->n_gdn = s->t->n_gdn;
  v->capacity = s->capacity;
  return DFLASH_OK;
}

extern "C" int dflash_prof_enable(dflash_state* s, int on) {
  if (!s) return fail(DFLASH_E_INVALID, "null state");
  if (on && !s->prof) {
    for (auto& r : s->prof_recs) { s->ev_pool.push_back(r.a); s->ev_pool.push_back(r.b); }
    s->prof_recs.clear();
  }
  s->prof = on != 0;
  return DFLASH_OK;
}

extern "C" int dflash_prof_replay(dflash_state* s, const char* variant, int reps, void* stream, double* h_ms,
                                  int64_t* h_launches) {
  if (!s || !variant || !h_ms || !h_launches || reps < 1) return fail(DFLASH_E_INVALID, "bad argument");
  std::vector<const GemmCall*> calls;
  for (auto& r : s->prof_recs)
    if (std::strcmp(r.name, variant) == 0) calls.push_back(&r.call);
  *h_ms = 0;
  *h_launches = 0;
  if (calls.empty()) return DFLASH_OK;
  hipStream_t st = (hipStream_t)stream;
  hipEvent_t ea = take_event(s), eb = take_event(s);
  HIPCHK(hipEventRecord(ea, st));
  for (int r = 0; r < reps; ++r)
    for (const GemmCall* c : calls) {
      const char* nm = nullptr;
      hipError_t e = launch_gemm(*c, s->ws, st, &nm, nullptr, nullptr);
      if (e != hipSuccess) return fail(DFLASH_E_DEVICE, std::string("gemm replay: ") + hipGetErrorString(e));
    }
  HIPCHK(hipEventRecord(eb, st));
  HIPCHK(hipEventSynchronize(eb));
  float e = 0.f;
  HIPCHK(hipEventElapsedTime(&e, ea, eb));
  s->ev_pool.push_back(ea);
  s->ev_pool.push_back(eb);
  *h_ms = e;
  *h_launches = (int64_t)calls.size() * reps;
  return DFLASH_OK;
}

namespace dfl {
hipError_t launch_read_floor(const void* buf, size_t bytes, int nwg, uint32_t* sink, hipStream_t s);
hipError_t launch_bf16_round_check(unsigned long long* counts, hipStream_t s);
}

extern "C" int dflash_read_floor(const void* d_buf, size_t bytes, int copies, int nwg, int reps, uint32_t* d_sink,
                                 void* stream, double* h_ms) {
  if (!d_buf || !d_sink || !h_ms || copies < 1 || reps < 1 || nwg < 1 || nwg > 65536 || bytes == 0 || bytes % 16)
    return fail(DFLASH_E_INVALID, "bad argument");
  hipStream_t st = (hipStream_t)stream;
  hipEvent_t ea, eb;
  HIPCHK(hipEventCreate(&ea));
  HIPCHK(hipEventCreate(&eb));
  HIPCHK(launch_read_floor(d_buf, bytes, nwg, d_sink, st));           // warm-up launch
  HIPCHK(hipEventRecord(ea, st));
  for (int r = 0; r < reps; ++r)
    for (int c = 0; c < copies; ++c) HIPCHK(launch_read_floor((const char*)d_buf + (size_t)c * bytes, bytes, nwg, d_sink, st));
  HIPCHK(hipEventRecord(eb, st));
  HIPCHK(hipEventSynchronize(eb));
  float ms = 0.f;
  HIPCHK(hipEventElapsedTime(&ms, ea, eb));
  hipEventDestroy(ea);
  hipEventDestroy(eb);
  *h_ms = ms;
  return DFLASH_OK;
}

extern "C" int dflash_prof_read(dflash_state* s, const char** names, int64_t* launches, double* ms, double* bytes,
                                double* io_bytes, int cap, int* h_n) {
  if (!s || !h_n) return fail(DFLASH_E_INVALID, "null argument");
  std::vector<const char*> nm;
  std::vector<int64_t> cnt;
  std::vector<double> tms, tb, tio;
  for (auto& r : s->prof_recs) {
    HIPCHK(hipEventSynchronize(r.b));
    float e = 0.f;
    HIPCHK(hipEventElapsedTime(&e, r.a, r.b));
    size_t i = 0;
    while (i < nm.size() && std::strcmp(nm[i], r.name) != 0) ++i;
    if (i == nm.size()) { nm.push_back(r.name); cnt.push_back(0); tms.push_back(0); tb.push_back(0); tio.push_back(0); }
    cnt[i] += 1;
    tms[i] += e;
    tb[i] += r.bytes;
    tio[i] += r.io_bytes;
  }
  *h_n = (int)nm.size();
  for (int i = 0; i < (int)nm.size() && i < cap; ++i) {
    if (names) names[i] = nm[i];
    if (launches) launches[i] = cnt[i];
    if (ms) ms[i] = tms[i];
    if (bytes) bytes[i] = tb[i];
    if (io_bytes) io_bytes[i] = tio[i];
  }
  return DFLASH_OK;
}

extern "C" int dflash_check_bf16_rounding(uint64_t* d_counts, void* stream, uint64_t* h_counts) {
  if (!d_counts || !h_counts) return fail(DFLASH_E_INVALID, "bad argument");
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(launch_fill_i32((int32_t*)d_counts, 4, 0, st));
  HIPCHK(launch_bf16_round_check((unsigned long long*)d_counts, st));
  HIPCHK(hipMemcpyAsync(h_counts, d_counts, 2 * sizeof(uint64_t), hipMemcpyDeviceToHost, st));
  HIPCHK(hipStreamSynchronize(st));
  return DFLASH_OK;
}
