/*
 * dflash.h -- C ABI of the DFlash draft+verify step on MI355X (gfx950).
 *
 * One step of DFlash block-diffusion speculative decoding:
 *   draft   a small drafter, conditioned on projected intermediate hidden
 *           states of the target and sharing the target's embedding and
 *           lm-head, denoises a whole block of B slots in ONE parallel pass
 *           (mlx-dspark v0.0.3 notes, "Highlights"; dflash-mlx note,
 *           "How it works" and "Technical challenges");
 *   verify  the target runs the block in one batched forward and takes the
 *           argmax of every row (mirror-sd README, "How It Works" step 1);
 *   accept  the longest prefix of drafts equal to the target's argmax is
 *           kept, plus one correction token (mirror-sd README, "How It
 *           Works" step 3; agentlens dflash-mlx summary, "How it works");
 *   commit  the KV cache keeps the accepted positions and drops the rest;
 *           GatedDeltaNet layers restore their state by replaying a tape
 *           recorded during verify (dflash-mlx note, "Technical challenges").
 *
 * Conventions for every function below:
 *   - All functions are extern "C", never throw, and return DFLASH_OK (0) or
 *     a negative DFLASH_E_* code; dflash_last_error() gives a message.
 *   - Argument and shape errors are detected on the host, before any launch.
 *   - "d_" pointers are device pointers; "h_" pointers are host pointers.
 *   - Hot-path calls (draft, verify, accept, commit, inject) only enqueue
 *     kernels on the given stream: no host synchronisation, no allocation.
 *     Lengths that change per step (n, accepted count a) live in device
 *     memory, so a captured hipGraph of a step can be replayed.
 *   - The library never allocates device memory.  The caller owns the
 *     weights, the state arena and all I/O buffers and keeps them alive
 *     until the objects that reference them are destroyed.
 *   - Device-side faults found while running (context capacity exceeded,
 *     token id out of range) set a status word in the arena instead of
 *     trapping; dflash_state_status() reads it.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DFLASH_OK = 0,
  DFLASH_E_INVALID = -1,     /* bad argument (null pointer, bad enum) */
  DFLASH_E_SHAPE = -2,       /* dimensions the kernels do not support */
  DFLASH_E_CAPACITY = -3,    /* arena too small / context capacity exceeded */
  DFLASH_E_DEVICE = -4,      /* HIP error (no device, launch failure) */
  DFLASH_E_UNSUPPORTED = -5  /* valid request the library does not implement */
};

/* Weight formats. Activations are fp32 for DFLASH_FMT_F32 models and bf16
 * for the others (mirror-sd README, "The Story": W8A16 = int8 weights with
 * per-channel fp16 scales, 16-bit activations; "Results": 4-bit target). */
enum {
  DFLASH_FMT_F32 = 0,        /* fp32 [N][K] row-major */
  DFLASH_FMT_BF16 = 1,       /* bf16 [N][K] */
  DFLASH_FMT_W8A16 = 2,      /* int8 codes [N][K], fp16 scale per row n */
  DFLASH_FMT_W4A16 = 3       /* int4 codes [N][K] in [-8,7], fp16 scale per (n, 64-wide K group) */
};

enum { DFLASH_LAYER_ATTN = 0, DFLASH_LAYER_GDN = 1 };

enum {                       /* device status word bits */
  DFLASH_STATUS_CAPACITY = 1,    /* a commit would pass the context capacity; it was skipped */
  DFLASH_STATUS_TOKEN_RANGE = 2, /* a token id outside [0, vocab) was clamped */
  DFLASH_STATUS_ACT_RANGE = 4    /* W8A16 / W4A16 stacks: a bf16 activation feeding an fp16 GEMM
                                    input (RMSNorm output, residual row of a conditioning layer,
                                    attention or GatedDeltaNet output, SiLU*mul output) was NaN
                                    or larger than 65504 in magnitude, where its fp16 encoding is
                                    inf; the results of that step are not valid.  (Magnitudes
                                    below 2^-17 are rounded to the fp16 subnormal grid, an
                                    absolute error of at most 2^-25; they are not flagged.) */
};

const char *dflash_last_error(void);   /* message of this thread's last failure */
int dflash_device_count(int *h_count); /* number of visible HIP devices */

/* ------------------------------------------------------------- weights
 * Packed device layout of one linear layer Y = X W^T (W is [N][K]).
 * The kernels read weights in a private tile-major order so that every
 * 64-lane load is one contiguous 1 KiB block; dflash_pack_weight converts a
 * canonical [N][K] matrix into it on the device.
 *
 * dflash_packed_bytes: sizes of the packed weight and scale buffers.
 *   N % 16 == 0; K % 128 == 0 for W4A16, K % 64 for W8A16, K % 32 for BF16,
 *   any K for F32.  gate_up != 0 packs a fused [gate; up] matrix (rows
 *   0..N/2-1 gate, N/2..N-1 up) so that matching gate/up rows sit in the
 *   same tile pair (needed by the fused SiLU*mul epilogue); then N % 32 == 0.
 * dflash_pack_weight: src_codes is float [N][K] (F32), bf16 bits uint16
 *   [N][K] (BF16) or int8 [N][K] (W8A16 codes in [-127,127], W4A16 codes in
 *   [-8,7]); src_scales is fp16 [N] (W8A16), fp16 [N][K/64] (W4A16) or NULL.
 *   dst / dst_scales must hold dflash_packed_bytes bytes.  Asynchronous on
 *   stream; the sources may be freed after the stream has passed the call. */
int dflash_packed_bytes(int fmt, int n, int k, size_t *h_weight_bytes, size_t *h_scale_bytes);
int dflash_pack_weight(int fmt, int n, int k, int gate_up, const void *d_src_codes,
                       const void *d_src_scales, void *d_dst, void *d_dst_scales, void *stream);

/* Apply one packed linear layer on its own: Y = X W^T, the GEMM behind every
 * projection of the step (same kernels, same split plan).
 *   d_x      activations X[m][k], 1 <= m <= 64, in the GEMM-input encoding
 *            of the format: fp32 row-major [m][ldx] (F32, ldx >= k); for the
 *            16-bit formats (bf16 for BF16, fp16 codes of bf16 values for
 *            W8A16 / W4A16) the tiled layout the library's own producers
 *            write: ceil(m/16) blocks of 16 rows, element (t, j) at
 *              ((t/16)*(k/32) + j/32)*512 + ((t%16) + 16*((j%32)/8))*8 + j%8
 *            (every 32-column step of a block is one contiguous 1 KiB MFMA
 *            operand); ldx is ignored there.
 *   epilogue 0: d_out = Y as fp32 [m][n] (not rounded);
 *            1: d_argmax[i] = argmax_j Y[i][j] (lowest index on ties) and, if
 *               d_out is not NULL, the fp32 logits Y [m][n].
 *   d_ws     device workspace of dflash_linear_workspace_bytes(fmt,n,k,m)
 *            bytes, zero-filled once before first use (every call leaves its
 *            counters zero again).
 *   Prompt chunks: BF16, W8A16 and W4A16 (K % 128 == 0) with epilogue 0
 *            also take m = 80, 96, ..., 1024 (multiples of 16 above 64).
 *            These run the dense kernel prefill uses (activations staged in
 *            LDS and reused across 256 weight rows; same exact
 *            dequantisation: fp16 MFMA on the raw codes, one fp32 sum per
 *            64-wide group times its scale for W4, the row scale on the
 *            finished sum for W8; bf16 MFMA on the stored weights for BF16).
 * Errors: SHAPE for unsupported dims, INVALID for null pointers or an
 * undersized workspace. */
size_t dflash_linear_workspace_bytes(int fmt, int n, int k, int m);
int dflash_linear(int fmt, int n, int k, const void *d_w, const void *d_s, const void *d_x, int ldx,
                  int m, int epilogue, float *d_out, int32_t *d_argmax, void *d_ws, size_t ws_bytes,
                  void *stream);

/* dflash_linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same GEMM with the same kernels and results, but its workspace is a
 * static device array of the library, one per device, allocated when the
 * library's code is loaded on that device and held until the process ends.
 * The call allocates nothing and takes no workspace argument; it runs on the
 * current device (the caller's stream must belong to it).
 * dflash_linear_noalloc_scratch_bytes() is the array's size (64 MiB); a
 * call whose workspace (dflash_linear_workspace_bytes) is larger fails with
 * DFLASH_E_CAPACITY before any launch.  Every call on one device uses that
 * device's array: calls that overlap on one device (other streams, other
 * threads) race and give wrong results; calls in stream order do not.
 * Arguments and errors otherwise as dflash_linear. */
size_t dflash_linear_noalloc_scratch_bytes(void);
int dflash_linear_noalloc(int fmt, int n, int k, const void *d_w, const void *d_s, const void *d_x, int ldx,
                          int m, int epilogue, float *d_out, int32_t *d_argmax, void *stream);

/* ------------------------------------------------------------- models */
typedef struct {
  int kind;                         /* DFLASH_LAYER_ATTN or DFLASH_LAYER_GDN */
  const float *in_norm;             /* [H] fp32 gain of the input RMSNorm */
  const float *post_norm;           /* [H] fp32 gain of the FFN RMSNorm */
  const float *q_norm, *k_norm;     /* [head_dim] fp32 per-head QK-norm gains (attn) */
  const void *w_qkv, *s_qkv;        /* packed [(hq+2hkv)d][H] (attn) or
                                       [gh*(2dk+dv)+2gh][H] q,k,v,a,b rows (gdn) */
  const void *w_o, *s_o;            /* packed [H][hq*d] (attn) or [H][gh*dv] (gdn) */
  const void *w_gu, *s_gu;          /* packed with gate_up=1: [2F][H] */
  const void *w_down, *s_down;      /* packed [H][F] */
} dflash_layer_desc;

typedef struct {
  int hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, n_layers;
  int gdn_heads, gdn_dk, gdn_dv;    /* GatedDeltaNet layer shape (hybrid targets) */
  float eps;                        /* RMSNorm epsilon */
  double rope_base;                 /* neox RoPE base */
  int fmt;                          /* DFLASH_FMT_* of every linear layer of this stack */
  /* target only (NULL for a drafter; the drafter uses the bound target's) */
  const void *embed;                /* [V][H]: fp32 (F32 models) or bf16 */
  const void *w_lm, *s_lm;          /* packed lm-head [V][H] */
  const float *final_norm;          /* [H] */
  /* drafter only */
  int n_sel;                        /* number of conditioning target layers */
  int sel_layers[8];                /* their indices in the target, ascending */
  int mask_token;                   /* id of the drafter's mask slot */
  const void *w_fc, *s_fc;          /* packed [H][n_sel*H] context projection */
  const float *hidden_norm;         /* [H] RMSNorm after the projection */
  const dflash_layer_desc *layers;  /* n_layers entries; copied by create */
} dflash_model_desc;

typedef struct dflash_model dflash_model;
typedef struct dflash_state dflash_state;

/* Create a model from a descriptor (host copy; device pointers are borrowed).
 * Errors: INVALID for null/unknown fields, SHAPE for dimensions the kernels do
 * not support (head_dim must be 64 or 128 and even; hq % hkv == 0; H % 128). */
int dflash_model_create(const dflash_model_desc *desc, dflash_model **out);
void dflash_model_destroy(dflash_model *m);

/* The drafter reuses the target's embedding and lm-head
 * (mlx-dspark v0.0.3, "Highlights": drafter.bind(target.model)).
 * Errors: SHAPE if widths/vocab differ or a conditioning layer index is out
 * of range of the target. */
int dflash_drafter_bind(dflash_model *drafter, const dflash_model *target);

/* ------------------------------------------------------------- state
 * All per-sequence device memory of one target/drafter pair lives in one
 * caller-provided arena: paged KV caches of target and drafter (64-token
 * pages), GatedDeltaNet states, tape and snapshot, activations, split-K and
 * attention workspaces, RoPE table, the token log, device lengths.
 * block is B (16 or 32); max_ctx is the longest committed context.
 * dflash_state_bytes returns 0 on invalid input. */
size_t dflash_state_bytes(const dflash_model *target, const dflash_model *drafter,
                          int max_ctx, int block);
/* Carves the arena, uploads the RoPE table and clears the device lengths
 * (synchronous). Errors: CAPACITY if arena_bytes is too small; INVALID if
 * the drafter is not bound to this target. */
int dflash_state_init(dflash_state **out, const dflash_model *target,
                      const dflash_model *drafter, void *d_arena, size_t arena_bytes,
                      int max_ctx, int block);
void dflash_state_destroy(dflash_state *st);

/* Prefill P prompt tokens (target forward in chunks of B, causal; the
 * drafter's context rows for all P positions).  An int4 or bf16 target runs
 * the prompt in chunks of up to 1024 rows (dense GEMMs, one-pass causal
 * attention); with GatedDeltaNet layers (run B tokens at a time) or a drafter
 * without the dense path, the chunks stop at the last whole block before the
 * last token and that block runs as a block.  An fp32 target runs every
 * chunk as a block.  Writes the first generated
 * token (argmax of the last prompt row) to d_first_tok[0] and sets n = P.
 * The committed token log holds the prompt then every emitted token.
 * Not graph-capturable (host loop over chunks).  Errors: CAPACITY if
 * P + B > max_ctx. */
int dflash_prefill(dflash_state *st, const int32_t *d_tokens, int n_tokens,
                   int32_t *d_first_tok, void *stream);

/* One drafter pass.  d_block[0] holds the anchor (last emitted token, at
 * position n); the block [anchor, mask x (B-1)] at positions n..n+B-1 is
 * denoised in one pass over the drafter's context (every slot sees every
 * committed context row and every block slot).  Context rows committed by the
 * previous verify are projected and appended first.  Writes the drafts
 * d_1..d_{B-1} to d_block[1..B-1].  d_logits, if not NULL, receives the fp32
 * draft logits of rows 1..B-1 as [B-1][V]. */
int dflash_draft_block(dflash_state *st, int32_t *d_block, float *d_logits, void *stream);

/* Target verify of d_block[0..R-1] at positions n..n+R-1 (causal inside the
 * block, full committed context), R = B, or the verify rows set by
 * dflash_set_max_draft.  Writes y_i = argmax of row i (lowest index on ties)
 * to d_argmax[0..R-1], K/V of all R positions to the cache (the rejected
 * ones are overwritten by the next verify), the conditioning layers' outputs
 * to the drafter's context buffer, and for GatedDeltaNet layers the
 * per-token tape.  d_logits, if not NULL, receives [R][vocab] fp32 logits. */
int dflash_verify_block(dflash_state *st, const int32_t *d_block, int32_t *d_argmax,
                        float *d_logits, void *stream);

/* Draft cap (mlx-dspark v0.0.3, "Highlights" and "API": --max-draft, where 0
 * runs the whole block): later verifies check only the first
 * N = min(max_draft, B-1) drafts (N = B-1 for max_draft = 0).  Each verify
 * then runs V rows, V the smallest multiple of the target attention's row
 * quantum (G*V query rows of one KV head fill whole 16-row MFMA blocks, G =
 * query heads per KV head; 1 for fp32 models) that is >= N+1, capped at B:
 * d_argmax[0..V-1] and d_logits [V][vocab] are written, rows past N+1 are
 * computed but play no part.  The caller passes N+1 as `block` to
 * dflash_accept so that a <= N.  The drafter still drafts B-1 tokens and
 * prefill still runs whole blocks.  *h_verify_rows = V and *h_accept_block =
 * N+1 (either may be NULL).  Errors: DFLASH_E_INVALID (null state),
 * DFLASH_E_SHAPE (max_draft < 0).  Host-only call; it changes what later
 * calls enqueue, so a captured graph must be recaptured. */
int dflash_set_max_draft(dflash_state *st, int max_draft, int *h_verify_rows, int *h_accept_block);

/* Draft/verify overlap (mirror-sd README, "How It Works": the drafter runs
 * concurrently with the target's verify).  With on != 0, each later
 * dflash_verify_block also enqueues, on a second stream the state owns
 * (default priority, created on the first call), the part of the next draft
 * that depends on that verify alone: the drafter's context rows -- the fc
 * projection and hidden norm of every verify row's conditioning features, then
 * every drafter layer's k/v of them with QK-norm and RoPE, written to the
 * drafter cache at the rows' positions n+i.  That work starts once the last
 * conditioning layer's rows are complete (an event recorded on the verify's
 * stream) and runs while the target's remaining layers, the lm-head, the
 * acceptance and the commit run; dflash_kv_commit makes its stream wait for it
 * (as do the next draft, verify, prefill and rollback, if no commit came in
 * between), and the next dflash_draft_block skips those rows.  Rows past the
 * accepted prefix are written at positions the next draft's block rows
 * overwrite before any read, so every result equals the sequential path's (up
 * to the rounding of a draft QKV projection over B instead of 2B rows).  A
 * step captured into a graph (draft, verify, accept, commit) holds the fork and
 * the join, so the graph has two concurrent branches.  on = 0 returns to the
 * sequential path.  Errors: DFLASH_E_INVALID (null state), DFLASH_E_DEVICE
 * (stream or event creation failed).  Host-only call; it changes what later
 * calls enqueue, so a captured graph must be recaptured. */
int dflash_set_overlap(dflash_state *st, int on);

/* Temperature sampling (mlx-dspark v0.0.3, "Highlights": --temperature T > 0
 * stays lossless, an exact sample of the target at T).  temperature 0 (the
 * default) is greedy decoding; T > 0 switches later calls to speculative
 * sampling: dflash_draft_block draws slot j from softmax(z_j / T) of the
 * drafter's logits; dflash_verify_block keeps the target's logits of its
 * rows; dflash_accept_sampled (instead of dflash_accept) keeps d_j while
 * u_j < p_{j-1}(d_j) / q_j(d_j) and draws the correction from
 * max(0, p_a - q_{a+1}) renormalised, or a bonus token from p_N when all N
 * verified drafts are kept; dflash_prefill draws the first token from the
 * last prompt row.  Uniforms: Philox4x32-10 (Salmon et al., SC 2011) with
 * counter (n, row, stream, 0) and key (seed low 32 bits, seed high 32 bits),
 * n the committed length at the start of the step; stream 0 drafts, 1
 * acceptance tests, 2 correction/bonus, 3 first token (counter (P, 0, 3, 0)).
 * Errors: DFLASH_E_INVALID (null state), DFLASH_E_SHAPE (T < 0 or not
 * finite).  Host-only call; recapture a graph after changing it. */
int dflash_set_sampling(dflash_state *st, float temperature, uint64_t seed);

/* Speculative-sampling acceptance of the last draft+verify at the state's
 * temperature, over the N drafts the verify checked (dflash_set_max_draft):
 * d_accept[0] = a; d_emit[0..a-1] = d_1..d_a, d_emit[a] = the drawn
 * correction or bonus token, d_emit[a+1..B-1] = -1; d_next_anchor (may alias
 * d_block, may be NULL) receives d_emit[a].  Reads the drafter and target
 * logits the state kept from those calls.  Errors: DFLASH_E_INVALID (null
 * argument), DFLASH_E_UNSUPPORTED (temperature 0), DFLASH_E_DEVICE. */
int dflash_accept_sampled(dflash_state *st, const int32_t *d_block, int32_t *d_accept, int32_t *d_emit,
                          int32_t *d_next_anchor, void *stream);

/* Stateless forms of the two sampling steps, on caller logits (fp32, device):
 * dflash_sample_logits: for r < rows, the log-normaliser log sum_v
 * exp(logits[r][v] / T) -> d_lse[r] (may be NULL) and, for stream_id in
 * [0, 3], a draw from softmax(logits[r] / T) with counter (n, row0 + r,
 * stream_id) -> d_tokens[r]; stream_id < 0 computes d_lse only.  Row r
 * starts at d_logits + r*ld (ld >= vocab).
 * dflash_accept_logits: the acceptance of dflash_accept_sampled for one
 * block: d_block[0..block-1] (anchor, drafts), d_dlog [n_drafts][vocab] the
 * drafter logits of slots 1..n_drafts, d_vlog [n_drafts+1][vocab] the target
 * logits of rows 0..n_drafts, n the committed length of the step;
 * d_lse [2*block] fp32 is caller scratch.  Outputs as dflash_accept_sampled.
 * Errors: DFLASH_E_INVALID (null pointer), DFLASH_E_SHAPE (sizes, counter,
 * T <= 0).  Neither allocates. */
int dflash_sample_logits(const float *d_logits, int ld, int rows, int vocab, float temperature, uint64_t seed,
                         int n, int row0, int stream_id, int32_t *d_tokens, float *d_lse, void *stream);
int dflash_accept_logits(const int32_t *d_block, const float *d_dlog, const float *d_vlog, int vocab,
                         int n_drafts, int block, float temperature, uint64_t seed, int n, float *d_lse,
                         int32_t *d_accept, int32_t *d_emit, int32_t *d_next_anchor, void *stream);

/* Longest-prefix acceptance: a = max{k <= B-1 : d_block[j] == d_argmax[j-1]
 * for all 1 <= j <= k}.  d_accept[0] = a; d_emit[0..a-1] = drafts d_1..d_a,
 * d_emit[a] = d_argmax[a] (the correction), d_emit[a+1..B-1] = -1.
 * d_next_anchor (may alias d_block) receives d_argmax[a]; may be NULL. */
int dflash_accept(const int32_t *d_block, const int32_t *d_argmax, int block,
                  int32_t *d_accept, int32_t *d_emit, int32_t *d_next_anchor, void *stream);

/* Commit the a+1 tokens of the last verify (a read from d_accept on the
 * device): n <- n + a + 1, the emitted tokens are appended to the token log,
 * the a+1 verified rows become pending drafter context rows, and every
 * GatedDeltaNet layer replays its tape for those a+1 tokens from the
 * committed state (pinned fp32 op order; bit-reproducible).  KV of rejected
 * positions needs no copy: it lies beyond n and is overwritten.  If the new
 * length would leave no room for the next block, nothing changes and the
 * CAPACITY status bit is set. */
int dflash_kv_commit(dflash_state *st, const int32_t *d_accept, const int32_t *d_emit,
                     void *stream);

/* Truncate the committed context to new_len (<= current n, >= 1) on the
 * host-visible stream order: KV beyond new_len is dropped, the token at
 * new_len in the log becomes the anchor (written to d_block[0] if not NULL).
 * Hybrid targets restore the GatedDeltaNet state from the snapshot taken by
 * dflash_gdn_snapshot, which must have been taken at length new_len
 * (UNSUPPORTED otherwise).  Synchronises the stream to read n. */
int dflash_kv_rollback(dflash_state *st, int new_len, int32_t *d_block, void *stream);

/* Copy the committed GatedDeltaNet states (and n) to the snapshot area. */
int dflash_gdn_snapshot(dflash_state *st, void *stream);

/* Benchmark harness (not part of the method): overwrite the drafts with a
 * reference stream so that a known number is accepted.  With s the device
 * step counter and k = d_sched[s % n_sched]: d_block[j] = d_ref[n+j] for
 * j <= k; d_block[k+1] = d_filler[(s % n_sched)*B + k+1], bumped by one
 * (mod V) if it equals d_ref[n+k+1]; later slots take filler tokens.
 * Positions at or past ref_len take filler tokens. */
int dflash_inject(dflash_state *st, int32_t *d_block, const int32_t *d_ref, int ref_len,
                  const int32_t *d_sched, int n_sched, const int32_t *d_filler, void *stream);

/* Read back (synchronises the stream): committed length n, device step count
 * and status word.  h_out = {n, steps, status, pending_ctx_rows}. */
int dflash_state_query(dflash_state *st, int32_t *h_out, void *stream);

/* Device pointers of internal buffers, for tests and tooling. */
typedef struct {
  int32_t *tokens;      /* token log [capacity] */
  int32_t *acc_log;     /* accepted count a of step s at [s % acc_log_len] */
  int acc_log_len;
  void *side;           /* drafter context input rows [B][n_sel*H] (fp16 codes of bf16 values, or fp32/bf16) */
  void *ctx_feat;       /* projected context features c [B][H] (same encoding) */
  float *gdn_state;     /* [n_gdn][gh][dv][dk] committed fp32 states */
  float *gdn_tape;      /* [n_gdn][B][gh][tape_stride] tape of the last verify: per
                           (token, head) k_hat[dk], v[dv], alpha, beta (fp32) */
  int tape_stride;      /* floats per (token, head) tape record: dk + dv + 2 */
  int n_gdn;
  int capacity;         /* positions the caches hold */
} dflash_state_view;
int dflash_state_buffers(dflash_state *st, dflash_state_view *out);

/* Optional per-launch timing of the GEMM kernels with hipEvents on the
 * launch stream (eager mode only; never while a graph is being captured).
 * Turning profiling on discards the previous records.
 * dflash_prof_read synchronises and returns per-kernel-variant totals:
 * names[i] (static strings), launches, total milliseconds, algorithmic
 * bytes (packed weights + scales, each streamed once) and, apart from
 * them, io_bytes (the 16-bit activations read once and the product
 * written once) summed over launches, for up to cap variants; any output
 * array may be NULL; *h_n receives the number of variants. */
int dflash_prof_enable(dflash_state *st, int on);
int dflash_prof_read(dflash_state *st, const char **names, int64_t *launches,
                     double *ms, double *bytes, double *io_bytes, int cap, int *h_n);

/* Kernel-only timing of one GEMM variant: re-launches, back to back on
 * `stream`, every launch of that variant recorded since profiling was
 * enabled (same weights, shapes and epilogues, in recorded order), the
 * whole series `reps` times, between two events; *h_ms receives the total
 * milliseconds and *h_launches the launch count (0 if the variant was not
 * recorded).  Unlike dflash_prof_read it has no marker between launches,
 * so total / launches is the kernel's average duration.  It rewrites the
 * step's per-step activations and the pending drafter context, so the
 * sequence state is not to be stepped again afterwards; it does not touch
 * the KV caches, the token log or the committed length.  Errors: DFLASH_E_INVALID
 * for a null argument or reps < 1, DFLASH_E_DEVICE if a launch fails. */
int dflash_prof_replay(dflash_state *st, const char *variant, int reps,
                       void *stream, double *h_ms, int64_t *h_launches);

/* What a weight-streaming launch of a given size and grid can reach at all:
 * reads `copies` consecutive regions of `bytes` each (d_buf holds copies *
 * bytes, bytes % 16 == 0; use more than the 256 MiB last-level cache in
 * total), one launch of nwg work-groups per region and nothing else (16-byte
 * non-temporal loads, no arithmetic on the data), the whole series `reps`
 * times back to back on `stream` after one warm-up launch; *h_ms receives
 * the total milliseconds of the copies * reps launches.  d_sink holds nwg
 * uint32 (written only in a case the data never produces).  Synchronises
 * the stream.  Errors: DFLASH_E_INVALID for a bad argument, DFLASH_E_DEVICE
 * if a launch fails. */
int dflash_read_floor(const void *d_buf, size_t bytes, int copies, int nwg, int reps, uint32_t *d_sink,
                      void *stream, double *h_ms);

/* Check of the hardware bf16 rounding the small kernels use: every fp32 bit
 * pattern is converted by the packed v_cvt_pk_bf16_f32 and by the integer
 * round-to-nearest-even: the rounding every bf16 activation of the step
 * goes through (the models of the dflash-mlx note, "Benchmarks" and
 * "Supported Models", run in bf16).  d_counts: 2 uint64 of device scratch
 * (cleared by the call);
 * h_counts[0] receives the mismatches on non-NaN inputs, h_counts[1] on NaN
 * inputs.  Synchronises the stream.  Errors: DFLASH_E_INVALID for a null
 * pointer, DFLASH_E_DEVICE if a launch or copy fails. */
int dflash_check_bf16_rounding(uint64_t *d_counts, void *stream, uint64_t *h_counts);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
