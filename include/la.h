/*
 * la.h - gated delta rule recurrence with fused dynamic state fake-quantization,
 * hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * What is computed (linear-attention state-QAT pages: "Torch GDN/KDA decode QAT + INT8",
 * "What does this PR do?"; "GDN state/W QAT foundation", "What does this PR do?"; "Fused
 * Triton GDN/KDA decode QAT", "What does this PR do?").  Per sequence b, head h and token t,
 * with the state S (d_k x d_v, key rows, value columns) held in FP32:
 *
 *     a     = exp(g_t)                  scalar (GDN) or one factor per key channel (KDA)
 *     S~    = diag(a) S_{t-1}
 *     u     = S~^T k_t
 *     delta = beta_t (v_t - u)
 *     S'    = S~ + k_t delta^T          (= the transpose of S diag(a)(I - beta k k^T) + beta v k^T)
 *     o_t   = S'^T q_t                  (read before rounding)
 *     S_t   = Q(S') at quantization points, else S'
 *
 * Q is one of
 *   INT8 group : per key row, groups of `group` (16|32|64) consecutive value columns;
 *                s = amax/127 (s = 1 when amax == 0), code = clamp(rne(x/s), -127, 127),
 *                xhat = code * s; x/s is an IEEE-correctly-rounded FP32 division.
 *   INT8 group after a Walsh-Hadamard rotation of the key axis (hadamard = 1):
 *                S_t = Hn Q(Hn S') with Hn the normalized Sylvester Hadamard matrix.
 *   E4M3 tile  : per tile of all d_k rows x 64 value columns; s = amax/448 (1 when amax == 0),
 *                y = x/s rounded to the nearest OCP E4M3FN value (ties to even, saturating
 *                at +-448), xhat = y_rounded * s.
 * Quantization points: after every token (qdq_interval = 1), or after tokens n, 2n, ... and
 * after the last token of the call (qdq_interval = n).  S_0 is not rounded on entry.
 * The backward pass uses an identity straight-through gradient through Q (and through the
 * rotations, whose product is the identity).
 *
 * Layouts (row-major, contiguous, every pointer 16-byte aligned):
 *   q, k       [B][T][H][d_k]          dtype qkv_dtype
 *   v          [B][T][H][d_v]          dtype qkv_dtype
 *   g          [B][T][H]  (GDN) or [B][T][H][d_k] (KDA)   dtype gate_dtype
 *   beta       [B][T][H]               dtype gate_dtype
 *   o          [B][T][H][d_v]          dtype out_dtype
 *   S0, S_T, S [B][H][d_k][d_v]        float32
 *   ckpts      [B][H][ceil(T/ckpt_interval)][d_k][d_v] float32: the carried state entering
 *              tokens 0, n, 2n, ... (n = ckpt_interval).  In Hadamard mode with the scalar
 *              gate the carried state is kept, and checkpointed, in its rotated form
 *              Y = Hu S (Hu the unnormalized Sylvester matrix, Hu Hu = d_k I), on which the
 *              INT8 codes act; S = Hu Y / d_k.  With per-key gates (a row decay does not
 *              commute with the rotation) S is carried and checkpointed unrotated and rotated
 *              to Hu S' only at each rounding point, where the codes act on it.
 *   dout       [B][T][H][d_v]          float32
 *   dq, dk     [B][T][H][d_k], dv [B][T][H][d_v], dg like g, dbeta [B][T][H],
 *   dS_T, dS0  [B][H][d_k][d_v]        all float32
 *
 * Ownership and threading: every tensor pointer is a device pointer owned by the caller;
 * the library never allocates, frees or retains a pointer past the call.  All work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs asynchronously;
 * a returned LA_OK means the arguments were valid and the kernels were enqueued.  Argument
 * checks happen on the host before any HIP call, so an invalid call touches no device
 * state.  Calls are thread-safe; la_last_error() is per thread.  Unsupported combinations
 * return LA_ERR_UNSUPPORTED; there is no fallback path.
 *
 * Supported: d_k in {16, 32, 64, 128}; d_v a multiple of 64 up to 4096; INT8 group 16, 32
 * or 64; E4M3 tile width 64; Hadamard with INT8, for either gate (state_rotated = 1 with the
 * scalar gate only).
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = 1, /* null pointer, bad size or enum value */
    LA_ERR_UNSUPPORTED = 2, /* valid but not implemented (shape or mode combination) */
    LA_ERR_ALIGNMENT = 3,   /* a tensor pointer is not 16-byte aligned */
    LA_ERR_WORKSPACE = 4,   /* backward workspace missing or too small */
    LA_ERR_HIP = 5          /* the HIP runtime reported an error while enqueuing */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;
typedef enum { LA_GATE_SCALAR = 0, LA_GATE_KEY = 1 } la_gate;
typedef enum { LA_QDQ_NONE = 0, LA_QDQ_INT8_GROUP = 1, LA_QDQ_E4M3_TILE = 2 } la_qdq;
/* Forward kernel choice (see la_fwd_kernel_name): automatic, or one kernel by name. */
typedef enum {
    LA_KERNEL_AUTO = 0,
    LA_KERNEL_BLOCK = 1,
    LA_KERNEL_WAVE = 2,
    LA_KERNEL_FAST = 3,
    LA_KERNEL_TOKEN = 4,
    LA_KERNEL_CHUNK = 5  /* the 64-token chunk form (la_recurrent_fwd_chunk): d_k = 128 */
} la_kernel;
/* The chunk form's triangular solve ("Experimental GDN/KDA approximate-inverse QAT", What does
   this PR do?: exact solve by default, or an explicit Neumann polynomial degree). */
typedef enum { LA_SOLVE_EXACT = 0, LA_SOLVE_NEUMANN = 1 } la_solve;

typedef struct la_config {
    int32_t B, T, H, d_k, d_v;
    int32_t gate;          /* la_gate */
    int32_t qdq;           /* la_qdq */
    int32_t group;         /* INT8: 16 | 32 | 64 columns; E4M3: tile width, 64 */
    int32_t hadamard;      /* 0 | 1 (INT8 only) */
    int32_t qdq_interval;  /* >= 1 when qdq != LA_QDQ_NONE */
    int32_t ckpt_interval; /* 0 = no checkpoints; backward: the recompute chunk length */
    int32_t qkv_dtype;     /* la_dtype of q, k, v */
    int32_t gate_dtype;    /* la_dtype of g, beta */
    int32_t out_dtype;     /* la_dtype of o */
    int32_t state_rotated; /* Hadamard mode with the scalar gate only.  0: S0, S_T, S (decode),
                              dS_T and dS0 hold the state S.  1: they hold the rotated state
                              Y = Hu S (and the gradients dL/dY), the representation the
                              codes act on; chained calls then resume bit for bit and a
                              decode step rotates only the key and query vectors, never the
                              state. */
    int32_t kernel;        /* la_kernel.  LA_KERNEL_AUTO: the first kernel of la_fwd_kernel_name's
                              list that serves cfg.  Any other value runs that forward kernel
                              (la_recurrent_fwd, and the backward's recompute) or returns
                              LA_ERR_UNSUPPORTED where it cannot serve cfg; the kernels differ
                              only in the order of floating-point operations between rounding
                              points.  la_recurrent_fwd_varlen accepts AUTO and TOKEN only;
                              the decode steps accept AUTO only. */
    int32_t replay;        /* 0 | 1: replay windows of qdq_interval tokens ("Torch GDN/KDA decode
                              QAT + INT8", What does this PR do?: larger windows keep BF16 key and
                              update entries and refresh at the window boundary; "Fused Triton
                              GDN/KDA decode QAT": encode-once factors).  The rounding points
                              stay those of qdq_interval; at every other token the carried state
                              takes the token's update from its key and delta each rounded once
                              to BF16 (nearest, ties to even), S_t = S~ + bf16(k) bf16(delta)^T,
                              while o_t reads the unrounded update.  A window of one token is
                              rounding after every token.  Needs a quantizer and bf16 q/k/v
                              (keys are then their own BF16 entries); runs the per-token kernel.
                              The backward passes straight through the encoding as through Q. */
    int32_t solve;         /* la_solve.  LA_SOLVE_EXACT (0): the recurrence above, on any kernel.
                              LA_SOLVE_NEUMANN (1): the 64-token chunk form in which each chunk's
                              (I + A)^-1 is replaced by the Neumann polynomial
                              sum_{n=0}^{degree} (-A)^n ("Experimental GDN/KDA approximate-inverse
                              QAT", What does this PR do?), a different function of the inputs;
                              runs on the chunk kernel only (la_recurrent_fwd_chunk), whose
                              comment states the chunk form. */
    int32_t degree;        /* Neumann degree, 3 | 7 | 15 | 31 with LA_SOLVE_NEUMANN, else 0.  It is
                              used as given: never raised, lowered or replaced by the exact solve. */
} la_config;

/*
 * Forward recurrence over T tokens for every (b, h): the training forward of the state QAT
 * ("GDN state/W QAT foundation", What does this PR do?: the recurrence with per-tile E4M3
 * state QDQ at 64-token boundaries; "Torch GDN/KDA decode QAT + INT8", What does this PR do?:
 * the GDN/KDA recurrent path with token state QDQ, INT8 groups and the Hadamard mode).
 * S0 may be NULL (zero initial state).  S_T may be NULL (not written).  ckpts may be NULL;
 * when non-NULL, cfg->ckpt_interval must be >= 1.  T == 0 writes S_T = S0.
 * Errors: LA_ERR_INVALID_ARG / LA_ERR_UNSUPPORTED / LA_ERR_ALIGNMENT from the host checks
 * (nothing is enqueued), LA_ERR_HIP if a launch fails.
 */
la_status la_recurrent_fwd(const la_config* cfg, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, const float* S0, void* o,
                           float* S_T, float* ckpts, void* stream);

/*
 * Forward over 64-token chunks ("GDN state/W QAT foundation", What does this PR do?: the state
 * rounded at 64-token chunk boundaries; "Experimental GDN/KDA approximate-inverse QAT", What
 * does this PR do?: the chunk's triangular solve exact or by a Neumann polynomial).  Tokens are
 * cut into chunks of 64 from the start of the call; a chunk of L tokens entering with the
 * carried state S, with cumulative log decays G_r = g_0 + ... + g_r per key (the scalar gate's
 * value on every key), computes
 *     A_ri  = beta_r sum_k k_r[k] k_i[k] exp(G_r[k] - G_i[k])   (i < r; 0 elsewhere)
 *     M_ri  = sum_k q_r[k] k_i[k] exp(G_r[k] - G_i[k])          (i <= r; 0 elsewhere)
 *     P     = (I + A)^-1 (solve = EXACT) or sum_{n=0}^{degree} (-A)^n (solve = NEUMANN)
 *     Delta = P diag(beta) (V - (K o E) S),  E_r = exp(G_r)
 *     O     = (Q o E) S + M Delta
 *     S_end = diag(exp(G_{L-1})) S + (K o F)^T Delta,  F_r = exp(G_{L-1} - G_r)
 * and S_end is rounded when the chunk ends on a rounding point.  With the exact solve this is
 * the recurrence in the header comment (up to the order of floating-point operations).
 * cfg->kernel must be LA_KERNEL_CHUNK, or LA_KERNEL_AUTO with solve = NEUMANN.  Needs d_k = 128,
 * no Hadamard rotation and no replay windows, qdq_interval a multiple of 64 with a quantizer,
 * ckpt_interval 0 or a multiple of 64.  workspace: device memory of at least
 * la_chunk_workspace_bytes(cfg) bytes (the chunks' matrices), owned by the caller, contents
 * ignored on entry and undefined on return.  Other arguments and errors as la_recurrent_fwd;
 * LA_ERR_WORKSPACE when the workspace is missing or too small.
 */
la_status la_recurrent_fwd_chunk(const la_config* cfg, const void* q, const void* k, const void* v,
                                 const void* g, const void* beta, const float* S0, void* o,
                                 float* S_T, float* ckpts, void* workspace, size_t ws_bytes,
                                 void* stream);

/* Workspace bytes la_recurrent_fwd_chunk needs for cfg (0 if cfg is invalid or not served by
   the chunk kernel). */
size_t la_chunk_workspace_bytes(const la_config* cfg);

/*
 * la_recurrent_fwd in replay mode (cfg->replay = 1) that also writes every token's update
 * entry: entries [B][T][H][d_v] bf16 bit patterns, delta_t rounded once to BF16 (nearest,
 * ties to even), the value the carried state takes at every token that is not a rounding
 * point (written for the rounding points' tokens too, whose refresh uses delta itself).  For
 * inspection of the replay encoding; runs the per-token kernel.  LA_ERR_INVALID_ARG without
 * replay.
 */
la_status la_recurrent_fwd_entries(const la_config* cfg, const void* q, const void* k, const void* v,
                                   const void* g, const void* beta, const float* S0, void* o, float* S_T,
                                   float* ckpts, void* entries, void* stream);

/*
 * Forward over packed sequences of different lengths (the packed sequence tails of the
 * linear-attention state-QAT pages' GDN/KDA state QAT, serving prefill).  cfg->B is the
 * number of sequences and cfg->T the packed length; sequence b is tokens
 * cu_seqlens[b] .. cu_seqlens[b + 1] - 1 of q, k [T][H][d_k], v, o [T][H][d_v], g [T][H]
 * ([T][H][d_k] for per-key gates) and beta [T][H].  Each sequence starts from S0[b] (NULL =
 * zeros), has its own rounding points (counted from its first token) and ends in S_T[b]
 * (NULL = not written); S0 and S_T are [B][H][d_k][d_v].  cu_seqlens is int32 [B + 1] in
 * device memory, non-decreasing from 0 to T; the kernel clamps every boundary to [0, T] (a
 * sequence whose boundaries are out of order is empty).  No checkpoints; the per-token kernel
 * serves every configuration.
 */
la_status la_recurrent_fwd_varlen(const la_config* cfg, const int32_t* cu_seqlens, const void* q,
                                  const void* k, const void* v, const void* g, const void* beta,
                                  const float* S0, void* o, float* S_T, void* stream);

/*
 * Packed sequences with a per-sequence prefix/suffix boundary ("Torch GDN/KDA decode QAT +
 * INT8", What does this PR do?: an explicit per-sequence boundary selects a chunked prefill
 * prefix and a recurrent suffix; suffix gradients flow through the handoff into prefill).
 * Layouts as in la_recurrent_fwd_varlen (cfg->B sequences packed into cfg->T tokens).  Sequence
 * b's first prefix_len[b] tokens (int32 [B], device memory, clamped to the sequence) run with
 * prefix_cfg from S0[b] (NULL = zeros), its rounding points counted from its first token and
 * the prefix's last token a rounding point; the state there, S_mid[b] (float32
 * [B][H][d_k][d_v], written, the handoff the backward needs), starts the remaining tokens,
 * which run with suffix_cfg and end in S_T[b] (NULL = not written).  The two configurations
 * must agree in B, T, H, d_k, d_v, gate and dtypes; their quantizers, intervals, Hadamard and
 * replay settings may differ; state_rotated must be 0 in both.  Per-token kernel, two launches.
 */
la_status la_recurrent_fwd_split(const la_config* prefix_cfg, const la_config* suffix_cfg,
                                 const int32_t* cu_seqlens, const int32_t* prefix_len, const void* q,
                                 const void* k, const void* v, const void* g, const void* beta,
                                 const float* S0, void* o, float* S_mid, float* S_T, void* stream);

/*
 * Straight-through backward of la_recurrent_fwd_varlen for the upstream gradients dout
 * ([T][H][d_v]) and dS_T ([B][H][d_k][d_v]; NULL = zero): every gradient in the packed layout,
 * dS0 per sequence.  Chunks of cfg->ckpt_interval (>= 1) tokens are recomputed from
 * checkpoints that the call first recomputes into the workspace (at least
 * la_bwd_varlen_workspace_bytes(cfg) bytes).  Tokens outside every sequence get zero gradients.
 */
la_status la_recurrent_bwd_ste_varlen(const la_config* cfg, const int32_t* cu_seqlens, const void* q,
                                      const void* k, const void* v, const void* g, const void* beta,
                                      const float* S0, const float* dout, const float* dS_T, float* dq,
                                      float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                                      void* workspace, size_t ws_bytes, void* stream);
size_t la_bwd_varlen_workspace_bytes(const la_config* cfg);

/*
 * Straight-through backward of la_recurrent_fwd_split: the suffix backward from S_mid (the
 * forward's handoff states) for dout and dS_T, whose dS0 is the gradient at the handoff; then
 * the prefix backward from S0 with that gradient as its dS_T.  Each part recomputes with its
 * own configuration (ckpt_interval >= 1 in both).  Workspace: at least
 * la_bwd_split_workspace_bytes(prefix_cfg, suffix_cfg) bytes.
 */
la_status la_recurrent_bwd_ste_split(const la_config* prefix_cfg, const la_config* suffix_cfg,
                                     const int32_t* cu_seqlens, const int32_t* prefix_len, const void* q,
                                     const void* k, const void* v, const void* g, const void* beta,
                                     const float* S0, const float* S_mid, const float* dout,
                                     const float* dS_T, float* dq, float* dk, float* dv, float* dg,
                                     float* dbeta, float* dS0, void* workspace, size_t ws_bytes,
                                     void* stream);
size_t la_bwd_split_workspace_bytes(const la_config* prefix_cfg, const la_config* suffix_cfg);

/*
 * One decode token (cfg->T must be 1): the serving-side recurrent step with token state QDQ
 * ("Torch GDN/KDA decode QAT + INT8", What does this PR do?: the recurrent decode takes BF16
 * inputs and works in FP32; "Fused Triton GDN/KDA decode QAT", What does this PR do?: the
 * fused token update with FP8 or INT8 state QDQ).  S [B][H][d_k][d_v] is read, updated,
 * quantized at the token (a single-token call always ends on a quantization point) and
 * written back in place; the caller owns S.  codes/scales are optional (NULL = not written):
 *   INT8:  codes int8 [B][H][d_k][d_v], scales float [B][H][d_k][d_v/group]
 *          (Hadamard: codes and scales of H S' with H the unnormalized Sylvester matrix,
 *          i.e. scales are sqrt(d_k) times those of the normalized rotation)
 *   E4M3:  codes uint8 E4M3FN bit patterns [B][H][d_k][d_v], scales float [B][H][d_v/64]
 */
la_status la_decode_step(const la_config* cfg, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, float* S, void* o, void* codes,
                         float* scales, void* stream);

/*
 * One decode token for a serving batch whose states live in a pool of slots (the decode-side
 * neighbour of la_decode_step; linear-attention state-QAT pages, "Torch/Triton GDN/KDA decode
 * QAT", the serving adapter's reserved paged-cache index zero).  Batch entry b advances the
 * state S_pool[slots[b]] in place exactly as la_decode_step advances S[b]; q, k, v, g, beta,
 * o, codes and scales are indexed by batch entry as there.
 *   S_pool  float [n_slots][H][d_k][d_v], device memory owned by the caller.
 *   slots   int32 [B], device memory.  Slot 0 is reserved: an entry with slots[b] == 0 (the
 *           padding of a packed batch) leaves the pool untouched, writes zeros to o[b] and
 *           writes no codes or scales; so does an index outside [0, n_slots).  Two entries of
 *           one call must not name the same slot other than 0 (their updates would race).
 * With B <= 1024 and n_slots <= 16384 the workgroups serve the entries in increasing slot
 * order, so that the pool is streamed in address order whatever the order of the entries;
 * every result is the same as in entry order.
 * cfg->T must be 1; n_slots >= 1.
 */
la_status la_decode_step_slots(const la_config* cfg, const void* q, const void* k, const void* v,
                               const void* g, const void* beta, float* S_pool, const int32_t* slots,
                               int32_t n_slots, void* o, void* codes, float* scales, void* stream);

/*
 * One decode token of a serving batch in replay mode (cfg->replay = 1, cfg->T = 1, window
 * W = cfg->qdq_interval): the serving side of replay windows ("Torch GDN/KDA decode QAT +
 * INT8", What does this PR do?: the runtime reconstructs its state from BF16 key/update entries
 * and refreshes the checkpoint at the window boundary, promoting working values to FP32).
 * Per sequence b the decode state is the window's checkpoint S[b] [H][d_k][d_v] (float32,
 * unrotated) and a log of the window's earlier tokens, entries 0 .. pos[b] - 1:
 *   log_k  bf16 [B][H][W - 1][d_k]   the keys' BF16 bits
 *   log_d  bf16 [B][H][W - 1][d_v]   the updates delta rounded once to BF16
 *   log_g  float [B][H][W - 1] (scalar gate) or [B][H][W - 1][d_k] (per-key gates): g
 *   pos    int32 [B] in device memory: entries already logged (clamped to [0, W - 1])
 * The call reconstructs the state entering the token in FP32 from the checkpoint and the
 * entries (S <- diag(exp g_i) S + k_i d_i^T in log order), advances it by the token and writes
 * o.  If pos[b] < W - 1 the token's entries are appended at index pos[b] and S[b] is left
 * unchanged; if pos[b] == W - 1 the token ends the window: S[b] <- Q(S') in place (codes and
 * scales as in la_decode_step, written only then).  The caller advances pos (pos + 1, or 0
 * after a window end).  Tokens of a window evolve exactly as la_recurrent_fwd's replay
 * tokens with the same window.  The log pointers may be NULL when W == 1.
 */
la_status la_decode_step_replay(const la_config* cfg, const void* q, const void* k, const void* v,
                                const void* g, const void* beta, float* S, void* log_k, void* log_d,
                                float* log_g, const int32_t* pos, void* o, void* codes, float* scales,
                                void* stream);

/*
 * Straight-through backward of la_recurrent_fwd ("GDN state/W QAT foundation", What does
 * this PR do?: identity straight-through gradients through the state QDQ; "Fused Triton
 * GDN/KDA decode QAT", What does this PR do?: a checkpointed custom backward with a
 * differentiable continuation carry, i.e. dS0) for the upstream gradients dout (o) and
 * dS_T (S_T; NULL = zero).  Recomputation runs in chunks of cfg->ckpt_interval (>= 1)
 * tokens from ckpts (the forward's checkpoints with the same interval); ckpts == NULL
 * recomputes them into the workspace first.  Where la_bwd_kernel_name(cfg) is "block", the
 * sequence is walked in segments, last first: the state entering every 16-token block of a
 * segment is recomputed from ckpts, all checkpoint chunks in parallel, with the block
 * forward's own arithmetic (no rounding point lies inside a chunk there), then the segment's
 * blocks are walked backwards on the matrix cores.
 * The workspace (device memory, at least la_bwd_workspace_bytes(cfg) bytes, contents
 * undefined on entry and exit) is owned by the caller.  Writes every gradient output in full.
 */
la_status la_recurrent_bwd_ste(const la_config* cfg, const void* q, const void* k,
                               const void* v, const void* g, const void* beta, const float* S0,
                               const float* ckpts, const float* dout, const float* dS_T,
                               float* dq, float* dk, float* dv, float* dg, float* dbeta,
                               float* dS0, void* workspace, size_t ws_bytes, void* stream);

/*
 * la_recurrent_bwd_ste without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The workspace is a fixed device array inside the library, la_noalloc_workspace_limit()
 * bytes (128 MiB) on each GPU the library runs on, held until the process ends.  A cfg whose
 * la_bwd_workspace_bytes exceeds it returns LA_ERR_WORKSPACE before any HIP call.  The call
 * allocates nothing.  Every call on a GPU shares that GPU's array: calls that overlap in time
 * on one GPU (several streams or threads) race and must be serialized by the caller.
 * Arguments, results and other errors are those of la_recurrent_bwd_ste.
 */
la_status la_recurrent_bwd_ste_noalloc(const la_config* cfg, const void* q, const void* k,
                                       const void* v, const void* g, const void* beta,
                                       const float* S0, const float* ckpts, const float* dout,
                                       const float* dS_T, float* dq, float* dk, float* dv,
                                       float* dg, float* dbeta, float* dS0, void* stream);

/* Bytes of la_recurrent_bwd_ste_noalloc's device array. */
size_t la_noalloc_workspace_limit(void);

/* Workspace bytes la_recurrent_bwd_ste needs for cfg (0 for an invalid cfg; the requirement
 * includes room for recomputed checkpoints, so it does not depend on whether ckpts is NULL). */
size_t la_bwd_workspace_bytes(const la_config* cfg);

/*
 * Which forward kernel la_recurrent_fwd runs for cfg (diagnostic; no GPU work, no state):
 *   "block"  GDN or KDA, no Hadamard, d_k = 128, bf16 q/k/v, rounding at most every 16 tokens
 *            (interval and checkpoint spacing multiples of 16; KDA: no rounding point strictly
 *            inside a checkpoint chunk): 16-token blocks on the matrix cores;
 *   "wave"   GDN or KDA, no Hadamard, interval and checkpoint spacing multiples of 8 (and
 *            no rounding point strictly inside a checkpoint chunk): one wave per 16 value
 *            columns, no barrier per token;
 *   "fast"   GDN, no Hadamard, rounding at most every 2 tokens, no rounding point strictly
 *            inside a checkpoint chunk: eight waves per 64 columns, rescaled state;
 *   "token"  every other valid configuration (Hadamard, rounding every token, KDA with an
 *            interval or checkpoint spacing that is not a multiple of 8);
 *   "chunk"  cfg->kernel = LA_KERNEL_CHUNK, or solve = LA_SOLVE_NEUMANN (never chosen by
 *            LA_KERNEL_AUTO for the exact solve): the 64-token chunk form, run by
 *            la_recurrent_fwd_chunk only (la_recurrent_fwd returns LA_ERR_UNSUPPORTED).
 * With cfg->kernel other than LA_KERNEL_AUTO the named kernel is returned if it serves cfg.
 * Returns "" (and sets la_last_error) for an invalid cfg or a requested kernel that cannot
 * serve it.  The kernels differ only in the order of floating-point operations; every one
 * computes the same recurrence.
 */
const char* la_fwd_kernel_name(const la_config* cfg);

/*
 * Which backward la_recurrent_bwd_ste runs for cfg (diagnostic; no GPU work, no state):
 *   "block"  the GDN configurations whose forward runs the "block" kernel: segment by
 *            segment (last first), the state entering every 16-token block is recomputed from
 *            the checkpoints into the workspace, then the blocks are walked last to first on
 *            the matrix cores (the block form of the adjoint);
 *   "token"  every other valid configuration: chunks of ckpt_interval tokens recomputed from
 *            the checkpoints and walked token by token.
 * Returns "" (and sets la_last_error) for an invalid cfg.
 */
const char* la_bwd_kernel_name(const la_config* cfg);

/* Static description of a status code. */
const char* la_status_string(la_status s);

/* Detail of the last non-LA_OK status returned on the calling thread ("" if none). */
const char* la_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LA_H */
