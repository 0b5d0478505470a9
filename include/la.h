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
} la_config;

/*
 * Forward recurrence over T tokens for every (b, h).
 * S0 may be NULL (zero initial state).  S_T may be NULL (not written).  ckpts may be NULL;
 * when non-NULL, cfg->ckpt_interval must be >= 1.  T == 0 writes S_T = S0.
 */
la_status la_recurrent_fwd(const la_config* cfg, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, const float* S0, void* o,
                           float* S_T, float* ckpts, void* stream);

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
 * One decode token (cfg->T must be 1): S [B][H][d_k][d_v] is read, updated, quantized at
 * the token (a single-token call always ends on a quantization point) and written back in
 * place.  codes/scales are optional (NULL = not written):
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
 * cfg->T must be 1; n_slots >= 1.
 */
la_status la_decode_step_slots(const la_config* cfg, const void* q, const void* k, const void* v,
                               const void* g, const void* beta, float* S_pool, const int32_t* slots,
                               int32_t n_slots, void* o, void* codes, float* scales, void* stream);

/*
 * Straight-through backward of la_recurrent_fwd for the upstream gradients dout (o) and
 * dS_T (S_T; NULL = zero).  Recomputation runs in chunks of cfg->ckpt_interval (>= 1)
 * tokens from ckpts (the forward's checkpoints with the same interval); ckpts == NULL
 * recomputes them into the workspace first.  Where la_bwd_kernel_name(cfg) is "block", the
 * states are instead recomputed from S0 with the block forward (the same arithmetic as
 * la_recurrent_fwd's "block" kernel, so the same rounding decisions) and ckpts is not read.
 * The workspace (device memory, at least la_bwd_workspace_bytes(cfg) bytes, contents
 * undefined on entry and exit) is owned by the caller.  Writes every gradient output in full.
 */
la_status la_recurrent_bwd_ste(const la_config* cfg, const void* q, const void* k,
                               const void* v, const void* g, const void* beta, const float* S0,
                               const float* ckpts, const float* dout, const float* dS_T,
                               float* dq, float* dk, float* dv, float* dg, float* dbeta,
                               float* dS0, void* workspace, size_t ws_bytes, void* stream);

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
 *            interval or checkpoint spacing that is not a multiple of 8).
 * Returns "" (and sets la_last_error) for an invalid cfg.  The kernels differ only in the
 * order of floating-point operations; every one computes the same recurrence.
 */
const char* la_fwd_kernel_name(const la_config* cfg);

/*
 * Which backward la_recurrent_bwd_ste runs for cfg (diagnostic; no GPU work, no state):
 *   "block"  the GDN configurations of the "block" forward: the state
 *            entering every 16-token block is recomputed into the workspace, then the blocks
 *            are walked last to first on the matrix cores (the block form of the adjoint);
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
