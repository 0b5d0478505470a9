// C ABI of the recurrence library: argument validation (host only, before any HIP call),
// workspace layout and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "la_internal.hpp"

namespace {

thread_local char g_err[512] = "";

la_status fail(la_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

la_status ok() {
    g_err[0] = '\0';
    return LA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

la_status check_config(const la_config* c, bool decode) {
    if (!c) return fail(LA_ERR_INVALID_ARG, "cfg is NULL");
    if (c->B < 0 || c->T < 0 || c->H < 0 || c->d_k <= 0 || c->d_v <= 0)
        return fail(LA_ERR_INVALID_ARG, "negative or zero size (B=%d T=%d H=%d d_k=%d d_v=%d)", c->B, c->T,
                    c->H, c->d_k, c->d_v);
    if (c->B > 65535 || c->H > 65535)
        return fail(LA_ERR_UNSUPPORTED, "B and H must each be <= 65535 (B=%d H=%d)", c->B, c->H);
    if (decode && c->T != 1) return fail(LA_ERR_INVALID_ARG, "decode needs T == 1 (T=%d)", c->T);
    if (c->d_k != 16 && c->d_k != 32 && c->d_k != 64 && c->d_k != 128)
        return fail(LA_ERR_UNSUPPORTED, "d_k must be 16, 32, 64 or 128 (d_k=%d)", c->d_k);
    if (c->d_v % 64 != 0 || c->d_v > 4096)
        return fail(LA_ERR_UNSUPPORTED, "d_v must be a multiple of 64 up to 4096 (d_v=%d)", c->d_v);
    if (c->gate != LA_GATE_SCALAR && c->gate != LA_GATE_KEY)
        return fail(LA_ERR_INVALID_ARG, "unknown gate %d", c->gate);
    for (int dt : {c->qkv_dtype, c->gate_dtype, c->out_dtype})
        if (dt != LA_F32 && dt != LA_BF16) return fail(LA_ERR_INVALID_ARG, "unknown dtype %d", dt);
    if (c->ckpt_interval < 0) return fail(LA_ERR_INVALID_ARG, "ckpt_interval < 0");
    if (c->hadamard != 0 && c->hadamard != 1) return fail(LA_ERR_INVALID_ARG, "hadamard must be 0 or 1");
    if (c->state_rotated != 0 && c->state_rotated != 1)
        return fail(LA_ERR_INVALID_ARG, "state_rotated must be 0 or 1");
    if (c->state_rotated && !c->hadamard)
        return fail(LA_ERR_INVALID_ARG, "state_rotated needs the Hadamard rotation");
    if (c->kernel < LA_KERNEL_AUTO || c->kernel > LA_KERNEL_CHUNK)
        return fail(LA_ERR_INVALID_ARG, "unknown kernel %d", c->kernel);
    if (c->solve != LA_SOLVE_EXACT && c->solve != LA_SOLVE_NEUMANN)
        return fail(LA_ERR_INVALID_ARG, "unknown solve %d", c->solve);
    if (c->solve == LA_SOLVE_NEUMANN && c->degree != 3 && c->degree != 7 && c->degree != 15 && c->degree != 31)
        return fail(LA_ERR_INVALID_ARG, "Neumann degree must be 3, 7, 15 or 31 (degree=%d)", c->degree);
    if (c->solve == LA_SOLVE_EXACT && c->degree != 0)
        return fail(LA_ERR_INVALID_ARG, "degree is the Neumann solve's (set solve = 1) and must be 0 otherwise");
    if (decode && c->solve != LA_SOLVE_EXACT)
        return fail(LA_ERR_INVALID_ARG, "the decode steps have no chunks: solve must be exact");
    if (c->replay != 0 && c->replay != 1) return fail(LA_ERR_INVALID_ARG, "replay must be 0 or 1");
    if (c->replay && c->qdq == LA_QDQ_NONE)
        return fail(LA_ERR_INVALID_ARG, "replay windows end in a rounding point: they need a quantizer");
    if (c->replay && c->qkv_dtype != LA_BF16)
        return fail(LA_ERR_UNSUPPORTED, "replay windows take bf16 q/k/v (the keys are their own BF16 entries)");
    if (decode && c->kernel != LA_KERNEL_AUTO)
        return fail(LA_ERR_INVALID_ARG, "the decode steps choose their kernel themselves (kernel must be 0)");
    switch (c->qdq) {
        case LA_QDQ_NONE:
            if (c->hadamard) return fail(LA_ERR_INVALID_ARG, "hadamard needs the INT8 quantizer");
            break;
        case LA_QDQ_INT8_GROUP:
            if (c->group != 16 && c->group != 32 && c->group != 64)
                return fail(LA_ERR_UNSUPPORTED, "INT8 group must be 16, 32 or 64 (group=%d)", c->group);
            if (c->hadamard && c->gate == LA_GATE_KEY && c->state_rotated)
                return fail(LA_ERR_UNSUPPORTED,
                            "state_rotated is implemented for the scalar gate only (per-key gates carry S)");
            if (c->qdq_interval < 1) return fail(LA_ERR_INVALID_ARG, "qdq_interval must be >= 1");
            break;
        case LA_QDQ_E4M3_TILE:
            if (c->group != 64) return fail(LA_ERR_UNSUPPORTED, "E4M3 tile width must be 64 (group=%d)", c->group);
            if (c->hadamard) return fail(LA_ERR_UNSUPPORTED, "Hadamard rotation is implemented for INT8 only");
            if (c->qdq_interval < 1) return fail(LA_ERR_INVALID_ARG, "qdq_interval must be >= 1");
            break;
        default:
            return fail(LA_ERR_INVALID_ARG, "unknown qdq mode %d", c->qdq);
    }
    return LA_OK;
}

la_status check_ptr(const void* p, const char* name, bool required) {
    if (!p) return required ? fail(LA_ERR_INVALID_ARG, "%s is NULL", name) : LA_OK;
    if (!aligned16(p)) return fail(LA_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
    return LA_OK;
}

#define CHECK(expr)                   \
    do {                              \
        la_status s_ = (expr);        \
        if (s_ != LA_OK) return s_;   \
    } while (0)

la_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

constexpr size_t kAlign = 256;
size_t round_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

struct WsLayout {
    size_t states, part, ckpts, total;
    size_t carry = 0;  // block backward: dS between segments
};

WsLayout ws_layout(const la_config& c) {
    WsLayout L;
    if (la::bwd_mfma_eligible(c)) {
        // block backward, per segment: the state entering every 16-token block, the partial
        // records; then dS carried between segments and room for the forward's checkpoints
        // (used when the caller gives none)
        L.states = 0;
        L.part = round_up(la::bwd_mfma_state_bytes(c));
        L.carry = L.part + round_up(la::bwd_mfma_part_bytes(c));
        L.ckpts = L.carry + round_up(static_cast<size_t>(c.B) * c.H * c.d_k * c.d_v * sizeof(float));
        L.total = L.ckpts + round_up(static_cast<size_t>(c.B) * c.H * la::n_ckpts(c) * c.d_k * c.d_v * sizeof(float));
        return L;
    }
    // the backward runs in the token layout: tiles of tok_tile_cols value columns
    const size_t tiles = static_cast<size_t>(la::tok_tiles(c));
    const size_t nwg = static_cast<size_t>(c.B) * c.H * tiles;
    L.states = 0;
    L.part = round_up(nwg * la::bwd_tok_ws_floats(c) * sizeof(float));
    L.ckpts = L.part + round_up(tiles * c.B * c.T * c.H * la::part_width(c) * sizeof(float));
    L.total = L.ckpts + round_up(static_cast<size_t>(c.B) * c.H * la::n_ckpts(c) * c.d_k * c.d_v * sizeof(float));
    return L;
}

// Packed sequences (token backward only): sub-states per workgroup (B sequences), partial
// row sums per value tile and packed token-head, checkpoints in the packed slot layout.
WsLayout ws_layout_varlen(const la_config& c) {
    WsLayout L;
    const size_t tiles = static_cast<size_t>(la::tok_tiles(c));
    const size_t nwg = static_cast<size_t>(c.B) * c.H * tiles;
    L.states = 0;
    L.part = round_up(nwg * la::bwd_tok_ws_floats(c) * sizeof(float));
    L.ckpts = L.part + round_up(tiles * static_cast<size_t>(c.T) * c.H * la::part_width(c) * sizeof(float));
    L.total = L.ckpts + round_up(static_cast<size_t>(c.H) * la::varlen_ckpt_slots(c) * c.d_k * c.d_v * sizeof(float));
    return L;
}

const char* la_status_string_impl(la_status s) {
    switch (s) {
        case LA_OK: return "ok";
        case LA_ERR_INVALID_ARG: return "invalid argument";
        case LA_ERR_UNSUPPORTED: return "unsupported configuration";
        case LA_ERR_ALIGNMENT: return "misaligned pointer";
        case LA_ERR_WORKSPACE: return "workspace missing or too small";
        case LA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}


la_status check_kernel(const la_config& c) {
    if (la::fwd_kernel(c) == LA_KERNEL_AUTO)
        return fail(LA_ERR_UNSUPPORTED, "the requested forward kernel (%d) cannot serve this configuration", c.kernel);
    return LA_OK;
}

}  // namespace

extern "C" {

const char* la_status_string(la_status s) { return la_status_string_impl(s); }

const char* la_last_error(void) { return g_err; }

const char* la_fwd_kernel_name(const la_config* cfg) {
    if (check_config(cfg, false) != LA_OK || check_kernel(*cfg) != LA_OK) return "";
    return la::fwd_kernel_name(*cfg);
}

const char* la_bwd_kernel_name(const la_config* cfg) {
    if (check_config(cfg, false) != LA_OK || check_kernel(*cfg) != LA_OK) return "";
    switch (la::bwd_kernel(*cfg)) {
        case LA_KERNEL_CHUNK: return "chunk";
        case LA_KERNEL_BLOCK: return "block";
        default: return "token";
    }
}

la_status la_recurrent_fwd(const la_config* cfg, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, const float* S0, void* o,
                           float* S_T, float* ckpts, void* stream) {
    CHECK(check_config(cfg, false));
    const la_config& c = *cfg;
    CHECK(check_kernel(c));
    if (la::fwd_kernel(c) == LA_KERNEL_CHUNK)
        return fail(LA_ERR_UNSUPPORTED, "the chunk kernel needs a workspace: call la_recurrent_fwd_chunk");
    const bool work = c.B > 0 && c.H > 0 && c.T > 0;
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(o, "o", work));
    CHECK(check_ptr(S0, "S0", false));
    CHECK(check_ptr(S_T, "S_T", false));
    CHECK(check_ptr(ckpts, "ckpts", false));
    if (ckpts && c.ckpt_interval < 1) return fail(LA_ERR_INVALID_ARG, "ckpts given but ckpt_interval < 1");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c.B == 0 || c.H == 0) return ok();
    if (c.T == 0) {
        if (!S_T) return ok();
        return hip_status(la::launch_copy_state(c, S0, S_T, s), "copy S0 -> S_T");
    }
    la::FwdArgs a{q, k, v, g, beta, S0, o, S_T, ckpts};
    return hip_status(la::launch_fwd(c, a, s), "la_recurrent_fwd launch");
}

size_t la_chunk_workspace_bytes(const la_config* cfg) {
    if (check_config(cfg, false) != LA_OK || la::fwd_kernel(*cfg) != LA_KERNEL_CHUNK) return 0;
    return la::chunk_fwd_workspace_bytes(*cfg);
}

la_status la_recurrent_fwd_chunk(const la_config* cfg, const void* q, const void* k, const void* v,
                                 const void* g, const void* beta, const float* S0, void* o,
                                 float* S_T, float* ckpts, void* workspace, size_t ws_bytes,
                                 void* stream) {
    CHECK(check_config(cfg, false));
    const la_config& c = *cfg;
    if (la::fwd_kernel(c) != LA_KERNEL_CHUNK)
        return fail(LA_ERR_UNSUPPORTED, "the chunk kernel needs kernel = LA_KERNEL_CHUNK (or the Neumann solve), "
                    "d_k = 128, no rotation or replay, rounding points and checkpoints on multiples of 64");
    const bool work = c.B > 0 && c.H > 0 && c.T > 0;
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(o, "o", work));
    CHECK(check_ptr(S0, "S0", false));
    CHECK(check_ptr(S_T, "S_T", false));
    CHECK(check_ptr(ckpts, "ckpts", false));
    CHECK(check_ptr(workspace, "workspace", false));
    if (ckpts && c.ckpt_interval < 1) return fail(LA_ERR_INVALID_ARG, "ckpts given but ckpt_interval < 1");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c.B == 0 || c.H == 0) return ok();
    if (c.T == 0) {
        if (!S_T) return ok();
        return hip_status(la::launch_copy_state(c, S0, S_T, s), "copy S0 -> S_T");
    }
    const size_t need = la::chunk_fwd_workspace_bytes(c);
    if (!workspace || ws_bytes < need)
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? ws_bytes : static_cast<size_t>(0));
    la::FwdArgs a{q, k, v, g, beta, S0, o, S_T, ckpts};
    return hip_status(la::launch_chunk_fwd(c, a, static_cast<float*>(workspace), s), "la_recurrent_fwd_chunk launch");
}

la_status la_recurrent_fwd_entries(const la_config* cfg, const void* q, const void* k, const void* v,
                                   const void* g, const void* beta, const float* S0, void* o, float* S_T,
                                   float* ckpts, void* entries, void* stream) {
    CHECK(check_config(cfg, false));
    const la_config& c = *cfg;
    if (!c.replay) return fail(LA_ERR_INVALID_ARG, "update entries exist in replay mode only (cfg->replay = 1)");
    CHECK(check_kernel(c));
    const bool work = c.B > 0 && c.H > 0 && c.T > 0;
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(o, "o", work));
    CHECK(check_ptr(entries, "entries", work));
    CHECK(check_ptr(S0, "S0", false));
    CHECK(check_ptr(S_T, "S_T", false));
    CHECK(check_ptr(ckpts, "ckpts", false));
    if (ckpts && c.ckpt_interval < 1) return fail(LA_ERR_INVALID_ARG, "ckpts given but ckpt_interval < 1");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c.B == 0 || c.H == 0) return ok();
    if (c.T == 0) {
        if (!S_T) return ok();
        return hip_status(la::launch_copy_state(c, S0, S_T, s), "copy S0 -> S_T");
    }
    la::FwdArgs a{q, k, v, g, beta, S0, o, S_T, ckpts};
    a.entries = static_cast<uint16_t*>(entries);
    return hip_status(la::launch_fwd_tok(c, a, s), "la_recurrent_fwd_entries launch");
}

la_status la_recurrent_fwd_varlen(const la_config* cfg, const int32_t* cu_seqlens, const void* q,
                                  const void* k, const void* v, const void* g, const void* beta,
                                  const float* S0, void* o, float* S_T, void* stream) {
    CHECK(check_config(cfg, false));
    const la_config& c = *cfg;
    if ((c.kernel != LA_KERNEL_AUTO && c.kernel != LA_KERNEL_TOKEN) || c.solve != LA_SOLVE_EXACT)
        return fail(LA_ERR_UNSUPPORTED, "packed sequences run on the per-token kernel only (kernel=%d, solve=%d)",
                    c.kernel, c.solve);
    const bool units = c.B > 0 && c.H > 0;
    const bool work = units && c.T > 0;
    CHECK(check_ptr(cu_seqlens, "cu_seqlens", units));
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(o, "o", work));
    CHECK(check_ptr(S0, "S0", false));
    CHECK(check_ptr(S_T, "S_T", false));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!units) return ok();
    if (c.T == 0) {
        if (!S_T) return ok();
        return hip_status(la::launch_copy_state(c, S0, S_T, s), "copy S0 -> S_T");
    }
    la::FwdArgs a{q, k, v, g, beta, S0, o, S_T, nullptr};
    a.cu_seqlens = cu_seqlens;
    return hip_status(la::launch_fwd_tok(c, a, s), "la_recurrent_fwd_varlen launch");
}

la_status la_decode_step(const la_config* cfg, const void* q, const void* k, const void* v,
                         const void* g, const void* beta, float* S, void* o, void* codes,
                         float* scales, void* stream) {
    CHECK(check_config(cfg, true));
    const la_config& c = *cfg;
    const bool work = c.B > 0 && c.H > 0;
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(S, "S", work));
    CHECK(check_ptr(o, "o", work));
    CHECK(check_ptr(codes, "codes", false));
    CHECK(check_ptr(scales, "scales", false));
    if ((codes || scales) && c.qdq == LA_QDQ_NONE)
        return fail(LA_ERR_INVALID_ARG, "codes/scales requested without a quantizer");
    if (!work) return ok();
    la::DecodeArgs a{q, k, v, g, beta, S, o, codes, scales};
    return hip_status(la::launch_decode(c, a, static_cast<hipStream_t>(stream)), "la_decode_step launch");
}

la_status la_decode_step_slots(const la_config* cfg, const void* q, const void* k, const void* v,
                               const void* g, const void* beta, float* S_pool, const int32_t* slots,
                               int32_t n_slots, void* o, void* codes, float* scales, void* stream) {
    CHECK(check_config(cfg, true));
    const la_config& c = *cfg;
    const bool work = c.B > 0 && c.H > 0;
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(S_pool, "S_pool", work));
    CHECK(check_ptr(slots, "slots", work));
    CHECK(check_ptr(o, "o", work));
    CHECK(check_ptr(codes, "codes", false));
    CHECK(check_ptr(scales, "scales", false));
    if (n_slots < 1) return fail(LA_ERR_INVALID_ARG, "n_slots must be >= 1 (slot 0 is reserved), got %d", n_slots);
    if ((codes || scales) && c.qdq == LA_QDQ_NONE)
        return fail(LA_ERR_INVALID_ARG, "codes/scales requested without a quantizer");
    if (!work) return ok();
    la::DecodeArgs a{q, k, v, g, beta, S_pool, o, codes, scales};
    a.slots = slots;
    a.n_slots = n_slots;
    return hip_status(la::launch_decode(c, a, static_cast<hipStream_t>(stream)), "la_decode_step_slots launch");
}

la_status la_decode_step_replay(const la_config* cfg, const void* q, const void* k, const void* v,
                                const void* g, const void* beta, float* S, void* log_k, void* log_d,
                                float* log_g, const int32_t* pos, void* o, void* codes, float* scales,
                                void* stream) {
    CHECK(check_config(cfg, true));
    const la_config& c = *cfg;
    if (!c.replay) return fail(LA_ERR_INVALID_ARG, "la_decode_step_replay needs cfg->replay = 1");
    if (c.hadamard && c.state_rotated)
        return fail(LA_ERR_UNSUPPORTED, "replay decode carries the unrotated state (state_rotated must be 0)");
    const bool work = c.B > 0 && c.H > 0;
    const bool logs = work && c.qdq_interval > 1;
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(S, "S", work));
    CHECK(check_ptr(o, "o", work));
    CHECK(check_ptr(pos, "pos", work));
    CHECK(check_ptr(log_k, "log_k", logs));
    CHECK(check_ptr(log_d, "log_d", logs));
    CHECK(check_ptr(log_g, "log_g", logs));
    CHECK(check_ptr(codes, "codes", false));
    CHECK(check_ptr(scales, "scales", false));
    if (!work) return ok();
    la::DecodeArgs a{q, k, v, g, beta, S, o, codes, scales};
    a.pos = pos;
    a.log_k = static_cast<uint16_t*>(log_k);
    a.log_d = static_cast<uint16_t*>(log_d);
    a.log_g = log_g;
    a.window = c.qdq_interval;
    return hip_status(la::launch_decode(c, a, static_cast<hipStream_t>(stream)), "la_decode_step_replay launch");
}

size_t la_bwd_varlen_workspace_bytes(const la_config* cfg) {
    if (check_config(cfg, false) != LA_OK || cfg->ckpt_interval < 1) return 0;
    if ((cfg->kernel != LA_KERNEL_AUTO && cfg->kernel != LA_KERNEL_TOKEN) || cfg->solve != LA_SOLVE_EXACT) return 0;
    return ws_layout_varlen(*cfg).total;
}

la_status la_recurrent_bwd_ste_varlen(const la_config* cfg, const int32_t* cu_seqlens, const void* q,
                                      const void* k, const void* v, const void* g, const void* beta,
                                      const float* S0, const float* dout, const float* dS_T, float* dq,
                                      float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                                      void* workspace, size_t ws_bytes, void* stream) {
    CHECK(check_config(cfg, false));
    return la::bwd_varlen(*cfg, cu_seqlens, nullptr, 0, q, k, v, g, beta, S0, dout, dS_T, dq, dk, dv, dg, dbeta,
                          dS0, workspace, ws_bytes, stream);
}

la_status la_recurrent_fwd_split(const la_config* prefix_cfg, const la_config* suffix_cfg,
                                 const int32_t* cu_seqlens, const int32_t* prefix_len, const void* q,
                                 const void* k, const void* v, const void* g, const void* beta,
                                 const float* S0, void* o, float* S_mid, float* S_T, void* stream) {
    CHECK(la::check_split(prefix_cfg, suffix_cfg));
    const la_config& c = *prefix_cfg;
    const bool units = c.B > 0 && c.H > 0;
    const bool work = units && c.T > 0;
    CHECK(check_ptr(cu_seqlens, "cu_seqlens", units));
    CHECK(check_ptr(prefix_len, "prefix_len", units));
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(o, "o", work));
    CHECK(check_ptr(S0, "S0", false));
    CHECK(check_ptr(S_mid, "S_mid", units));
    CHECK(check_ptr(S_T, "S_T", false));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!units) return ok();
    la::FwdArgs a{q, k, v, g, beta, S0, o, S_mid, nullptr};
    a.cu_seqlens = cu_seqlens;
    a.split = prefix_len;
    a.split_part = 0;
    CHECK(hip_status(la::launch_fwd_tok(c, a, s), "la_recurrent_fwd_split prefix launch"));
    la::FwdArgs b{q, k, v, g, beta, S_mid, o, S_T, nullptr};
    b.cu_seqlens = cu_seqlens;
    b.split = prefix_len;
    b.split_part = 1;
    return hip_status(la::launch_fwd_tok(*suffix_cfg, b, s), "la_recurrent_fwd_split suffix launch");
}

size_t la_bwd_split_workspace_bytes(const la_config* prefix_cfg, const la_config* suffix_cfg) {
    if (la::check_split(prefix_cfg, suffix_cfg) != LA_OK) return 0;
    if (prefix_cfg->ckpt_interval < 1 || suffix_cfg->ckpt_interval < 1) return 0;
    const size_t a = ws_layout_varlen(*prefix_cfg).total, b = ws_layout_varlen(*suffix_cfg).total;
    const la_config& c = *prefix_cfg;
    return round_up(static_cast<size_t>(c.B) * c.H * c.d_k * c.d_v * sizeof(float)) + (a > b ? a : b);
}

la_status la_recurrent_bwd_ste_split(const la_config* prefix_cfg, const la_config* suffix_cfg,
                                     const int32_t* cu_seqlens, const int32_t* prefix_len, const void* q,
                                     const void* k, const void* v, const void* g, const void* beta,
                                     const float* S0, const float* S_mid, const float* dout,
                                     const float* dS_T, float* dq, float* dk, float* dv, float* dg,
                                     float* dbeta, float* dS0, void* workspace, size_t ws_bytes,
                                     void* stream) {
    CHECK(la::check_split(prefix_cfg, suffix_cfg));
    const la_config& c = *prefix_cfg;
    const bool units = c.B > 0 && c.H > 0;
    CHECK(check_ptr(S_mid, "S_mid", units));
    CHECK(check_ptr(prefix_len, "prefix_len", units));
    CHECK(check_ptr(workspace, "workspace", false));
    if (!units) return ok();
    const size_t need = la_bwd_split_workspace_bytes(prefix_cfg, suffix_cfg);
    if (need == 0) return fail(LA_ERR_INVALID_ARG, "backward needs ckpt_interval >= 1 in both configurations");
    if (!workspace || ws_bytes < need)
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? ws_bytes : static_cast<size_t>(0));
    // suffix first: its dS0 is the gradient at the handoff, the prefix's dS_T
    const size_t mid_bytes = round_up(static_cast<size_t>(c.B) * c.H * c.d_k * c.d_v * sizeof(float));
    float* dS_mid = static_cast<float*>(workspace);
    void* ws = static_cast<char*>(workspace) + mid_bytes;
    CHECK(la::bwd_varlen(*suffix_cfg, cu_seqlens, prefix_len, 1, q, k, v, g, beta, S_mid, dout, dS_T, dq, dk, dv, dg,
                         dbeta, dS_mid, ws, ws_bytes - mid_bytes, stream));
    return la::bwd_varlen(*prefix_cfg, cu_seqlens, prefix_len, 0, q, k, v, g, beta, S0, dout, dS_mid, dq, dk, dv, dg,
                          dbeta, dS0, ws, ws_bytes - mid_bytes, stream);
}

size_t la_bwd_workspace_bytes(const la_config* cfg) {
    if (check_config(cfg, false) != LA_OK || check_kernel(*cfg) != LA_OK || cfg->ckpt_interval < 1) return 0;
    if (la::bwd_kernel(*cfg) == LA_KERNEL_CHUNK)
        return cfg->ckpt_interval == la::kChunkTokens ? la::chunk_bwd_layout(*cfg).total : 0;
    return ws_layout(*cfg).total;
}

la_status la_recurrent_bwd_ste(const la_config* cfg, const void* q, const void* k,
                               const void* v, const void* g, const void* beta, const float* S0,
                               const float* ckpts, const float* dout, const float* dS_T,
                               float* dq, float* dk, float* dv, float* dg, float* dbeta,
                               float* dS0, void* workspace, size_t ws_bytes, void* stream) {
    return la::bwd_ste(cfg, q, k, v, g, beta, S0, ckpts, dout, dS_T, dq, dk, dv, dg, dbeta, dS0, workspace,
                       ws_bytes, nullptr, stream);
}

}  // extern "C"

namespace la {

la_status bwd_ste(const la_config* cfg, const void* q, const void* k, const void* v, const void* g,
                  const void* beta, const float* S0, const float* ckpts, const float* dout,
                  const float* dS_T, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                  float* dS0, void* workspace, size_t ws_bytes, WorkspaceProvider provide, void* stream) {
    CHECK(check_config(cfg, false));
    const la_config& c = *cfg;
    CHECK(check_kernel(c));
    const bool chunk = la::bwd_kernel(c) == LA_KERNEL_CHUNK;
    if (chunk && c.ckpt_interval != la::kChunkTokens)
        return fail(LA_ERR_UNSUPPORTED, "the chunk form's backward takes a checkpoint per chunk (ckpt_interval = 64)");
    if (c.ckpt_interval < 1) return fail(LA_ERR_INVALID_ARG, "backward needs ckpt_interval >= 1");
    const bool units = c.B > 0 && c.H > 0;
    const bool work = units && c.T > 0;
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(dout, "dout", work));
    CHECK(check_ptr(dq, "dq", work));
    CHECK(check_ptr(dk, "dk", work));
    CHECK(check_ptr(dv, "dv", work));
    CHECK(check_ptr(dg, "dg", work));
    CHECK(check_ptr(dbeta, "dbeta", work));
    CHECK(check_ptr(dS0, "dS0", units));
    CHECK(check_ptr(S0, "S0", false));
    CHECK(check_ptr(ckpts, "ckpts", false));
    CHECK(check_ptr(dS_T, "dS_T", false));
    CHECK(check_ptr(workspace, "workspace", false));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!units) return ok();
    if (c.T == 0) return hip_status(la::launch_copy_state(c, dS_T, dS0, s), "copy dS_T -> dS0");
    WsLayout L = ws_layout(c);
    if (chunk) L.total = la::chunk_bwd_layout(c).total;
    if (provide) {
        // the allocation-free entry point: its fixed device array must hold the workspace
        if (ws_bytes < L.total)
            return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, the allocation-free entry point's "
                        "device array holds %zu", L.total, ws_bytes);
        CHECK(hip_status(provide(&workspace), "device array of the allocation-free entry point"));
        CHECK(check_ptr(workspace, "device array", true));
    }
    if (!workspace || ws_bytes < L.total)
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                    workspace ? ws_bytes : static_cast<size_t>(0));
    char* ws = static_cast<char*>(workspace);
    if (chunk) {
        la::FwdArgs fa{q, k, v, g, beta, S0, nullptr, nullptr, nullptr};
        la::BwdArgs a{q, k, v, g, beta, ckpts, dout, dS_T, dq, dk, dv, dg, dbeta, dS0, nullptr, nullptr};
        return hip_status(la::launch_chunk_bwd(c, fa, a, ws, s), "la_recurrent_bwd_ste chunk launch");
    }
    if (la::bwd_kernel(c) == LA_KERNEL_BLOCK) {
        float* states = reinterpret_cast<float*>(ws + L.states);
        la::FwdArgs fa{q, k, v, g, beta, S0, nullptr, nullptr, nullptr};
        la::BwdArgs a{q, k, v, g, beta, ckpts, dout, dS_T, dq, dk, dv, dg, dbeta, dS0,
                      states, reinterpret_cast<float*>(ws + L.part)};
        return hip_status(la::launch_bwd_mfma(c, fa, a, reinterpret_cast<float*>(ws + L.carry),
                                              reinterpret_cast<float*>(ws + L.ckpts), s),
                          "la_recurrent_bwd_ste launch");
    }
    const float* ck = ckpts;
    if (!ck) {
        float* ckw = reinterpret_cast<float*>(ws + L.ckpts);
        la::FwdArgs fa{q, k, v, g, beta, S0, nullptr, nullptr, ckw};
        la_status st = hip_status(la::launch_fwd(c, fa, s), "checkpoint recompute launch");
        if (st != LA_OK) return st;
        ck = ckw;
    }
    la::BwdArgs a{q, k, v, g, beta, ck, dout, dS_T, dq, dk, dv, dg, dbeta, dS0,
                  reinterpret_cast<float*>(ws + L.states), reinterpret_cast<float*>(ws + L.part)};
    return hip_status(la::launch_bwd(c, a, s), "la_recurrent_bwd_ste launch");
}

}  // namespace la

namespace la {

la_status check_split(const la_config* a, const la_config* b) {
    CHECK(check_config(a, false));
    CHECK(check_config(b, false));
    if (a->B != b->B || a->T != b->T || a->H != b->H || a->d_k != b->d_k || a->d_v != b->d_v ||
        a->gate != b->gate || a->qkv_dtype != b->qkv_dtype || a->gate_dtype != b->gate_dtype ||
        a->out_dtype != b->out_dtype)
        return fail(LA_ERR_INVALID_ARG, "prefix and suffix configurations differ in shape, gate or dtypes");
    if (a->state_rotated || b->state_rotated)
        return fail(LA_ERR_UNSUPPORTED, "the handoff state is the unrotated S (state_rotated must be 0)");
    for (const la_config* c : {a, b})
        if ((c->kernel != LA_KERNEL_AUTO && c->kernel != LA_KERNEL_TOKEN) || c->solve != LA_SOLVE_EXACT)
            return fail(LA_ERR_UNSUPPORTED, "packed sequences run on the per-token kernel only (kernel=%d, solve=%d)",
                        c->kernel, c->solve);
    return LA_OK;
}

la_status bwd_varlen(const la_config& c, const int32_t* cu_seqlens, const int32_t* split, int part, const void* q,
                     const void* k, const void* v, const void* g, const void* beta, const float* S0,
                     const float* dout, const float* dS_T, float* dq, float* dk, float* dv, float* dg,
                     float* dbeta, float* dS0, void* workspace, size_t ws_bytes, void* stream) {
    if ((c.kernel != LA_KERNEL_AUTO && c.kernel != LA_KERNEL_TOKEN) || c.solve != LA_SOLVE_EXACT)
        return fail(LA_ERR_UNSUPPORTED, "packed sequences run on the per-token kernel only (kernel=%d, solve=%d)",
                    c.kernel, c.solve);
    if (c.ckpt_interval < 1) return fail(LA_ERR_INVALID_ARG, "backward needs ckpt_interval >= 1");
    const bool units = c.B > 0 && c.H > 0;
    const bool work = units && c.T > 0;
    CHECK(check_ptr(cu_seqlens, "cu_seqlens", units));
    CHECK(check_ptr(q, "q", work));
    CHECK(check_ptr(k, "k", work));
    CHECK(check_ptr(v, "v", work));
    CHECK(check_ptr(g, "g", work));
    CHECK(check_ptr(beta, "beta", work));
    CHECK(check_ptr(dout, "dout", work));
    CHECK(check_ptr(dq, "dq", work));
    CHECK(check_ptr(dk, "dk", work));
    CHECK(check_ptr(dv, "dv", work));
    CHECK(check_ptr(dg, "dg", work));
    CHECK(check_ptr(dbeta, "dbeta", work));
    CHECK(check_ptr(dS0, "dS0", units));
    CHECK(check_ptr(S0, "S0", false));
    CHECK(check_ptr(dS_T, "dS_T", false));
    CHECK(check_ptr(workspace, "workspace", false));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!units) return ok();
    if (c.T == 0) return hip_status(launch_copy_state(c, dS_T, dS0, s), "copy dS_T -> dS0");
    const WsLayout L = ws_layout_varlen(c);
    if (!workspace || ws_bytes < L.total)
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                    workspace ? ws_bytes : static_cast<size_t>(0));
    char* ws = static_cast<char*>(workspace);
    float* ckw = reinterpret_cast<float*>(ws + L.ckpts);
    FwdArgs fa{q, k, v, g, beta, S0, nullptr, nullptr, ckw};
    fa.cu_seqlens = cu_seqlens;
    fa.split = split;
    fa.split_part = part;
    CHECK(hip_status(launch_fwd_tok(c, fa, s), "checkpoint recompute launch"));
    BwdArgs a{q, k, v, g, beta, ckw, dout, dS_T, dq, dk, dv, dg, dbeta, dS0,
              reinterpret_cast<float*>(ws + L.states), reinterpret_cast<float*>(ws + L.part)};
    a.cu_seqlens = cu_seqlens;
    a.split = split;
    a.split_part = part;
    return hip_status(launch_bwd(c, a, s), "packed backward launch");
}

}  // namespace la
