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
};

WsLayout ws_layout(const la_config& c) {
    WsLayout L;
    if (la::bwd_mfma_eligible(c)) {
        // block backward: the state entering every 16-token block, then the partial records
        L.states = 0;
        L.part = round_up(la::bwd_mfma_state_bytes(c));
        L.ckpts = L.part + round_up(la::bwd_mfma_part_bytes(c));
        L.total = L.ckpts;
        return L;
    }
    // the backward runs in the token layout: tiles of tok_tile_cols value columns
    const size_t tc = static_cast<size_t>(la::tok_tile_cols(c.d_k, c.qdq, c.group));
    const size_t tiles = static_cast<size_t>(la::tok_tiles(c));
    const size_t nwg = static_cast<size_t>(c.B) * c.H * tiles;
    L.states = 0;
    L.part = round_up(nwg * static_cast<size_t>(la::n_sub_states(c)) * c.d_k * tc * sizeof(float));
    L.ckpts = L.part + round_up(tiles * c.B * c.T * c.H * la::part_width(c) * sizeof(float));
    L.total = L.ckpts + round_up(static_cast<size_t>(c.B) * c.H * la::n_ckpts(c) * c.d_k * c.d_v * sizeof(float));
    return L;
}

}  // namespace

extern "C" {

const char* la_status_string(la_status s) {
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

const char* la_last_error(void) { return g_err; }

const char* la_fwd_kernel_name(const la_config* cfg) {
    if (check_config(cfg, false) != LA_OK) return "";
    return la::fwd_kernel_name(*cfg);
}

const char* la_bwd_kernel_name(const la_config* cfg) {
    if (check_config(cfg, false) != LA_OK) return "";
    return la::bwd_mfma_eligible(*cfg) ? "block" : "token";
}

la_status la_recurrent_fwd(const la_config* cfg, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, const float* S0, void* o,
                           float* S_T, float* ckpts, void* stream) {
    CHECK(check_config(cfg, false));
    const la_config& c = *cfg;
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

la_status la_recurrent_fwd_varlen(const la_config* cfg, const int32_t* cu_seqlens, const void* q,
                                  const void* k, const void* v, const void* g, const void* beta,
                                  const float* S0, void* o, float* S_T, void* stream) {
    CHECK(check_config(cfg, false));
    const la_config& c = *cfg;
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

size_t la_bwd_workspace_bytes(const la_config* cfg) {
    if (check_config(cfg, false) != LA_OK || cfg->ckpt_interval < 1) return 0;
    return ws_layout(*cfg).total;
}

la_status la_recurrent_bwd_ste(const la_config* cfg, const void* q, const void* k,
                               const void* v, const void* g, const void* beta, const float* S0,
                               const float* ckpts, const float* dout, const float* dS_T,
                               float* dq, float* dk, float* dv, float* dg, float* dbeta,
                               float* dS0, void* workspace, size_t ws_bytes, void* stream) {
    CHECK(check_config(cfg, false));
    const la_config& c = *cfg;
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
    const WsLayout L = ws_layout(c);
    if (!workspace || ws_bytes < L.total)
        return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                    workspace ? ws_bytes : static_cast<size_t>(0));
    char* ws = static_cast<char*>(workspace);
    if (la::bwd_mfma_eligible(c)) {
        float* dense = reinterpret_cast<float*>(ws + L.states);
        la::FwdArgs fa{q, k, v, g, beta, S0, nullptr, nullptr, dense};
        la::BwdArgs a{q, k, v, g, beta, dense, dout, dS_T, dq, dk, dv, dg, dbeta, dS0,
                      dense, reinterpret_cast<float*>(ws + L.part)};
        return hip_status(la::launch_bwd_mfma(c, fa, a, s), "la_recurrent_bwd_ste launch");
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

}  // extern "C"
