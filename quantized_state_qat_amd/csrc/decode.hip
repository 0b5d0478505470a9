// Single-token batched decode: the FP32 state is streamed HBM -> VGPR -> HBM in place.
//
// One workgroup per (sequence, head, 64-column value tile), laid out as 16 column quads x
// (d_k / R) row groups: thread (rg, cq) holds rows [rg*R, rg*R + R) of the four columns
// 4cq..4cq+3, loaded as float4 so that every wave reads 256-byte contiguous row segments.
// The state is streamed with non-temporal loads and stores (it is touched once per step).  One pass over the state produces both key-axis reductions the
// token needs, u = S~^T k and r = S~^T q, because the output read before rounding is
//     o = S'^T q = S~^T q + delta (k . q),
// so a single reduction round (in-thread over R rows, across the 4 row groups of a wave
// with permlane swaps, across the 4 waves through LDS in a fixed order) precedes the update.
// INT8 groups are 4..16 consecutive quads of one row (DPP within a row of 16 lanes).
#include "la_device.hpp"
#include "la_internal.hpp"

namespace la {

struct DecParams {
    int H, dv;
    int qkv_dt, gate_dt, out_dt;
    int rot;  // Hadamard mode with the state held rotated (Y = Hu S)
    int sort_slots;  // slot pool: visit the entries in slot order (slot_rank_pick)
};

template <int DK, int NW>
struct DecSmem {
    float k[DK], a[DK], ak[DK], aq[DK];
    float q[DK];
    float beta, kqp[2];
    float4 red[NW][16][2];
    float amax[NW];
};

typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float* p) {
    v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_nt(float* p, float4 x) {
    v4f v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p));
}

// 4 consecutive elements starting at element idx (idx % 4 == 0), float32 or bfloat16.
__device__ __forceinline__ float4 load4(const void* p, size_t idx, int dtype) {
    if (dtype == 0) return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + idx);
    uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + idx);
    return make_float4(bf16_bits_to_f32(u.x & 0xFFFFu), bf16_bits_to_f32(u.x >> 16),
                       bf16_bits_to_f32(u.y & 0xFFFFu), bf16_bits_to_f32(u.y >> 16));
}

__device__ __forceinline__ void store4(void* p, size_t idx, int dtype, float4 x) {
    if (dtype == 0) {
        *reinterpret_cast<float4*>(static_cast<float*>(p) + idx) = x;
    } else {
        uint2 u;
        u.x = static_cast<uint32_t>(f32_to_bf16_bits(x.x)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.y)) << 16);
        u.y = static_cast<uint32_t>(f32_to_bf16_bits(x.z)) | (static_cast<uint32_t>(f32_to_bf16_bits(x.w)) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + idx) = u;
    }
}

__device__ __forceinline__ float4 rows_sum4(float4 x) {
    return make_float4(rows_sum(x.x), rows_sum(x.y), rows_sum(x.z), rows_sum(x.w));
}
__device__ __forceinline__ float4 add4(float4 x, float4 y) {
    return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
}
__device__ __forceinline__ float max4abs(float4 x) {
    return fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
}

// In-LDS unnormalized Walsh-Hadamard transform over the key axis of a DK x 64 tile
// (all NT threads call).
template <int DK, int NT>
__device__ __forceinline__ void dec_tile_wht(float* tile) {
#pragma unroll 1
    for (int hs = 1; hs < DK; hs <<= 1) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < DK * 32; idx += NT) {
            int c = idx & 63, pp = idx >> 6;
            int i = (pp / hs) * 2 * hs + (pp % hs);
            float x0 = tile[i * 64 + c], x1 = tile[(i + hs) * 64 + c];
            tile[i * 64 + c] = x0 + x1;
            tile[(i + hs) * 64 + c] = x0 - x1;
        }
    }
    __syncthreads();
}

// Slot-ordered visiting of a slot pool.  A serving batch names its pool slots in any order;
// visited in entry order, the step streams 1 MB states scattered over the pool (256 shuffled
// slots of a 769-slot pool: 102.5 us per step, against 91.6 us for the same slots in
// increasing order).  Each workgroup therefore ranks the batch's entries (padding entries
// first, in entry order, then the valid entries by increasing slot) and serves the entry whose
// rank is its blockIdx.z, so that consecutive workgroups walk the pool in address order.  The
// ranking is a bitmap of the named slots in LDS with per-word prefix counts; every workgroup
// computes the same ranking, so workgroups and entries stay in one-to-one correspondence.  If
// two entries name the same valid slot (a caller error: their updates race) the number of
// distinct slots falls short of the number of valid entries, and every workgroup keeps the
// identity map instead.  Used for B <= kSortPerThread * NT and n_slots <= 32 kSortWords.
constexpr int kSortWords = 512;
constexpr int kSortPerThread = 4;

template <int NW>
struct SlotRankSmem {
    unsigned bm[kSortWords];  // bit s: slot s is named by a valid entry
    int pre[kSortWords];      // set bits in the words before this one
    int npad[kSortPerThread][NW];
    int wsum[NW];
    int pick;
};

template <int NT>
__device__ __forceinline__ int slot_rank_pick(const int32_t* slots, int B, int n_slots, SlotRankSmem<NT / 64>& ss) {
    constexpr int NW = NT / 64, WPT = kSortWords / NT;
    static_assert(kSortWords % NT == 0, "bitmap words per thread");
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int z = blockIdx.z;
#pragma unroll
    for (int j = 0; j < WPT; j++) ss.bm[WPT * tid + j] = 0u;
    if (tid == 0) ss.pick = z;
    __syncthreads();
    int sl[kSortPerThread];
    unsigned long long padmask[kSortPerThread];
#pragma unroll
    for (int i = 0; i < kSortPerThread; i++) {
        const int e = i * NT + tid;
        sl[i] = e < B ? slots[e] : 0;
        const bool valid = sl[i] > 0 && sl[i] < n_slots;
        if (valid) atomicOr(&ss.bm[sl[i] >> 5], 1u << (sl[i] & 31));
        padmask[i] = __ballot(e < B && !valid);
        if (lane == 0) ss.npad[i][w] = __popcll(padmask[i]);
    }
    __syncthreads();
    // exclusive prefix of the words' bit counts: WPT words per thread, a scan across the
    // wave's lanes, then the totals of the waves before
    int cnt[WPT], local = 0;
#pragma unroll
    for (int j = 0; j < WPT; j++) {
        cnt[j] = __popc(ss.bm[WPT * tid + j]);
        local += cnt[j];
    }
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
    }
    if (lane == 63) ss.wsum[w] = incl;
    __syncthreads();
    int run = incl - local, distinct = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ww++) {
        run += ww < w ? ss.wsum[ww] : 0;
        distinct += ss.wsum[ww];
    }
#pragma unroll
    for (int j = 0; j < WPT; j++) {
        ss.pre[WPT * tid + j] = run;
        run += cnt[j];
    }
    int npad = 0;
#pragma unroll
    for (int i = 0; i < kSortPerThread; i++)
#pragma unroll
        for (int ww = 0; ww < NW; ww++) npad += ss.npad[i][ww];
    __syncthreads();
    if (distinct != B - npad) return z;  // a valid slot named twice: identity map
    int before = 0;  // padding entries before this thread's entry of pass i
#pragma unroll
    for (int i = 0; i < kSortPerThread; i++) {
        const int e = i * NT + tid;
        int pb = before;
#pragma unroll
        for (int ww = 0; ww < NW; ww++) pb += ww < w ? ss.npad[i][ww] : 0;
        pb += __popcll(padmask[i] & ((1ull << lane) - 1ull));
        if (e < B) {
            const bool valid = sl[i] > 0 && sl[i] < n_slots;
            const int rank = valid ? npad + ss.pre[sl[i] >> 5] + __popc(ss.bm[sl[i] >> 5] & ((1u << (sl[i] & 31)) - 1u))
                                   : pb;
            if (rank == z) ss.pick = e;
        }
#pragma unroll
        for (int ww = 0; ww < NW; ww++) before += ss.npad[i][ww];
    }
    __syncthreads();
    return ss.pick;
}

template <int DK, int R, int QMODE, int G, bool HAD, bool KDA, bool CODES>
__global__ __launch_bounds__(16 * (DK / R)) void decode_kernel(DecParams p, DecodeArgs a) {
    constexpr int NT = 16 * (DK / R);  // threads
    constexpr int NW = NT / 64;        // waves
    __shared__ DecSmem<DK, NW> sm;
    __shared__ float tile[HAD ? DK * 64 : 1];
    __shared__ SlotRankSmem<NW> ss;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cq = tid & 15, rg = tid >> 4;
    const int blk = blockIdx.x, h = blockIdx.y;
    const int b = a.slots && p.sort_slots ? slot_rank_pick<NT>(a.slots, gridDim.z, a.n_slots, ss) : blockIdx.z;
    const int H = p.H, DV = p.dv;
    const size_t tok = static_cast<size_t>(b) * H + h;  // T == 1
    const int col0 = blk * 64 + cq * 4;
    // the state this entry advances: S[b], or pool slot slots[b] (slot 0 and indices outside
    // the pool are padding: zero output, nothing else written; uniform over the workgroup)
    size_t stok = tok;
    if (a.slots) {
        const int sl = a.slots[b];
        if (sl <= 0 || sl >= a.n_slots) {
            if (rg == 0) store4(a.o, tok * DV + col0, p.out_dt, make_float4(0.f, 0.f, 0.f, 0.f));
            return;
        }
        stok = static_cast<size_t>(sl) * H + h;
    }
    float* Srow = a.S + (stok * DK + static_cast<size_t>(rg) * R) * DV + col0;

    // token vectors first, so that waiting for them does not wait for the state
    float kk = 0.f, qv = 0.f, ai = 0.f, gv = 0.f;
    if (tid < DK) {
        kk = load_elem(a.k, tok * DK + tid, p.qkv_dt);
        qv = load_elem(a.q, tok * DK + tid, p.qkv_dt);
        gv = KDA ? load_elem(a.g, tok * DK + tid, p.gate_dt) : load_elem(a.g, tok, p.gate_dt);
        ai = expf(gv);
    }
    const float beta = load_elem(a.beta, tok, p.gate_dt);
    const float4 vv = load4(a.v, tok * DV + col0, p.qkv_dt);
    float4 s[R];
#pragma unroll
    for (int m = 0; m < R; m++) s[m] = load_nt(Srow + static_cast<size_t>(m) * DV);

    // replay windows: the state entering the token is the window's checkpoint advanced by the
    // logged entries of its earlier tokens, S <- diag(exp g_i) S + k_i d_i^T in log order
    // (the carried update of the forward's replay tokens); pos is uniform per workgroup
    const int W1 = a.window - 1;
    const int pos = a.pos ? min(max(a.pos[b], 0), W1) : W1;
    const int npos = a.pos ? pos : 0;
    const size_t lbase = tok * static_cast<size_t>(W1 > 0 ? W1 : 1);
    // one entry's operands for this thread: its R rows of the key (R consecutive bf16 values,
    // one load), its four columns of the update (one 8-byte load) and the gate(s); loaded one
    // entry ahead of use so the loads overlap the previous entry's arithmetic
    struct Ent {
        uint32_t kw[(R + 1) / 2];
        uint2 dw;
        float g[KDA ? R : 1];
    };
    auto load_ent = [&](int i, Ent& en) __attribute__((always_inline)) {
        const size_t e = lbase + i;
        const uint16_t* kp = a.log_k + e * DK + rg * R;
        if constexpr (R == 8) {
            const uint4 x = *reinterpret_cast<const uint4*>(kp);
            en.kw[0] = x.x; en.kw[1] = x.y; en.kw[2] = x.z; en.kw[3] = x.w;
        } else if constexpr (R == 4) {
            const uint2 x = *reinterpret_cast<const uint2*>(kp);
            en.kw[0] = x.x; en.kw[1] = x.y;
        } else if constexpr (R == 2) {
            en.kw[0] = *reinterpret_cast<const uint32_t*>(kp);
        } else {
            en.kw[0] = *kp;
        }
        en.dw = *reinterpret_cast<const uint2*>(a.log_d + e * DV + col0);
        if constexpr (KDA) {
#pragma unroll
            for (int m = 0; m < R; m++) en.g[m] = a.log_g[e * DK + rg * R + m];
        } else {
            en.g[0] = a.log_g[e];
        }
    };
    Ent cur, nxt;
    if (npos > 0) load_ent(0, cur);
#pragma unroll 1
    for (int i = 0; i < npos; i++) {
        if (i + 1 < npos) load_ent(i + 1, nxt);
        const float4 dh = make_float4(bf16_bits_to_f32(cur.dw.x & 0xFFFFu), bf16_bits_to_f32(cur.dw.x >> 16),
                                      bf16_bits_to_f32(cur.dw.y & 0xFFFFu), bf16_bits_to_f32(cur.dw.y >> 16));
        const float ga = KDA ? 1.0f : expf(cur.g[0]);
#pragma unroll
        for (int m = 0; m < R; m++) {
            const float ar = KDA ? expf(cur.g[m]) : ga;
            const uint32_t kb = R == 1 ? cur.kw[0] : ((m & 1) ? (cur.kw[m / 2] >> 16) : (cur.kw[m / 2] & 0xFFFFu));
            const float kr = bf16_bits_to_f32(kb);
            s[m].x = __builtin_fmaf(kr, dh.x, ar * s[m].x);
            s[m].y = __builtin_fmaf(kr, dh.y, ar * s[m].y);
            s[m].z = __builtin_fmaf(kr, dh.z, ar * s[m].z);
            s[m].w = __builtin_fmaf(kr, dh.w, ar * s[m].w);
        }
        cur = nxt;
    }

    if (tid < DK) {
        sm.k[tid] = kk;
        sm.q[tid] = qv;
        sm.a[tid] = ai;
    }
    if (w < 2) {  // k . q: one partial per 64 keys, fixed butterfly order
        float kqp = wave_sum(tid < DK ? kk * qv : 0.0f);
        if (lane == 0) sm.kqp[w] = kqp;
    }
    if (HAD && !KDA && p.rot) {  // (per-key gates take only the unrotated state)
        // state held as Y = Hu S: rotate the key and query instead of the state.
        // u = Y~^T (Hu k) / d_k, Y' = Y~ + (Hu k) delta^T, o = Y~^T (Hu q) / d_k + delta (k . q).
#pragma unroll 1
        for (int hs = 1; hs < DK; hs <<= 1) {
            __syncthreads();
            if (tid < DK) {
                float* vec = (tid < DK / 2) ? sm.k : sm.q;
                int pp = tid & (DK / 2 - 1);
                int i = (pp / hs) * 2 * hs + (pp % hs);
                float x0 = vec[i], x1 = vec[i + hs];
                vec[i] = x0 + x1;
                vec[i + hs] = x0 - x1;
            }
        }
        __syncthreads();
        if (tid < DK) {
            constexpr float inv = 1.0f / DK;
            sm.ak[tid] = sm.a[tid] * (sm.k[tid] * inv);
            sm.aq[tid] = sm.a[tid] * (sm.q[tid] * inv);
        }
    } else if (tid < DK) {
        sm.ak[tid] = ai * kk;
        sm.aq[tid] = ai * qv;
    }
    __syncthreads();

    // one pass: u = S~^T k and r = S~^T q (partial over this thread's rows)
    float4 pu = make_float4(0.f, 0.f, 0.f, 0.f), pr = pu;
#pragma unroll
    for (int m = 0; m < R; m++) {
        const float wk = sm.ak[rg * R + m], wq = sm.aq[rg * R + m];
        pu.x = __builtin_fmaf(s[m].x, wk, pu.x);
        pu.y = __builtin_fmaf(s[m].y, wk, pu.y);
        pu.z = __builtin_fmaf(s[m].z, wk, pu.z);
        pu.w = __builtin_fmaf(s[m].w, wk, pu.w);
        pr.x = __builtin_fmaf(s[m].x, wq, pr.x);
        pr.y = __builtin_fmaf(s[m].y, wq, pr.y);
        pr.z = __builtin_fmaf(s[m].z, wq, pr.z);
        pr.w = __builtin_fmaf(s[m].w, wq, pr.w);
    }
    pu = rows_sum4(pu);
    pr = rows_sum4(pr);
    if (lane < 16) {
        sm.red[w][cq][0] = pu;
        sm.red[w][cq][1] = pr;
    }
    __syncthreads();
    float4 u = sm.red[0][cq][0], r = sm.red[0][cq][1];
#pragma unroll
    for (int ww = 1; ww < NW; ww++) {
        u = add4(u, sm.red[ww][cq][0]);
        r = add4(r, sm.red[ww][cq][1]);
    }
    const float kq = sm.kqp[0] + sm.kqp[1];
    const float4 dl = make_float4(beta * (vv.x - u.x), beta * (vv.y - u.y), beta * (vv.z - u.z), beta * (vv.w - u.w));
    if (rg == 0) {
        const float4 o = make_float4(__builtin_fmaf(dl.x, kq, r.x), __builtin_fmaf(dl.y, kq, r.y),
                                     __builtin_fmaf(dl.z, kq, r.z), __builtin_fmaf(dl.w, kq, r.w));
        store4(a.o, tok * DV + col0, p.out_dt, o);
    }
    if (a.pos && pos < W1) {
        // a replay token inside the window: append its entries (delta rounded once to BF16, the
        // key's BF16 bits, the log gate); the checkpoint is left as it is
        const size_t e = lbase + pos;
        if (rg == 0) {
            uint2 dw;
            dw.x = static_cast<uint32_t>(f32_to_bf16_bits(dl.x)) | (static_cast<uint32_t>(f32_to_bf16_bits(dl.y)) << 16);
            dw.y = static_cast<uint32_t>(f32_to_bf16_bits(dl.z)) | (static_cast<uint32_t>(f32_to_bf16_bits(dl.w)) << 16);
            *reinterpret_cast<uint2*>(a.log_d + e * DV + col0) = dw;
        }
        if (blk == 0 && tid < DK) {
            a.log_k[e * DK + tid] = f32_to_bf16_bits(kk);
            if (KDA) a.log_g[e * DK + tid] = gv;
            else if (tid == 0) a.log_g[e] = gv;
        }
        return;
    }

    // S' = diag(a) S + k delta^T
#pragma unroll
    for (int m = 0; m < R; m++) {
        const int row = rg * R + m;
        const float ar = sm.a[row], kr = sm.k[row];
        s[m].x = __builtin_fmaf(kr, dl.x, ar * s[m].x);
        s[m].y = __builtin_fmaf(kr, dl.y, ar * s[m].y);
        s[m].z = __builtin_fmaf(kr, dl.z, ar * s[m].z);
        s[m].w = __builtin_fmaf(kr, dl.w, ar * s[m].w);
    }

    if (HAD && !p.rot) {
        // S' -> Hu S' through LDS (key axis); quantize there; S = Hu Yhat / d_k afterwards
#pragma unroll
        for (int m = 0; m < R; m++) *reinterpret_cast<float4*>(&tile[(rg * R + m) * 64 + cq * 4]) = s[m];
        dec_tile_wht<DK, NT>(tile);
#pragma unroll
        for (int m = 0; m < R; m++) s[m] = *reinterpret_cast<const float4*>(&tile[(rg * R + m) * 64 + cq * 4]);
    }

    if (QMODE == LA_QDQ_INT8_GROUP) {
        constexpr int QPG = G / 4;  // quads per group
#pragma unroll
        for (int m = 0; m < R; m++) {
            const float mx = group_max_abs<QPG>(max4abs(s[m]));
            float sc, y;
            float4 c;
            if (int8_scale_recip(mx, sc, y)) {
                c = make_float4(int8_code_fast(s[m].x, sc, y), int8_code_fast(s[m].y, sc, y),
                                int8_code_fast(s[m].z, sc, y), int8_code_fast(s[m].w, sc, y));
            } else {
                c = make_float4(int8_code(s[m].x, sc), int8_code(s[m].y, sc), int8_code(s[m].z, sc),
                                int8_code(s[m].w, sc));
            }
            s[m] = make_float4(c.x * sc, c.y * sc, c.z * sc, c.w * sc);
            if (CODES) {
                const int row = rg * R + m;
                if (a.codes) {
                    char4 cc = make_char4(static_cast<signed char>(c.x), static_cast<signed char>(c.y),
                                          static_cast<signed char>(c.z), static_cast<signed char>(c.w));
                    *reinterpret_cast<char4*>(static_cast<int8_t*>(a.codes) + (tok * DK + row) * DV + col0) = cc;
                }
                if (a.scales && (cq % QPG) == 0) a.scales[(tok * DK + row) * (DV / G) + col0 / G] = sc;
            }
        }
    } else if (QMODE == LA_QDQ_E4M3_TILE) {
        float mx = 0.0f;
#pragma unroll
        for (int m = 0; m < R; m++) mx = fmaxf(mx, max4abs(s[m]));
        mx = group_max<64>(mx);
        if (lane == 0) sm.amax[w] = mx;
        __syncthreads();
        float amax = sm.amax[0];
#pragma unroll
        for (int ww = 1; ww < NW; ww++) amax = fmaxf(amax, sm.amax[ww]);
        const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
        const bool fast = sc >= kFastQuotMinScaleE4M3;
        const float y = 1.0f / sc;
#pragma unroll
        for (int m = 0; m < R; m++) {
            float4 e;
            if (fast) {
                e = make_float4(e4m3_round(quot_rn(s[m].x, sc, y)), e4m3_round(quot_rn(s[m].y, sc, y)),
                                e4m3_round(quot_rn(s[m].z, sc, y)), e4m3_round(quot_rn(s[m].w, sc, y)));
            } else {
                e = make_float4(e4m3_round(s[m].x / sc), e4m3_round(s[m].y / sc), e4m3_round(s[m].z / sc),
                                e4m3_round(s[m].w / sc));
            }
            s[m] = make_float4(e.x * sc, e.y * sc, e.z * sc, e.w * sc);
            if (CODES && a.codes) {
                const int row = rg * R + m;
                uchar4 cc = make_uchar4(e4m3_bits(e.x), e4m3_bits(e.y), e4m3_bits(e.z), e4m3_bits(e.w));
                *reinterpret_cast<uchar4*>(static_cast<uint8_t*>(a.codes) + (tok * DK + row) * DV + col0) = cc;
            }
        }
        if (CODES && a.scales && tid == 0) a.scales[tok * (DV / 64) + blk] = sc;
    }

    if (HAD && !p.rot) {
        __syncthreads();
#pragma unroll
        for (int m = 0; m < R; m++) *reinterpret_cast<float4*>(&tile[(rg * R + m) * 64 + cq * 4]) = s[m];
        dec_tile_wht<DK, NT>(tile);
        constexpr float inv = 1.0f / DK;
#pragma unroll
        for (int m = 0; m < R; m++) {
            float4 y = *reinterpret_cast<const float4*>(&tile[(rg * R + m) * 64 + cq * 4]);
            s[m] = make_float4(y.x * inv, y.y * inv, y.z * inv, y.w * inv);
        }
    }

#pragma unroll
    for (int m = 0; m < R; m++) store_nt(Srow + static_cast<size_t>(m) * DV, s[m]);
}

// Rows per thread: 8 at d_k = 128 (256 threads; measured faster than 4 or 2 rows per thread
// for the in-place stream), one row group per 16 rows otherwise.
#ifndef LA_DECODE_R128
#define LA_DECODE_R128 8
#endif
template <int DK>
constexpr int dec_rows() { return DK == 128 ? LA_DECODE_R128 : DK / 16; }

// At d_k = 128 the in-place stream runs fastest with three workgroups (twelve waves) per CU
// in flight: measured on the B=256 H=16 batch, 91 us per step at three, 93 at two and 96 at
// four or more (the register budget alone admits five).  LDS is the resource that caps it:
// each workgroup asks for enough dynamic LDS (never accessed) that its total reaches
// kDecLdsPerWg, and a fourth no longer fits in a CU's 160 KiB.
constexpr size_t kDecLdsPerCu = 160 * 1024;
constexpr size_t kDecLdsPerWg = 44 * 1024;
static_assert(kDecLdsPerCu / kDecLdsPerWg == 3, "three workgroups per CU");

template <int DK, int QMODE, int G, bool HAD, bool KDA>
static hipError_t launch_dec_t(const la_config& c, const DecodeArgs& a, hipStream_t s) {
    DecParams p;
    p.H = c.H; p.dv = c.d_v; p.qkv_dt = c.qkv_dtype; p.gate_dt = c.gate_dtype; p.out_dt = c.out_dtype;
    p.rot = c.hadamard && c.state_rotated;
    constexpr int R = dec_rows<DK>();
    constexpr int NT = 16 * (DK / R);
    p.sort_slots = a.slots && c.B <= kSortPerThread * NT && a.n_slots <= 32 * kSortWords;
    constexpr size_t lds_static = sizeof(DecSmem<DK, NT / 64>) + sizeof(SlotRankSmem<NT / 64>) + sizeof(float) * (HAD ? DK * 64 : 1);
    constexpr size_t lds_dyn = DK == 128 && lds_static < kDecLdsPerWg ? kDecLdsPerWg - lds_static : 0;
    dim3 grid(c.d_v / 64, c.H, c.B);
    if (a.codes || a.scales)
        hipLaunchKernelGGL((decode_kernel<DK, R, QMODE, G, HAD, KDA, true>), grid, dim3(NT), lds_dyn, s, p, a);
    else
        hipLaunchKernelGGL((decode_kernel<DK, R, QMODE, G, HAD, KDA, false>), grid, dim3(NT), lds_dyn, s, p, a);
    return hipGetLastError();
}

template <int DK>
static hipError_t launch_dec_dk(const la_config& c, const DecodeArgs& a, hipStream_t s) {
    const bool kda = c.gate == LA_GATE_KEY;
    if (c.qdq == LA_QDQ_NONE)
        return kda ? launch_dec_t<DK, LA_QDQ_NONE, 4, false, true>(c, a, s)
                   : launch_dec_t<DK, LA_QDQ_NONE, 4, false, false>(c, a, s);
    if (c.qdq == LA_QDQ_E4M3_TILE)
        return kda ? launch_dec_t<DK, LA_QDQ_E4M3_TILE, 64, false, true>(c, a, s)
                   : launch_dec_t<DK, LA_QDQ_E4M3_TILE, 64, false, false>(c, a, s);
    if (c.hadamard) {
        switch (c.group) {
            case 16: return kda ? launch_dec_t<DK, LA_QDQ_INT8_GROUP, 16, true, true>(c, a, s)
                                : launch_dec_t<DK, LA_QDQ_INT8_GROUP, 16, true, false>(c, a, s);
            case 32: return kda ? launch_dec_t<DK, LA_QDQ_INT8_GROUP, 32, true, true>(c, a, s)
                                : launch_dec_t<DK, LA_QDQ_INT8_GROUP, 32, true, false>(c, a, s);
            default: return kda ? launch_dec_t<DK, LA_QDQ_INT8_GROUP, 64, true, true>(c, a, s)
                                : launch_dec_t<DK, LA_QDQ_INT8_GROUP, 64, true, false>(c, a, s);
        }
    }
    switch (c.group) {
        case 16: return kda ? launch_dec_t<DK, LA_QDQ_INT8_GROUP, 16, false, true>(c, a, s)
                            : launch_dec_t<DK, LA_QDQ_INT8_GROUP, 16, false, false>(c, a, s);
        case 32: return kda ? launch_dec_t<DK, LA_QDQ_INT8_GROUP, 32, false, true>(c, a, s)
                            : launch_dec_t<DK, LA_QDQ_INT8_GROUP, 32, false, false>(c, a, s);
        default: return kda ? launch_dec_t<DK, LA_QDQ_INT8_GROUP, 64, false, true>(c, a, s)
                            : launch_dec_t<DK, LA_QDQ_INT8_GROUP, 64, false, false>(c, a, s);
    }
}

hipError_t launch_decode(const la_config& c, const DecodeArgs& a, hipStream_t s) {
    switch (c.d_k) {
        case 16: return launch_dec_dk<16>(c, a, s);
        case 32: return launch_dec_dk<32>(c, a, s);
        case 64: return launch_dec_dk<64>(c, a, s);
        default: return launch_dec_dk<128>(c, a, s);
    }
}

}  // namespace la
