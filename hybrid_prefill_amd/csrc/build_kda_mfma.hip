// Chunked segment-record build for the KDA family at d_k = d_v = 128 on the fp32
// matrix cores (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4, lists KDA among the families whose reuse needs the transition
// operator):
//     A_t = (I - beta_t k_t k_t^T) diag(alpha_t),   X_t = A_t X_{t-1} + beta_t k_t [0 | v_t^T],
// on X = [T | S] (d_k rows, d_k + d_v columns, X_0 = [I | 0]); the record is
// (ell = 0, P = T_C, S).
//
// Chunk form (32 tokens, g_t = the chunk's cumulative log alpha up to and
// including token t, per key channel).  Writing each token's correction as
// e_t = beta_t (v_t - k_t^T diag(alpha_t) X_{t-1}) (a row, zero v in the T
// columns), unrolling the recurrence over the chunk gives
//     X_t = diag(e^{g_t}) X_0 + sum_{s<=t} diag(e^{g_t - g_s}) k_s e_s,
//     (I + diag(beta) A) E = diag(beta) (V - K_g X_0),
//     A_ts = sum_i k_t[i] k_s[i] e^{g_t[i] - g_s[i]}  (s < t),  K_g row t = k_t e^{g_t},
// so with T = (I + diag(beta) A)^{-1} (unit lower triangular),
// M = T diag(beta) K_g and U = T diag(beta) V, which do not depend on the state:
//     E = U - M X_0,     X_C = diag(e^{g_C}) X_0 + Khat^T E,   Khat row s = k_s e^{g_C - g_s}.
// The Gram A is formed in three 16 x 16 blocks, each as a product of two
// per-token scaled key tiles whose exponents are split at a reference token:
// the off-diagonal block at the boundary between the halves (both factors
// <= 1), a diagonal block at its eighth token (factors up to the decay over
// seven tokens).  A chunk whose factors would exceed 2^100 (a channel decaying
// by more than e^-69 within seven tokens) is instead applied token by token to
// the state, from the same staged keys, gates and values.
//
// Workgroup (segment, head, q): q = 0 keeps the T columns, q = 1 the S columns.
// Eight waves in two roles, one chunk apart, with two workgroup barriers per chunk:
//   state waves 0-3 keep 32 columns each as four 32 x 32 fp32 accumulator tiles;
//     phase A: W = K_g X_0 - V;
//              wave 0 then inverts T for this chunk (the Gram came a phase earlier);
//     phase B: E = -T diag(beta) W and X_C = diag(e^{g_C}) X_0 + Khat^T E;
//   prep waves 4-7 work on the next chunk;
//     phase A: staging (thread per key channel and token half: prefix of the
//              gates, range vote, scaled key tiles into the next LDS buffer);
//     phase B: Gram blocks (waves 4-6, 16x16x4 fp32 MFMA), then the v tile.
// The tiles the state side reads in both phases (K_g, Khat^T, e^{g_C}, beta,
// -T diag(beta)) are double-buffered by chunk parity; the Gram inputs and the v
// tile (read in phase A, written in phase B) are single.  A chunk voted out of
// range is applied token by token by the state waves, reading its raw keys and
// gates from memory (its tiles are computed but unused).  The two roles run
// loops of their own with the same barriers, so neither role's registers count
// against the other's (two waves per SIMD leave 256 each).
#include "hypic_internal.h"

namespace hypic {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 512;                 // waves 0-3 state, 4-7 prep
constexpr int CK = 32;                  // tokens per chunk
constexpr int D = 128;
constexpr int LP = 132;                 // row stride of the [CK][D] tiles (floats)
constexpr int TP = 36;                  // row stride of the [D][CK] and [CK][CK] tiles
constexpr float LOG2E = 1.4426950408889634f;
constexpr float EXP_LIMIT = 100.0f;     // largest base-2 exponent a scaled key may carry

struct KdaMfmaSmem {
    float kg[2][CK][LP];   // k_t e^{g_t}
    float kht[2][D][TP];   // Khat^T
    float tn[2][CK][TP];   // -T diag(beta) (upper right block zero)
    float gam[2][D];       // e^{g_C}
    float b[2][CK];
    float qd[CK][LP];      // diagonal blocks, query side
    float kd[CK][LP];      // diagonal blocks, key side
    float x1[CK][LP];      // off-diagonal block: key side (rows 0..15), query side (rows 16..31)
    float v[CK][LP];       // v of this workgroup's columns (written in phase B for the next chunk)
    float nm[CK][TP];      // beta_t A_ts for s < t
    float tw[CK][TP];      // T, diagonal blocks (state wave 0)
    int32_t vote[2][4];    // per prep wave: a factor of the chunk is out of range
    int64_t t0, n;
    int32_t slot, state;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive elements of a row through a buffer resource (the row's base in
// scalar registers, the constant part of the offset in the instruction): the rare
// token-by-token path then holds no per-group address registers.
template <typename XT> __device__ __forceinline__ f32x4 bload4(__amdgpu_buffer_rsrc_t r, int off);
template <> __device__ __forceinline__ f32x4 bload4<float>(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return f32x4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]), __uint_as_float(v[3])};
}
template <> __device__ __forceinline__ f32x4 bload4<uint16_t>(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                 __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
}
template <typename XT> __device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, int off);
template <> __device__ __forceinline__ float bload1<float>(__amdgpu_buffer_rsrc_t r, int off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <> __device__ __forceinline__ float bload1<uint16_t>(__amdgpu_buffer_rsrc_t r, int off) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0) << 16);
}

template <typename XT>
__global__ __launch_bounds__(NT, 1) void kda_chunk_mfma_kernel(BuildArgs a) {
    __shared__ KdaMfmaSmem sm;
    const int th = threadIdx.x, lane = th & 63;
    // wave index as a scalar: the role branches below are then scalar branches, so a
    // wave runs only its own role's loop and barriers
    const int w = __builtin_amdgcn_readfirstlane(th >> 6);
    const bool prep_role = w >= 4;
    const int q = blockIdx.x & 1;
    const int head = (blockIdx.x >> 1) % a.H;
    const int seg = (blockIdx.x >> 1) / a.H;
    if (th == 0) {
        const int64_t o0 = a.seg_offsets[seg], o1 = a.seg_offsets[seg + 1];
        const int32_t slot = a.dst_slots[seg];
        int st = 0;
        if (slot < 0 || slot >= a.num_slots) st = 1;
        else if (o0 < 0 || o1 < o0 || o1 > a.num_tokens) st = 2;
        if (st == 1 && q == 0) raise_flag(a.err_flag, HYPIC_EFLAG_SLOT_OUT_OF_RANGE);
        if (st == 2 && q == 0) raise_flag(a.err_flag, HYPIC_EFLAG_BAD_OFFSETS);
        sm.t0 = o0; sm.n = o1 - o0; sm.slot = slot; sm.state = st;
    }
    // The upper right block of both -T diag(beta) buffers stays zero.
    for (int e = th; e < 2 * 16 * 16; e += NT) sm.tn[e >> 8][(e >> 4) & 15][16 + (e & 15)] = 0.0f;
    __syncthreads();
    const int state = sm.state;
    if (state == 1) return;
    const int64_t t0 = sm.t0;
    const int64_t n = state == 2 ? 0 : sm.n;
    const int64_t rec = (int64_t)sm.slot * a.H + head;
    const int nch = (int)((n + CK - 1) / CK);
    const XT *kp = static_cast<const XT *>(a.k);
    const XT *vp = static_cast<const XT *>(a.v);
    const bool isS = q == 1;
    const bool has_la = a.log_alpha != nullptr, has_b = a.beta != nullptr;
    // A missing log alpha or beta is read from the keys with stride 0 and replaced
    // at use (the loads take no branch: a branch joining around a load makes the
    // compiler wait for it there).
    const float *la_base = has_la ? a.log_alpha + head * a.la_sh : static_cast<const float *>(a.k);
    const int64_t la_st = has_la ? a.la_st : 0;
    const float *b_base = has_b ? a.beta + head * a.b_sh : static_cast<const float *>(a.k);
    const int64_t b_st = has_b ? a.b_st : 0;
    const XT *k_base = kp + head * a.k_sh;
    const XT *v_base = vp + head * a.v_sh;
    // token index of chunk c, position t, clamped into the segment (n > 0)
    auto tok_of = [&](int c, int t) -> int64_t {
        const int64_t p = (int64_t)c * CK + t;
        return t0 + (p < n ? p : n - 1);
    };

    // ---- state role: lane (ln, hh) of wave w keeps column colw, rows 32r + 8(i/4) + 4hh + i%4.
    const int ln = lane & 31, hh = lane >> 5;
    const int colw = 32 * (w & 3) + ln;
    f32x16 X[4], Wt;
    f32x4 na10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            X[r][i] = (!isS && 32 * r + 8 * (i >> 2) + 4 * hh + (i & 3) == colw) ? 1.0f : 0.0f;

    // ---- prep role: key channel ch, tokens 16hf .. 16hf+15 of a chunk; the two halves
    // of a channel sit in lanes l and l + 32 of one wave.
    const int pt = th & 255, ch = 32 * (pt >> 6) + (pt & 31), hf = (pt >> 5) & 1;
    float rla[16], rk[16], rv[16], sv[16], rb;
    // The chunk's rows through buffer resources: the chunk's base in scalar registers,
    // one lane offset, and bounds that end at the segment's last row (rows past it
    // read as zero and are masked at use), so no per-lane 64-bit address arithmetic.
    auto fetch = [&](int c) {
        const int64_t row0 = t0 + (int64_t)c * CK, rem = n - (int64_t)c * CK;
        const int rows = rem > 0 ? (rem < CK ? (int)rem : CK) : 0;
        const __amdgpu_buffer_rsrc_t rl_ = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(la_base + row0 * la_st), (short)0,
            has_la && rows > 0 ? (int)(((int64_t)(rows - 1) * la_st + D) * 4) : 0, RSRC_WORD3);
        const __amdgpu_buffer_rsrc_t rk_ = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(k_base + row0 * a.k_st), (short)0,
            rows > 0 ? (int)(((int64_t)(rows - 1) * a.k_st + D) * (int)sizeof(XT)) : 0, RSRC_WORD3);
        const __amdgpu_buffer_rsrc_t rv_ = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(v_base + row0 * a.v_st), (short)0,
            rows > 0 ? (int)(((int64_t)(rows - 1) * a.v_st + D) * (int)sizeof(XT)) : 0, RSRC_WORD3);
        const int ol = (16 * hf * (int)la_st + ch) * 4;
        const int ok = (16 * hf * (int)a.k_st + ch) * (int)sizeof(XT);
        const int ov = (16 * hf * (int)a.v_st + ch) * (int)sizeof(XT);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            rla[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl_, ol + u * (int)la_st * 4, 0, 0));
            rk[u] = bload1<XT>(rk_, ok + u * (int)a.k_st * (int)sizeof(XT));
            rv[u] = bload1<XT>(rv_, ov + u * (int)a.v_st * (int)sizeof(XT));
        }
        rb = b_base[tok_of(c, pt & (CK - 1)) * b_st];
    };
    // Staging of chunk c into buffer c & 1 (and the Gram inputs), with the range vote.
    auto stage = [&](int c) {
        const int bf = c & 1;
        const int64_t rem = n - (int64_t)c * CK;
        const int cl = rem < CK ? (rem > 0 ? (int)rem : 0) : CK;
        // prefix over this half, then the halves' totals swapped across the wave
        float L[16];
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            acc += (16 * hf + u < cl && has_la ? rla[u] : 0.0f) * LOG2E;
            L[u] = acc;
        }
        const float other = __shfl_xor(acc, 32);
        const float off = hf ? other : 0.0f;    // the first half's total, for the second
        const float Gc = acc + other, Gh = hf ? other : acc, Gr = off + L[7];
        // Two exponentials per element: the query- and key-side factors of the
        // diagonal block, 2^{g-Gr} and 2^{Gr-g}, which the vote keeps inside
        // [2^-100, 2^100]; the other tiles are these times per-thread constants
        // (a constant that underflows only loses terms below 2^-26 |k|).
        const float cg = ex2(Gr), cc = ex2(Gc - Gr), ch_ = ex2(hf ? Gr - Gh : Gh - Gr);
        float emax = -INFINITY;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int t = 16 * hf + u;
            const float g = off + L[u];
            const float kk = t < cl ? rk[u] : 0.0f;
            const float ex = hf ? g - Gh : Gh - g;
            emax = fmaxf(emax, fmaxf(fmaxf(g, Gc - g), fmaxf(fmaxf(g - Gr, Gr - g), ex)));
            const float qv = kk * ex2(g - Gr), kv = kk * ex2(Gr - g);
            sm.kg[bf][t][ch] = qv * cg;                 // k 2^{g}
            sm.kht[bf][ch][t] = kv * cc;                // k 2^{Gc-g}
            sm.qd[t][ch] = qv;
            sm.kd[t][ch] = kv;
            sm.x1[t][ch] = (hf ? qv : kv) * ch_;        // k 2^{g-Gh} (second half), k 2^{Gh-g} (first)
            sv[u] = t < cl && isS ? rv[u] : 0.0f;   // into the v tile in phase B
        }
        if (hf == 0) sm.gam[bf][ch] = ex2(Gc);
        if (pt < CK) sm.b[bf][pt] = pt < cl ? (has_b ? rb : 1.0f) : 0.0f;
        const bool out = __ballot(!(emax <= EXP_LIMIT)) != 0;
        if (lane == 0) sm.vote[bf][w - 4] = out ? 1 : 0;
    };
    // Gram blocks of the staged chunk: wave 4 (0,0), wave 5 (1,1), wave 6 (1,0).
    auto gram = [&]() {
        const int pw = w - 4;
        if (pw < 3) {
            const float(*Qt)[LP] = pw == 2 ? sm.x1 : sm.qd;
            const float(*Kt)[LP] = pw == 2 ? sm.x1 : sm.kd;
            const int I = pw == 0 ? 0 : 1, J = pw == 1 ? 1 : 0;
            const int m = lane & 15, g = lane >> 4;
            f32x4 c0v = {0.f, 0.f, 0.f, 0.f}, c1v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 8; ++s) {       // contraction index 16s + 4g + j
                const f32x4 qa = *reinterpret_cast<const f32x4 *>(&Qt[16 * I + m][16 * s + 4 * g]);
                const f32x4 kb = *reinterpret_cast<const f32x4 *>(&Kt[16 * J + m][16 * s + 4 * g]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (s & 1) c1v = mfma16(qa[j], kb[j], c1v);
                    else c0v = mfma16(qa[j], kb[j], c0v);
                }
            }
            return c0v + c1v;                   // rows 16I + 4g + j, column 16J + m
        }
        return f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto gram_store = [&](int c, f32x4 Ab) {
        const int pw = w - 4;
        if (pw < 3) {
            const int I = pw == 0 ? 0 : 1, J = pw == 1 ? 1 : 0;
            const int m = lane & 15, g = lane >> 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * I + 4 * g + j, s = 16 * J + m;
                sm.nm[t][s] = t > s ? sm.b[c & 1][t] * Ab[j] : 0.0f;
            }
        }
    };

    auto store_v = [&]() {
#pragma unroll
        for (int u = 0; u < 16; ++u) sm.v[16 * hf + u][ch] = sv[u];
    };

    // Prologue: chunk 0 staged and its Gram formed; chunk 1's inputs in flight.
    if (nch > 0) {
        if (prep_role) {
            fetch(0);
            stage(0);
            fetch(1);
        }
    }
    __syncthreads();
    if (nch > 0 && prep_role) {
        gram_store(0, gram());
        store_v();
    }
    __syncthreads();

    // Two loops, one per role, with the same two workgroup barriers per chunk.
    if (prep_role) {
        for (int c = 0; c < nch; ++c) {
            stage(c + 1);                   // phase A
            fetch(c + 2);
            __syncthreads();
            gram_store(c + 1, gram());      // phase B
            store_v();
            __syncthreads();
        }
        return;
    }
    for (int c = 0; c < nch; ++c) {
        const int bf = c & 1;
        const int64_t rem = n - (int64_t)c * CK;
        const int cl = rem < CK ? (int)rem : CK;
        const bool serial = (sm.vote[bf][0] | sm.vote[bf][1] | sm.vote[bf][2] | sm.vote[bf][3]) != 0;
        // ---------------- phase A
        if (!serial) {
            // W = K_g X_0 - V on the wave's columns (contraction over state rows)
            f32x16 W0, W1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = 8 * (i >> 2) + 4 * hh + (i & 3);
                W0[i] = isS && t < cl ? -sm.v[t][colw] : 0.0f;
                W1[i] = 0.0f;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f32x4 kv = *reinterpret_cast<const f32x4 *>(&sm.kg[bf][ln][32 * r + 8 * s + 4 * hh]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (r & 1) W1 = mfma32(kv[j], X[r][4 * s + j], W1);
                        else W0 = mfma32(kv[j], X[r][4 * s + j], W0);
                    }
                }
            Wt = W0 + W1;
            if (w == 0) {
                // T = (I + N)^{-1}: the two diagonal 16 x 16 blocks by forward
                // substitution (lane per column; the upper half of the wave repeats
                // the lower), T_10 = -T_11 (N_10 T_00) on the 16x16x4 MFMA.
                const int cc = lane & 15, blk = (lane >> 4) & 1, o = 16 * blk;
                float tc[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) tc[i] = i == cc ? 1.0f : 0.0f;
#pragma unroll
                for (int i = 1; i < 16; ++i) {
                    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
                    for (int m4 = 0; m4 < i; m4 += 4) {
                        const f32x4 nv = *reinterpret_cast<const f32x4 *>(&sm.nm[o + i][o + m4]);
                        if (m4 + 0 < i) s0 += nv[0] * tc[m4 + 0];
                        if (m4 + 1 < i) s1 += nv[1] * tc[m4 + 1];
                        if (m4 + 2 < i) s0 += nv[2] * tc[m4 + 2];
                        if (m4 + 3 < i) s1 += nv[3] * tc[m4 + 3];
                    }
                    if (i > cc) tc[i] = -(s0 + s1);
                }
                const float bc = sm.b[bf][o + cc];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    sm.tw[o + i][o + cc] = tc[i];
                    sm.tn[bf][o + i][o + cc] = -tc[i] * bc;
                }
            }
            // N_10 for the merge in phase B (the prep waves rewrite nm meanwhile)
            na10 = *reinterpret_cast<const f32x4 *>(&sm.nm[16 + (lane & 15)][4 * (lane >> 4)]);
        } else {
            // Token by token, from memory: the lane pair (ln, 0), (ln, 1) holds the column.
            const int vk = 4 * hh * (int)sizeof(XT), vl = 16 * hh;
#pragma unroll 1
            for (int t = 0; t < cl; ++t) {
                const int64_t tok = t0 + (int64_t)c * CK + t;
                const __amdgpu_buffer_rsrc_t rk_ = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(k_base + tok * a.k_st), (short)0, D * (int)sizeof(XT), RSRC_WORD3);
                // a missing log alpha reads as zero (no records)
                const __amdgpu_buffer_rsrc_t rl_ = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(la_base + tok * la_st), (short)0, has_la ? D * 4 : 0, RSRC_WORD3);
                float u = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const f32x4 kk = bload4<XT>(rk_, vk + (32 * r + 8 * s) * (int)sizeof(XT));
                        const f32x4 lv = bload4<float>(rl_, vl + (32 * r + 8 * s) * 4);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            X[r][4 * s + j] *= ex2(lv[j] * LOG2E);
                            u += kk[j] * X[r][4 * s + j];
                        }
                        // one group's loads at a time (hoisting them all beside the
                        // state would overflow the register file)
                        __builtin_amdgcn_sched_barrier(0);
                    }
                u += __shfl_xor(u, 32);
                const float bt = has_b ? a.beta[tok * a.b_st + head * a.b_sh] : 1.0f;
                const float vt = sm.v[t][colw];
                const float cf = bt * (vt - u);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const f32x4 kk = bload4<XT>(rk_, vk + (32 * r + 8 * s) * (int)sizeof(XT));
#pragma unroll
                        for (int j = 0; j < 4; ++j) X[r][4 * s + j] += kk[j] * cf;
                        __builtin_amdgcn_sched_barrier(0);
                    }
            }
        }
        __syncthreads();
        // ---------------- phase B
        if (!serial) {
            {
                // T_10 = -T_11 (N_10 T_00), every wave on its own (identical values into
                // the shared tile, each wave reading back its own writes): Y = N_10 T_00,
                // then T_11 Y = -T_10 (contraction index 4g + j at step j).
                const int m = lane & 15, g = lane >> 4;
                f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) Y = mfma16(na10[j], sm.tw[4 * g + j][m], Y);
                const f32x4 ta = *reinterpret_cast<const f32x4 *>(&sm.tw[16 + m][16 + 4 * g]);
                f32x4 Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) Z = mfma16(ta[j], Y[j], Z);
                const float bm = sm.b[bf][m];
#pragma unroll
                for (int j = 0; j < 4; ++j) sm.tn[bf][16 + 4 * g + j][m] = Z[j] * bm;
            }
            f32x16 E;
#pragma unroll
            for (int i = 0; i < 16; ++i) E[i] = 0.0f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const f32x4 ta = *reinterpret_cast<const f32x4 *>(&sm.tn[bf][ln][8 * s + 4 * hh]);
#pragma unroll
                for (int j = 0; j < 4; ++j) E = mfma32(ta[j], Wt[4 * s + j], E);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f32x4 gg = *reinterpret_cast<const f32x4 *>(&sm.gam[bf][32 * r + 8 * s + 4 * hh]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) X[r][4 * s + j] *= gg[j];
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const f32x4 kh = *reinterpret_cast<const f32x4 *>(&sm.kht[bf][32 * r + ln][8 * s + 4 * hh]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) X[r] = mfma32(kh[j], E[4 * s + j], X[r]);
                }
            }
        }
        __syncthreads();
    }

    const float nanv = __int_as_float(0x7fc00000);
    const bool bad = state == 2;
    float *dst = (isS ? a.pool_S : a.pool_P) + rec * D * D + colw;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            dst[(int64_t)(32 * r + 8 * (i >> 2) + 4 * hh + (i & 3)) * D] = bad ? nanv : X[r][i];
    if (th == 0 && q == 0) a.pool_ell[rec] = bad ? nanv : 0.0f;
}

}  // namespace

hipError_t launch_build_kda_mfma(const BuildArgs &b, hipStream_t stream) {
    if (b.num_segments <= 0) return hipSuccess;
    if (b.dk != D || b.dv != D) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((int64_t)b.num_segments * b.H * 2));
    if (b.kv_dtype == HYPIC_BF16) hipLaunchKernelGGL(kda_chunk_mfma_kernel<uint16_t>, grid, dim3(NT), 0, stream, b);
    else hipLaunchKernelGGL(kda_chunk_mfma_kernel<float>, grid, dim3(NT), 0, stream, b);
    return hipGetLastError();
}

}  // namespace hypic
