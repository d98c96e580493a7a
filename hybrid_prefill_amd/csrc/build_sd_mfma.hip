// Segment-record build on MFMA for the scalar (RetNet / Mamba2-style) and
// diagonal (GLA-style) families, d_k = d_v = 128, bf16 k/v, fp32 records.
//
// What it computes (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4: RetNet, Mamba2 and GLA need the transition operator; podcast
// companion page, "Family comparison: scalar -> diagonal -> dense"): with no
// delta term the record is a decayed sum of outer products,
//     scalar    ell = sum_t log alpha_t,   S = sum_t beta_t e^{ell - L_t} k_t v_t^T
//     diagonal  ell_i = sum_t log alpha_{t,i},
//               S[i][:] = sum_t beta_t e^{ell_i - L_{t,i}} k_t[i] v_t^T
// (L_t = inclusive cumulative log decay).  Per 64-token chunk with in-chunk
// cumulative g and chunk total G this is
//     S <- e^{G} S + K^T diag(beta e^{G-g}) V            (scalar)
//     S <- diag(e^{G}) S + (e^{G-g} . K)^T diag(beta) V  (diagonal, per key channel)
// i.e. one 128 x 128 x 64 contraction per chunk.  The arithmetic intensity is
// 64 FLOP/B (scalar) and 32 FLOP/B (diagonal), so the build is bound by HBM;
// the contraction runs on bf16 MFMA so that the VALU is free for the scale
// factors.
//
// Work split: one 256-thread workgroup per (segment, head); wave w keeps rows
// [32w, 32w+32) of S, all 128 columns, as four fp32 32x32 accumulator tiles.
// The contraction runs over tokens, but k and v arrive token-major, so both
// are turned around on the MFMA itself: X . I (identity) returns X's columns in
// the accumulator layout, which is the A layout of K^T and the B layout of
// V^T with the same token order.  Wave w turns around its own 32 key channels
// (A operands it keeps) and 32 value channels (B operands, shared with the
// other waves through LDS).  The next chunk's k, v (and gates) are loaded into
// registers while the current chunk is reduced.
#include "hypic_internal.h"

namespace hypic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int CH = 64;
constexpr int D = 128;
constexpr int NT = 256;
constexpr int KML = 136;   // row length (bf16) of the token-major k / v tiles
constexpr int GL = 132;    // row length (fp32) of the token-major gate tile (diagonal)

template <int FAM, int NJB>
struct __align__(16) SdSmem {
    u16 Km[CH * KML];
    u16 Vm[CH * (32 * NJB + 8)];            // this workgroup's value columns, token-major
    uint32_t vx[NJB * 4 * 64 * 4];          // V^T B fragments: [j block][k-step][lane] x 16 B
    float gate[FAM == HYPIC_DIAGONAL ? CH * GL : 1];
    float la[CH], beta[CH], wsc[CH];        // per-token log decay, write gate, scalar-family scale
    float gd[D];                            // diagonal: per-channel chunk decay G_i
    float eG;
    int64_t t0, n;
    int32_t slot, state;
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const __bf16 x = (__bf16)a, y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(u16, x) | ((uint32_t)__builtin_bit_cast(u16, y) << 16);
}
__device__ __forceinline__ u32x4 pack8u(const f32x16 &c, int half) {
    const int o = 8 * half;
    return u32x4{pack2(c[o], c[o + 1]), pack2(c[o + 2], c[o + 3]), pack2(c[o + 4], c[o + 5]),
                 pack2(c[o + 6], c[o + 7])};
}
__device__ __forceinline__ bf16x8 lds8(const u16 *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// NSPLIT workgroups share one (segment, head): workgroup q keeps the value
// columns [128 q / NSPLIT, 128 (q+1) / NSPLIT).  They all read the keys (and
// gates); block ids are laid out so the NSPLIT workgroups of a unit land on the
// same XCD (consecutive block ids go to consecutive XCDs), where the repeated
// key reads hit that XCD's L2 instead of HBM.
template <int FAM, int NSPLIT>
__global__ __launch_bounds__(NT, FAM == HYPIC_DIAGONAL ? 1 : 2) void sd_build_mfma_kernel(BuildArgs a) {
    constexpr int NJB = 4 / NSPLIT;          // 32-column value blocks per workgroup
    constexpr int VML = 32 * NJB + 8;
    __shared__ SdSmem<FAM, NJB> sm;
    constexpr bool DIAG = FAM == HYPIC_DIAGONAL;

    const int th = threadIdx.x;
    const int w = th >> 6, l = th & 63, h = l >> 5, l32 = l & 31;
    const int b = blockIdx.x;
    const int q = (b >> 3) % NSPLIT;
    const int unit = (b / (8 * NSPLIT)) * 8 + (b & 7);
    const int head = unit % a.H;
    const int seg = unit / a.H;
    const int jc0 = 32 * NJB * q;            // first value column of this workgroup
    if (seg >= a.num_segments) return;       // grid padding

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
    __syncthreads();
    const int state = sm.state;
    if (state == 1) return;
    const int64_t t0 = sm.t0;
    const int64_t n = state == 2 ? 0 : sm.n;
    const int64_t slot = sm.slot;

    f32x16 st[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[jb][r] = 0.f;
    double ell = 0.0;   // scalar: thread 0; diagonal: lanes of half 0 keep channel 32w + l32

    // identity B fragments: B[k][n] = 1 if 16 ks + 8h + e == n
    bf16x8 eye[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) eye[ks][e] = (__bf16)((16 * ks + 8 * h + e == l32) ? 1.0f : 0.0f);

    const u16 *kp = static_cast<const u16 *>(a.k);
    const u16 *vp = static_cast<const u16 *>(a.v);
    // per thread: 16-byte pieces p = th + 256 u (u < 4) of the 64 x 128 chunk: row p/16, channels 8 (p%16)
    uint4 kr[4], vr[NJB];
    float4 gr[8];
    float br = 0.f, lr = 0.f;

#define HYPIC_SD_FETCH(BASE)                                                                           \
    do {                                                                                               \
        const int64_t rem_ = n - (BASE);                                                               \
        const int cl_ = rem_ < CH ? (int)rem_ : CH;                                                    \
        _Pragma("unroll") for (int u = 0; u < 4; ++u) {                                                \
            const int p = th + NT * u, t = p >> 4, c8 = 8 * (p & 15);                                  \
            kr[u] = t < cl_ ? *reinterpret_cast<const uint4 *>(kp + (t0 + (BASE) + t) * a.k_st +       \
                                                                head * a.k_sh + c8)                    \
                            : make_uint4(0, 0, 0, 0);                                                  \
        }                                                                                              \
        _Pragma("unroll") for (int u = 0; u < NJB; ++u) {                                              \
            const int p = th + NT * u, t = p / (4 * NJB), c8 = 8 * (p % (4 * NJB));                    \
            vr[u] = t < cl_ ? *reinterpret_cast<const uint4 *>(vp + (t0 + (BASE) + t) * a.v_st +       \
                                                                head * a.v_sh + jc0 + c8)              \
                            : make_uint4(0, 0, 0, 0);                                                  \
        }                                                                                              \
        if (DIAG) {                                                                                    \
            _Pragma("unroll") for (int u = 0; u < 8; ++u) {                                            \
                const int p = th + NT * u, t = p >> 5, c4 = 4 * (p & 31);                              \
                gr[u] = (t < cl_ && a.log_alpha)                                                       \
                            ? *reinterpret_cast<const float4 *>(                                      \
                                  a.log_alpha + (t0 + (BASE) + t) * a.la_st + head * a.la_sh + c4)     \
                            : make_float4(0.f, 0.f, 0.f, 0.f);                                         \
            }                                                                                          \
        }                                                                                              \
        if (th < CH) {                                                                                 \
            const int64_t tt = t0 + (BASE) + th;                                                       \
            br = th < cl_ ? (a.beta ? a.beta[tt * a.b_st + head * a.b_sh] : 1.0f) : 0.0f;              \
            lr = (!DIAG && th < cl_ && a.log_alpha) ? a.log_alpha[tt * a.la_st + head * a.la_sh] : 0.f; \
        }                                                                                              \
    } while (0)

    if (n > 0) HYPIC_SD_FETCH(0);

    for (int64_t base = 0; base < n; base += CH) {
        // ---- stage the chunk (token-major) and the per-token gates
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = th + NT * u, t = p >> 4, c8 = 8 * (p & 15);
            *reinterpret_cast<uint4 *>(&sm.Km[t * KML + c8]) = kr[u];
        }
#pragma unroll
        for (int u = 0; u < NJB; ++u) {
            const int p = th + NT * u, t = p / (4 * NJB), c8 = 8 * (p % (4 * NJB));
            *reinterpret_cast<uint4 *>(&sm.Vm[t * VML + c8]) = vr[u];
        }
        if (DIAG) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int p = th + NT * u, t = p >> 5, c4 = 4 * (p & 31);
                *reinterpret_cast<float4 *>(&sm.gate[t * GL + c4]) = gr[u];
            }
        }
        if (th < CH) { sm.beta[th] = br; sm.la[th] = lr; }
        if (base + CH < n) HYPIC_SD_FETCH(base + CH);    // next chunk flies while this one is reduced
        __syncthreads();

        // ---- scale factors
        if (!DIAG) {
            if (w == 0) {
                float gv = sm.la[l];
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const float y = __shfl_up(gv, o);
                    if (l >= o) gv += y;
                }
                const float G = __shfl(gv, 63);
                sm.wsc[l] = sm.beta[l] * __expf(G - gv);
                double sd = (double)sm.la[l];
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) sd += __shfl_xor(sd, o);
                if (l == 0) { ell += sd; sm.eG = __expf(G); }
            }
        }
        // ---- turn this wave's 32 key channels and 32 value channels around: X . I
        f32x16 dk[2], dv[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) { dk[tb][r] = 0.f; dv[tb][r] = 0.f; }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                dk[tb] = mfma(lds8(&sm.Km[(32 * tb + l32) * KML + 32 * w + 16 * ks + 8 * h]), eye[ks], dk[tb]);
                if (w < NJB)
                    dv[tb] = mfma(lds8(&sm.Vm[(32 * tb + l32) * VML + 32 * w + 16 * ks + 8 * h]), eye[ks], dv[tb]);
            }
        }
        // ---- per-channel gates (diagonal): lane (l32, h) runs the cumulative sum of channel
        //      i = 32w + l32 and keeps e^{G_i - g_{t,i}} at the 32 token positions it holds
        float ksc[2][16];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) ksc[tb][r] = 0.f;
        if (DIAG) {
            const int i = 32 * w + l32;
            float run = 0.f;
            double dsum = 0.0;
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const float x = sm.gate[t * GL + i];
                run += x;
                dsum += (double)x;
                // token t sits in lane half (t >> 2) & 1, tile t >> 5, register index below
                const int rr = ((t & 31) >> 3) * 4 + (t & 3);
                if (((t >> 2) & 1) == h) ksc[t >> 5][rr] = run;
            }
            const float G = run;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int r = 0; r < 16; ++r) ksc[tb][r] = __expf(G - ksc[tb][r]);
            if (h == 0) { sm.gd[i] = G; ell += dsum; }
        }
        __syncthreads();   // wsc / eG / gd visible; the k, v tiles may be overwritten after the next barrier
        // ---- scale: scalar: beta e^{G-g} on the value side; diagonal: beta on values, e^{G-g} on keys
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = 32 * tb + acc_row(r, h);
                dv[tb][r] *= DIAG ? sm.beta[t] : sm.wsc[t];
                if (DIAG) dk[tb][r] *= ksc[tb][r];
            }
        // A operands (K^T, own rows) stay in registers; B operands (V^T, own 32 value channels) go to LDS
        bf16x8 ka[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            ka[ks] = __builtin_bit_cast(bf16x8, pack8u(dk[ks >> 1], ks & 1));
            if (w < NJB) *reinterpret_cast<u32x4 *>(&sm.vx[((w * 4 + ks) * 64 + l) * 4]) = pack8u(dv[ks >> 1], ks & 1);
        }
        // decay of the carried state
        if (DIAG) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float f = __expf(sm.gd[32 * w + acc_row(r, h)]);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) st[jb][r] *= f;
            }
        } else {
            const float f = sm.eG;
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int r = 0; r < 16; ++r) st[jb][r] *= f;
        }
        __syncthreads();
        // ---- S[own rows][own columns] += K^T V over the chunk's 64 tokens
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 vb =
                    __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&sm.vx[((jb * 4 + ks) * 64 + l) * 4]));
                st[jb] = mfma(ka[ks], vb, st[jb]);
            }
        __syncthreads();   // vx and the tiles are free for the next chunk
    }
#undef HYPIC_SD_FETCH

    // ---- record
    const float nanv = __int_as_float(0x7fc00000);
    const bool bad = state == 2;
    const int64_t rec = slot * a.H + head;
    float *dst = a.pool_S + rec * D * D;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dst[(int64_t)(32 * w + acc_row(r, h)) * D + jc0 + 32 * jb + l32] = bad ? nanv : st[jb][r];
    if (q != 0) return;
    if (DIAG) {
        if (h == 0) a.pool_ell[rec * D + 32 * w + l32] = bad ? nanv : (float)ell;
    } else if (th == 0) {
        a.pool_ell[rec] = bad ? nanv : (float)ell;
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_build_sd_mfma(const BuildArgs &a, hipStream_t stream, bool *taken) {
    *taken = false;
    if ((a.family != HYPIC_SCALAR && a.family != HYPIC_DIAGONAL) || a.kv_dtype != HYPIC_BF16 || a.dk != 128 ||
        a.dv != 128)
        return hipSuccess;
    if (!aligned16(a.k) || !aligned16(a.v) || (a.k_st % 8) || (a.k_sh % 8) || (a.v_st % 8) || (a.v_sh % 8))
        return hipSuccess;
    if (a.family == HYPIC_DIAGONAL && a.log_alpha &&
        (!aligned16(a.log_alpha) || (a.la_st % 4) || (a.la_sh % 4)))
        return hipSuccess;
    *taken = true;
    // split the value columns over more workgroups while the units alone leave CUs idle;
    // the grid is padded to a multiple of 8 units (padding blocks exit at once)
    const int64_t units = (int64_t)a.num_segments * a.H;
    // (the diagonal family re-reads its per-channel gates in every split and needs
    // one workgroup per CU for registers, so it is not split)
    const int nsplit = (a.family == HYPIC_DIAGONAL || units >= 1024) ? 1 : units >= 512 ? 2 : 4;
    const int64_t padded = (units + 7) / 8 * 8;
    const dim3 grid((unsigned)(padded * nsplit));
#define HYPIC_SD_LAUNCH(FAM_, NS_) hipLaunchKernelGGL((sd_build_mfma_kernel<FAM_, NS_>), grid, dim3(NT), 0, stream, a)
    if (a.family == HYPIC_SCALAR) {
        if (nsplit == 1) HYPIC_SD_LAUNCH(HYPIC_SCALAR, 1);
        else if (nsplit == 2) HYPIC_SD_LAUNCH(HYPIC_SCALAR, 2);
        else HYPIC_SD_LAUNCH(HYPIC_SCALAR, 4);
    } else {
        if (nsplit == 1) HYPIC_SD_LAUNCH(HYPIC_DIAGONAL, 1);
        else if (nsplit == 2) HYPIC_SD_LAUNCH(HYPIC_DIAGONAL, 2);
        else HYPIC_SD_LAUNCH(HYPIC_DIAGONAL, 4);
    }
#undef HYPIC_SD_LAUNCH
    return hipGetLastError();
}

}  // namespace hypic
