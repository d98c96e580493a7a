// Composition of GDN pool records on MFMA (d_k = d_v = 128).
//
// What it computes (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4: reuse composes T_C2*S(C1)+S(C2); podcast companion page,
// "Composition law, step by step"): per (request, head), over the chain in
// prompt order,
//     S <- e^{ell_i} (P_i S) + S_i
// and, in a second launch when the composed operator is asked for,
//     P <- P_i P        (P starts at I),   ell = sum_i ell_i.
//
// The chain is bandwidth-bound: every step streams one record (P_i and S_i,
// 128 KB) from HBM and does 4.2 MFLOP on it.  Accuracy needs more than one
// bf16 product (1e-4 relative for fp32 records), so P_i S is computed as
// hi.hi + hi.lo + lo.hi of the bf16 split x = hi + lo of both operands, which
// keeps about 16 significant bits and runs on the bf16 MFMA pipe.
//
// Work split: one 256-thread workgroup (4 waves) per (request, head).  Wave w
// keeps columns [32w, 32w+32) of the state as four fp32 32x32 accumulator
// tiles (rows 0-127).  P_i is staged once per step through LDS as bf16 hi/lo
// fragments laid out in MFMA operand order (one 16-byte read per lane, no bank
// conflicts); the B operand comes from the state's accumulator registers.  The
// next record is prefetched while the current product runs: P into registers
// (coalesced 16-byte loads), S straight from HBM into LDS (global_load_lds),
// read back from LDS in accumulator order.
#include <type_traits>

#include "hypic_internal.h"

namespace hypic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr int D = 128;
constexpr int NT = 256;
constexpr int NFRAG = 4 * 8;          // (row block mb, k-step kb) fragments of P
// One fragment holds 64 lanes x 8 bf16 (4 dwords per lane).  Lane half h is
// placed 132 dwords after half 0 and fragments 264 dwords apart, so that the
// 8-byte staging writes of 16 consecutive threads (4 k-steps x 4 pieces) hit
// 16 distinct bank pairs, and the 16-byte operand reads stay conflict-free.
constexpr int FRAG_U32 = 264;
__device__ __forceinline__ int lane_slot(int li, int hh) { return 4 * li + 132 * hh; }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u16 bf_bits(float x) { return __builtin_bit_cast(u16, (__bf16)x); }
__device__ __forceinline__ float bf_val(u16 b) { return __uint_as_float((uint32_t)b << 16); }

// bf16 split x = hi + lo (both rounded to nearest even)
__device__ __forceinline__ void split(float x, u16 &hi, u16 &lo) {
    hi = bf_bits(x);
    lo = bf_bits(x - bf_val(hi));
}

// the same split for two values at once, packed bf16 pairs (element 0 in the low half):
// one v_cvt_pk_bf16_f32 per part and the hi part unpacked with a shift and a mask
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x0, x1}, bf16x2_t));
    const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x0 - h0, x1 - h1}, bf16x2_t));
}

// The chain's slots and their ell values, staged in LDS as a ring of CHAIN_LDS
// entries (entry of chain position c at (c - c_lo) mod CHAIN_LDS): the validation
// pass fills the first CHAIN_LDS, and at every step c with c - c_lo a positive
// multiple of CHAIN_LDS / 2 the workgroup refills positions
// [c + CHAIN_LDS / 2, c + CHAIN_LDS), whose ring entries held positions already
// consumed.  The product loop then reads a step's slot with an LDS read only: a
// vector-memory load there (or a generic-pointer load) would make the compiler's
// wait for its result drain every record prefetch in flight.
constexpr int CHAIN_LDS = 1024;
struct ChainStage {
    int32_t slot[CHAIN_LDS];
    float ell[CHAIN_LDS];
};
// with head tokens: per chain entry, (first head token << 4) | count (count <= MAXH)
constexpr int MAXH = 8;
struct HeadStage {
    int32_t info[CHAIN_LDS];
    float k[MAXH][D], v[MAXH][D];     // the current entry's head tokens (this head's channels)
    float beta[MAXH], la[MAXH];
};
struct NoHeadStage { int32_t info[1]; };     // (chains without head tokens)
__device__ __forceinline__ int32_t head_info(const HeadStage &hs, int64_t c_lo, int64_t c) {
    return ((const __attribute__((address_space(3))) int32_t *)hs.info)[(c - c_lo) & (CHAIN_LDS - 1)];
}
// 0 when the entry's head tokens are well formed, else 2 (bad offsets)
__device__ __forceinline__ int head_entry(const ComposeArgs &a, int64_t c, int32_t &info) {
    const int64_t h0 = a.head_offsets[c], h1 = a.head_offsets[c + 1];
    if (h0 < 0 || h1 < h0 || h1 > a.num_head_tokens || h1 - h0 > MAXH) { info = 0; return 2; }
    info = (int32_t)((h0 << 4) | (h1 - h0));
    return 0;
}
typedef const __attribute__((address_space(3))) int32_t lds_i32;
typedef const __attribute__((address_space(3))) float lds_f32;
__device__ __forceinline__ int32_t chain_slot(const ChainStage &cs, int64_t c_lo, int64_t c) {
    return ((lds_i32 *)cs.slot)[(c - c_lo) & (CHAIN_LDS - 1)];
}
__device__ __forceinline__ float chain_ell(const ChainStage &cs, int64_t c_lo, int64_t c) {
    return ((lds_f32 *)cs.ell)[(c - c_lo) & (CHAIN_LDS - 1)];
}
// called by every thread of the workgroup at step c (the condition is uniform); the
// entries it writes are first read CHAIN_LDS / 2 - 3 steps later, after many barriers
__device__ __forceinline__ void chain_refill(ChainStage &cs, const ComposeArgs &a, int64_t c_lo, int64_t c_hi,
                                             int64_t c, int head, int th, int nthreads, HeadStage *hs = nullptr) {
    const int64_t d = c - c_lo;
    if (d < CHAIN_LDS / 2 || (d & (CHAIN_LDS / 2 - 1)) != 0) return;
    const int64_t j1 = c + CHAIN_LDS < c_hi ? c + CHAIN_LDS : c_hi;
    for (int64_t j = c + CHAIN_LDS / 2 + th; j < j1; j += nthreads) {
        const int32_t s = a.chain_slots[j];          // validated in range by the first pass
        cs.slot[(j - c_lo) & (CHAIN_LDS - 1)] = s;
        cs.ell[(j - c_lo) & (CHAIN_LDS - 1)] = a.pool_ell[(int64_t)s * a.H + head];
        if (hs) {
            int32_t info;
            head_entry(a, j, info);                  // validated by the first pass
            hs->info[(j - c_lo) & (CHAIN_LDS - 1)] = info;
        }
    }
}

__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// B operand from accumulator registers 8*half .. 8*half+7, as hi and lo parts
__device__ __forceinline__ void acc_to_b2(const f32x16 &c, int half, bf16x8 &bh, bf16x8 &bl) {
    uint32_t uh[4], ul[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) split2(c[8 * half + 2 * q], c[8 * half + 2 * q + 1], uh[q], ul[q]);
    bh = __builtin_bit_cast(bf16x8, u32x4{uh[0], uh[1], uh[2], uh[3]});
    bl = __builtin_bit_cast(bf16x8, u32x4{ul[0], ul[1], ul[2], ul[3]});
}

// Fragment slot of P element (i, k): A operand of row block mb = i/32 and
// k-step kb, in the order that pairs with acc_to_b2 (k-step kb covers the
// 16 columns 16*kb .. 16*kb+15; lane half h takes columns 4h..4h+3 and
// 8+4h..8+4h+3 of them, as elements 0-3 and 4-7).
struct __align__(16) PStage {
    uint32_t hi[NFRAG * FRAG_U32];
    uint32_t lo[NFRAG * FRAG_U32];
};

template <bool MODE_P, bool HEADS>
__global__ __launch_bounds__(NT, 1) void compose_dense_mfma_kernel(ComposeArgs a) {
    static_assert(!(MODE_P && HEADS), "head tokens act on the state only");
    __shared__ PStage ps;
    __shared__ typename std::conditional<HEADS, HeadStage, NoHeadStage>::type hst[1];
    // S_c, row-major, loaded straight from HBM into LDS; a separate LDS object from the
    // P fragments, so the compiler sees that staging P does not overlap the S loads
    // in flight and does not wait for them
    __shared__ __align__(16) float s_stage[D * D];
    __shared__ ChainStage cs;
    __shared__ int sh_bad;
    __shared__ float sh_pmax[4];      // P mode: each wave's largest |entry| of the product

    const int th = threadIdx.x;
    const int w = th >> 6, l = th & 63, h = l >> 5, l32 = l & 31;
    const int head = blockIdx.x % a.H;
    const int r = blockIdx.x / a.H;
    const int64_t orec = (int64_t)r * a.H + head;
    const int col0 = 32 * w;
    float *out = MODE_P ? a.out_P + orec * D * D : a.out_S + orec * D * D;

    // ---- chain validation (same rules as the reference kernel)
    if (th == 0) {
        const int64_t lo = a.chain_offsets[r], hi = a.chain_offsets[r + 1];
        sh_bad = (lo < 0 || hi < lo || hi > a.num_chain_slots) ? 2 : 0;
    }
    __syncthreads();
    const int64_t c_lo = a.chain_offsets[r], c_hi = a.chain_offsets[r + 1];
    if (sh_bad == 0) {
        __syncthreads();
        for (int64_t c = c_lo + th; c < c_hi; c += NT) {
            const int32_t s = a.chain_slots[c];
            const bool ok = s >= 0 && s < a.num_slots;
            if (!ok) sh_bad = 1;
            int32_t info = 0;
            if constexpr (HEADS) {
                if (head_entry(a, c, info)) sh_bad = 2;
            }
            if (c - c_lo < CHAIN_LDS) {
                cs.slot[c - c_lo] = ok ? s : 0;
                cs.ell[c - c_lo] = ok ? a.pool_ell[(int64_t)s * a.H + head] : 0.f;
                if constexpr (HEADS) hst[0].info[c - c_lo] = info;
            }
        }
    }
    __syncthreads();
    const int bad = sh_bad;
    if (bad) {
        if (th == 0 && !MODE_P)
            raise_flag(a.err_flag, bad == 1 ? HYPIC_EFLAG_SLOT_OUT_OF_RANGE : HYPIC_EFLAG_BAD_OFFSETS);
        const float nanv = __int_as_float(0x7fc00000);
        for (int e = th; e < D * D; e += NT) out[e] = nanv;
        if (!MODE_P && a.out_ell && th == 0) a.out_ell[orec] = nanv;
        return;
    }

    // ---- initial state; the first record from a zero (S) or identity (P) start is taken as is
    f32x16 st[4];
    int64_t c = c_lo;
    // (with head tokens the first record meets the state its head tokens made)
    const bool first_direct = !HEADS && (MODE_P || a.init_S == nullptr);
    double ell = 0.0;
    int pexp = 0;                     // P mode: the product is 2^pexp times the state
    if (first_direct && c < c_hi) {
        const int64_t rec = (int64_t)a.chain_slots[c] * a.H + head;
        const float *src = MODE_P ? a.pool_P + rec * D * D : a.pool_S + rec * D * D;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) st[mb][q] = src[(32 * mb + acc_row(q, h)) * D + col0 + l32];
        ell += (double)a.pool_ell[rec];
        ++c;
    } else {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = 32 * mb + acc_row(q, h);
                st[mb][q] = MODE_P ? (row == col0 + l32 ? 1.0f : 0.0f)
                                   : (a.init_S ? a.init_S[orec * D * D + (int64_t)row * D + col0 + l32] : 0.0f);
            }
    }

    // ---- head tokens of chain entry c (HEADS): fetched into registers with S_c (thread
    //      th takes channel th of [k | v] of each token, threads 0..MAXH-1 also its beta
    //      and log alpha; every load unconditional, the token index clamped into the
    //      stream), written to LDS at the top of step c and applied to the state before
    //      the product: per token S <- alpha (S - beta k (k^T S)) + beta k v^T.
    float hreg[MAXH], hb = 0.f, hl = 0.f;
    int32_t hinfo = 0;
#define HYPIC_FETCH_H(CC)                                                                        \
    do {                                                                                         \
        if constexpr (HEADS) {                                                                   \
            hinfo = head_info(hst[0], c_lo, (CC));                                               \
            const int64_t t0_ = hinfo >> 4;                                                      \
            const int n_ = hinfo & 15;                                                           \
            _Pragma("unroll") for (int j = 0; j < MAXH; ++j) {                                   \
                int64_t t_ = t0_ + (j < n_ ? j : 0);                                             \
                t_ = t_ < a.num_head_tokens ? t_ : a.num_head_tokens - 1;                        \
                hreg[j] = th < D ? a.head_k[(t_ * a.H + head) * D + th]                          \
                                 : a.head_v[(t_ * a.H + head) * D + th - D];                     \
            }                                                                                    \
            int64_t tb_ = t0_ + (th < n_ ? th : 0);                                              \
            tb_ = tb_ < a.num_head_tokens ? tb_ : a.num_head_tokens - 1;                         \
            hb = a.head_beta[tb_ * a.H + head];                                                  \
            hl = a.head_la[tb_ * a.H + head];                                                    \
        }                                                                                        \
    } while (0)
#define HYPIC_STAGE_H()                                                                          \
    do {                                                                                         \
        if constexpr (HEADS) {                                                                   \
            _Pragma("unroll") for (int j = 0; j < MAXH; ++j) {                                   \
                if (th < D) hst[0].k[j][th] = hreg[j];                                           \
                else hst[0].v[j][th - D] = hreg[j];                                              \
            }                                                                                    \
            if (th < MAXH) { hst[0].beta[th] = hb; hst[0].la[th] = hl; }                         \
        }                                                                                        \
    } while (0)
#define HYPIC_APPLY_H()                                                                          \
    do {                                                                                         \
        if constexpr (HEADS) {                                                                   \
            const int n_ = hinfo & 15;                                                           \
            for (int j = 0; j < n_; ++j) {                                                       \
                float kr_[4][16];                                                                \
                _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                 \
                    _Pragma("unroll") for (int qq = 0; qq < 4; ++qq) {                           \
                        const float4 k4 = *reinterpret_cast<const float4 *>(                     \
                            &hst[0].k[j][32 * mb + 8 * qq + 4 * h]);                             \
                        kr_[mb][4 * qq] = k4.x; kr_[mb][4 * qq + 1] = k4.y;                      \
                        kr_[mb][4 * qq + 2] = k4.z; kr_[mb][4 * qq + 3] = k4.w;                  \
                    }                                                                            \
                float u_ = 0.f;                                                                  \
                _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                 \
                    _Pragma("unroll") for (int q = 0; q < 16; ++q) u_ += kr_[mb][q] * st[mb][q]; \
                u_ += __shfl_xor(u_, 32);                /* the other half's rows */             \
                const float be_ = hst[0].beta[j], la_ = hst[0].la[j];                            \
                const float al_ = expf(la_);                                                     \
                const float bu_ = be_ * u_, bv_ = be_ * hst[0].v[j][col0 + l32];                 \
                _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                 \
                    _Pragma("unroll") for (int q = 0; q < 16; ++q)                               \
                        st[mb][q] = al_ * (st[mb][q] - kr_[mb][q] * bu_) + kr_[mb][q] * bv_;     \
                ell += (double)la_;                                                              \
            }                                                                                    \
        }                                                                                        \
    } while (0)

    // ---- records in flight: P_{c+1} is fetched into registers (coalesced 16-byte
    //      pieces q = th + 256 u) once P_c has been split to bf16 hi/lo fragments in LDS
    //      at the top of step c.  S_c goes HBM -> LDS directly (wave w's instruction u
    //      moves pieces (16 w + u) * 64 + lane) and is waited for only at the combine of
    //      step c.  Per wave the loads issued after S_c are exactly the 16 of P_{c+1}
    //      (the last step refetches its own P, an L2 hit), so the combine waits for
    //      vmcnt <= 16.
    //      Without head tokens both are issued inside the products of step c, four
    //      instructions per k-step (S_c in the first four k-steps, P_{c+1} in the last
    //      four): with one wave per SIMD a batch of 16 back-to-back loads stalls the
    //      wave's instruction stream while the memory pipe drains, whereas between
    //      products the MFMAs already issued keep the matrix pipe busy meanwhile.  S_c
    //      goes through inline asm there: the compiler then neither sees a pending
    //      HBM -> LDS load (while one is, it turns every wait for a register load into
    //      vmcnt(0), and it waits with vmcnt(0) before any read of the S stage) nor
    //      counts it, and P_{c+1}, the last load issued, is exactly what its wait at the
    //      top of step c + 1 covers.  The explicit vmcnt(16) and the workgroup barrier
    //      (both with a memory clobber) order the combine's reads after the load.
    //      With head tokens S_c is issued at the end of step c - 1 (with the builtin),
    //      after the entry's tokens, and P_{c+1} right after the split.
    constexpr bool SPREAD = !MODE_P && !HEADS;
    float4 pa[16];
    float ea = 0.f;               // ell of the record in pa
#define HYPIC_FETCH_P(PF, EL, CC)                                                                \
    do {                                                                                         \
        const int64_t frec = (int64_t)chain_slot(cs, c_lo, (CC)) * a.H + head;                \
        EL = chain_ell(cs, c_lo, (CC));                                                 \
        const float4 *fsrc = reinterpret_cast<const float4 *>(a.pool_P + frec * D * D);          \
        _Pragma("unroll") for (int u = 0; u < 16; ++u) PF[u] = load_nt(fsrc + th + NT * u);     \
    } while (0)
#define HYPIC_FETCH_P_PART(PF, FSRC, U0)                                                         \
    _Pragma("unroll") for (int u = (U0); u < (U0) + 4; ++u) PF[u] = load_nt(FSRC + th + NT * u);
#define HYPIC_FETCH_S_PART(FSS, U0)                                                              \
    _Pragma("unroll") for (int u = (U0); u < (U0) + 4; ++u)                                      \
        lds_dma16(FSS + (16 * w + u) * 64 + l, &s_stage[(16 * w + u) * 256]);
#define HYPIC_FETCH_S(CC)                                                                        \
    do {                                                                                         \
        const int64_t frec = (int64_t)chain_slot(cs, c_lo, (CC)) * a.H + head;                \
        const float4 *fss = reinterpret_cast<const float4 *>(a.pool_S + frec * D * D);           \
        _Pragma("unroll") for (int u = 0; u < 16; ++u)                                           \
            __builtin_amdgcn_global_load_lds(fss + (16 * w + u) * 64 + l,                        \
                                             &s_stage[(16 * w + u) * 256], 16, 0, kLoadNT);         \
    } while (0)
    // one step: stage P_c from PF (then fetch P_{c+1} into PF), acc = P_c state,
    // state <- e^{ell_c} acc + S_c (S), or state <- acc (P)
#define HYPIC_STEP(PF, EL)                                                                       \
    do {                                                                                         \
        if constexpr (HEADS) chain_refill(cs, a, c_lo, c_hi, c, head, th, NT, &hst[0]);          \
        else chain_refill(cs, a, c_lo, c_hi, c, head, th, NT);                                   \
        _Pragma("unroll") for (int u = 0; u < 16; ++u) {                                         \
            const int q = th + NT * u;                                                           \
            const int i = q >> 5, k0 = 4 * (q & 31);                                             \
            const int mb = i >> 5, li = i & 31;                                                  \
            const int kb = k0 >> 4, c16 = k0 & 15;                                               \
            const int hh = (c16 >> 2) & 1, e0 = (c16 >> 3) * 4;                                  \
            uint32_t h01, l01, h23, l23;                                                         \
            split2(PF[u].x, PF[u].y, h01, l01);                                                  \
            split2(PF[u].z, PF[u].w, h23, l23);                                                  \
            const int slot = (mb * 8 + kb) * FRAG_U32 + lane_slot(li, hh) + (e0 >> 1);          \
            *reinterpret_cast<u32x2 *>(&ps.hi[slot]) = u32x2{h01, h23};                          \
            *reinterpret_cast<u32x2 *>(&ps.lo[slot]) = u32x2{l01, l23};                          \
        }                                                                                        \
        const float le = EL;                                                                     \
        const float4 *fsrc_n = nullptr, *fss_c = nullptr;                                       \
        if constexpr (SPREAD) {                                                                  \
            const int64_t cn_ = c + 1 < c_hi ? c + 1 : c;                                         \
            const int64_t frn_ = (int64_t)chain_slot(cs, c_lo, cn_) * a.H + head;                 \
            const int64_t frc_ = (int64_t)chain_slot(cs, c_lo, c) * a.H + head;                   \
            EL = chain_ell(cs, c_lo, cn_);                                                       \
            fsrc_n = reinterpret_cast<const float4 *>(a.pool_P + frn_ * D * D);                  \
            fss_c = reinterpret_cast<const float4 *>(a.pool_S + frc_ * D * D);                   \
        } else {                                                                                 \
            HYPIC_FETCH_P(PF, EL, c + 1 < c_hi ? c + 1 : c);                                     \
        }                                                                                        \
        HYPIC_STAGE_H();                                                                         \
        lds_barrier();                                   /* fragments (and head tokens) visible */ \
        HYPIC_APPLY_H();                                                                         \
        bf16x8 bh[8], bl[8];                                                                     \
        _Pragma("unroll") for (int kb = 0; kb < 8; ++kb) acc_to_b2(st[kb >> 1], kb & 1, bh[kb], bl[kb]); \
        f32x16 acc[4];                                                                           \
        _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                         \
            _Pragma("unroll") for (int q = 0; q < 16; ++q) acc[mb][q] = 0.f;                    \
        /* A fragments of k-step kb + 1 are read while the products of kb run */               \
        bf16x8 ah[2][4], al[2][4];                                                               \
        _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) {                                       \
            const int f = (mb * 8) * FRAG_U32 + lane_slot(l32, h);                               \
            ah[0][mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&ps.hi[f])); \
            al[0][mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&ps.lo[f])); \
        }                                                                                        \
        _Pragma("unroll") for (int kb = 0; kb < 8; ++kb) {                                       \
            const int cb = kb & 1, nb = cb ^ 1;                                                  \
            if constexpr (SPREAD) {                                                              \
                if (kb < 4) { HYPIC_FETCH_S_PART(fss_c, 4 * kb) }                                \
                else { HYPIC_FETCH_P_PART(PF, fsrc_n, 4 * (kb - 4)) }                            \
                __builtin_amdgcn_sched_barrier(0);    /* keep each group at its k-step */        \
            }                                                                                    \
            if (kb + 1 < 8) {                                                                    \
                _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) {                               \
                    const int f = (mb * 8 + kb + 1) * FRAG_U32 + lane_slot(l32, h);              \
                    ah[nb][mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&ps.hi[f])); \
                    al[nb][mb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&ps.lo[f])); \
                }                                                                                \
            }                                                                                    \
            _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma(ah[cb][mb], bh[kb], acc[mb]); \
            _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma(ah[cb][mb], bl[kb], acc[mb]); \
            _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) acc[mb] = mfma(al[cb][mb], bh[kb], acc[mb]); \
        }                                                                                        \
        if (MODE_P) {                                                                            \
            _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) st[mb] = acc[mb];                   \
            float m_ = 0.f;                                                                      \
            _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                     \
                _Pragma("unroll") for (int q = 0; q < 16; ++q) m_ = fmaxf(m_, fabsf(st[mb][q])); \
            _Pragma("unroll") for (int o_ = 32; o_ >= 1; o_ >>= 1) m_ = fmaxf(m_, __shfl_xor(m_, o_)); \
            if (l == 0) sh_pmax[w] = m_;                                                         \
        } else {                                                                                 \
            if constexpr (SPREAD) __builtin_amdgcn_sched_barrier(0); /* products issued first */ \
            asm volatile("s_waitcnt vmcnt(16)" ::: "memory");   /* this wave's S_c pieces */     \
            lds_barrier();                               /* everyone's S_c pieces */            \
            const float sc = expf(le);                                                           \
            _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                     \
                _Pragma("unroll") for (int q = 0; q < 16; ++q)                                   \
                    st[mb][q] = sc * acc[mb][q] + s_stage[(32 * mb + acc_row(q, h)) * D + col0 + l32]; \
        }                                                                                        \
        ell += (double)le;                                                                       \
        lds_barrier();       /* fragments and S_c read by all before they are replaced */       \
        /* P mode: the product of contracting records drifts toward the fp32 subnormals;  */ \
        /* below 2^-32 it is scaled back to [1, 2) by a power of two (exact), recorded in */ \
        /* pexp.  Every wave takes the same decision from the same four maxima, read      */ \
        /* before the next barrier and rewritten only after it.                           */ \
        if (MODE_P) {                                                                            \
            const float m_ = fmaxf(fmaxf(sh_pmax[0], sh_pmax[1]), fmaxf(sh_pmax[2], sh_pmax[3]));  \
            if (m_ < 0x1p-32f && m_ > 0.f) {                                                     \
                const int s_ = -ilogbf(m_);                                                      \
                _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                 \
                    _Pragma("unroll") for (int q = 0; q < 16; ++q) st[mb][q] = ldexpf(st[mb][q], s_); \
                pexp -= s_;                                                                      \
            }                                                                                    \
        }                                                                                        \
        /* head tokens before S, so that the compiler's wait for them at the top of the   */ \
        /* next step does not also wait for S (loads complete in issue order)             */ \
        HYPIC_FETCH_H(c + 1 < c_hi ? c + 1 : c);                                                 \
        if (!MODE_P && !SPREAD) HYPIC_FETCH_S(c + 1 < c_hi ? c + 1 : c);  /* last: an L2 hit */   \
    } while (0)
    if (c < c_hi) {
        HYPIC_FETCH_P(pa, ea, c);
        HYPIC_FETCH_H(c);
        if (!MODE_P && !SPREAD) HYPIC_FETCH_S(c);
        while (true) {
            HYPIC_STEP(pa, ea);
            if (++c >= c_hi) break;
        }
        // every load (with head tokens the last step's S refetch) lands before the workgroup ends
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
#undef HYPIC_STEP
#undef HYPIC_FETCH_P
#undef HYPIC_FETCH_S
#undef HYPIC_FETCH_S_PART
#undef HYPIC_FETCH_P_PART
#undef HYPIC_FETCH_H
#undef HYPIC_STAGE_H
#undef HYPIC_APPLY_H
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 16; ++q) out[(int64_t)(32 * mb + acc_row(q, h)) * D + col0 + l32] = st[mb][q];
    // P mode runs after the state launch: its ell carries the renormalisation, so that
    // (out_ell, out_P) stays a record of the chain, T = e^ell P
    if (a.out_ell && th == 0) a.out_ell[orec] = (float)(ell + (double)pexp * 0.69314718055994530942);
}

// Sliced variant for few chains (the chain is sequential, so one workgroup per
// (request, head) leaves most of the chip idle when there are few of them): the
// state's columns evolve independently (column j of S only meets column j of S_i),
// so workgroup (request, head, slice) keeps columns [32 slice, 32 slice + 32) and
// four of them share a chain.  Eight waves in two roles:
//  - compute waves 0..3: wave w keeps row block w of the slice (one fp32 32x32 tile
//    in accumulators), multiplies P_c by the slice's state and folds in S_c, then
//    publishes its tile's hi/lo B fragments for the next step;
//  - split waves 4..7: wave 4 + s fetches rows 32s .. 32s + 31 of each P_i two
//    steps ahead (coalesced 16-byte pieces, two register sets) and writes them, split
//    to bf16 hi/lo, as row block s's A fragments into the fragment area of the next
//    step (double-buffered by step parity), while the compute waves run the products.
// Each step has two workgroup barriers: the first finds P_c staged and the state
// published; the compute waves then read the state's fragments into registers, and
// the second frees the exchange area for the new state and lets the split waves
// stage P_{c+1} (the other buffer) beside the products.
constexpr int NSL = 4;
constexpr int NT_SL = 512;
struct __align__(16) XStage {
    u32x4 f[8][2][64];        // [k-step][hi, lo][lane]
};

struct __align__(16) PFrag2 {
    uint32_t hi[2][NFRAG * FRAG_U32];     // [step parity][fragment]
    uint32_t lo[2][NFRAG * FRAG_U32];
};

__global__ __launch_bounds__(NT_SL, 1) void compose_sliced_mfma_kernel(ComposeArgs a) {
    __shared__ XStage xs;
    __shared__ PFrag2 xp;
    __shared__ ChainStage cs;
    __shared__ int sh_bad;

    const int th = threadIdx.x;
    const int wid = th >> 6, l = th & 63, h = l >> 5, l32 = l & 31;
    const bool splitter = wid >= 4;
    const int w = wid & 3;                      // row block (of the state, or of P_i)
    // the slices of a chain sit 8 blocks apart, so they land on the same XCD (block b
    // goes to XCD b % 8) and share each P_i through its L2
    const int bx = blockIdx.x;
    const int sl = (bx >> 3) % NSL;
    const int unit = (bx / (8 * NSL)) * 8 + (bx & 7);
    if (unit >= a.num_requests * a.H) return;   // grid padding
    const int head = unit % a.H;
    const int r = unit / a.H;
    const int64_t orec = (int64_t)r * a.H + head;
    const int col = 32 * sl + l32;              // this lane's state column
    float *out = a.out_S + orec * D * D;

    // ---- chain validation (same rules as the reference kernel)
    if (th == 0) {
        const int64_t lo = a.chain_offsets[r], hi = a.chain_offsets[r + 1];
        sh_bad = (lo < 0 || hi < lo || hi > a.num_chain_slots) ? 2 : 0;
    }
    __syncthreads();
    const int64_t c_lo = a.chain_offsets[r], c_hi = a.chain_offsets[r + 1];
    if (sh_bad == 0) {
        __syncthreads();
        for (int64_t c = c_lo + th; c < c_hi; c += NT_SL) {
            const int32_t s = a.chain_slots[c];
            const bool ok = s >= 0 && s < a.num_slots;
            if (!ok) sh_bad = 1;
            if (c - c_lo < CHAIN_LDS) {
                cs.slot[c - c_lo] = ok ? s : 0;
                cs.ell[c - c_lo] = ok ? a.pool_ell[(int64_t)s * a.H + head] : 0.f;
            }
        }
    }
    __syncthreads();
    const int bad = sh_bad;
    if (bad) {
        if (th == 0 && sl == 0)
            raise_flag(a.err_flag, bad == 1 ? HYPIC_EFLAG_SLOT_OUT_OF_RANGE : HYPIC_EFLAG_BAD_OFFSETS);
        const float nanv = __int_as_float(0x7fc00000);
        for (int e = th; e < 32 * D; e += NT_SL) out[(e >> 5) * D + 32 * sl + (e & 31)] = nanv;
        if (a.out_ell && th == 0 && sl == 0) a.out_ell[orec] = nanv;
        return;
    }

    // ---- initial tile (compute waves: rows 32w + acc_row, column col)
    f32x16 st = {};
    int64_t c = c_lo;
    const bool first_direct = a.init_S == nullptr;
    double ell = 0.0;
    if (first_direct && c < c_hi) {
        if (!splitter) {
            const int64_t rec = (int64_t)a.chain_slots[c] * a.H + head;
            const float *src = a.pool_S + rec * D * D;
#pragma unroll
            for (int q = 0; q < 16; ++q) st[q] = src[(32 * w + acc_row(q, h)) * D + col];
            ell += (double)a.pool_ell[rec];
        }
        ++c;
    } else if (!splitter) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = 32 * w + acc_row(q, h);
            st[q] = a.init_S ? a.init_S[orec * D * D + (int64_t)row * D + col] : 0.0f;
        }
    }

    // compute waves: S_c's 16 tile positions of this lane, two steps ahead (two sets),
    // and the ell of the record each set holds.  Split waves: P_i's rows 32w .. 32w + 31
    // as 16-byte pieces (piece u of lane l: row 32w + 2u + l / 32, columns 4 (l % 32)
    // .. +3), two register sets.
    float sa[16], sb[16];
    float ea = 0.f, eb = 0.f;
    float4 pa[16], pb[16];
#define HYPIC_PROW(CC) \
    (a.pool_P + ((int64_t)chain_slot(cs, c_lo, (CC)) * a.H + head) * D * D + (int64_t)(32 * w + (l >> 5)) * D + 4 * l32)
#define HYPIC_PFETCH(PF, PROW)                                                                      \
    do {                                                                                            \
        const float *pr_ = (PROW);                                                                  \
        _Pragma("unroll") for (int u = 0; u < 16; ++u)                                              \
            PF[u] = *reinterpret_cast<const float4 *>(pr_ + 2 * u * D);                             \
    } while (0)
#define HYPIC_SFETCH(SV, CC)                                                                        \
    do {                                                                                            \
        const float *ss_ = a.pool_S + ((int64_t)chain_slot(cs, c_lo, (CC)) * a.H + head) * D * D + col; \
        _Pragma("unroll") for (int q = 0; q < 16; ++q) SV[q] = ss_[(32 * w + acc_row(q, h)) * D];  \
    } while (0)
    // split wave: row block w's A fragments of a record, split to bf16 hi/lo, into
    // fragment buffer BUF
#define HYPIC_PSTAGE(PF, BUF)                                                                       \
    do {                                                                                            \
        _Pragma("unroll") for (int u = 0; u < 16; ++u) {                                            \
            const int li_ = 2 * u + (l >> 5), c0_ = 4 * l32;                                        \
            const int kb_ = c0_ >> 4, c16_ = c0_ & 15;                                              \
            const int slot_ = (w * 8 + kb_) * FRAG_U32 + lane_slot(li_, (c16_ >> 2) & 1) + 2 * (c16_ >> 3); \
            uint32_t h01_, l01_, h23_, l23_;                                                        \
            split2(PF[u].x, PF[u].y, h01_, l01_);                                                   \
            split2(PF[u].z, PF[u].w, h23_, l23_);                                                   \
            *reinterpret_cast<u32x2 *>(&xp.hi[BUF][slot_]) = u32x2{h01_, h23_};                     \
            *reinterpret_cast<u32x2 *>(&xp.lo[BUF][slot_]) = u32x2{l01_, l23_};                     \
        }                                                                                           \
    } while (0)
    // compute wave: the tile's hi/lo B fragments (k-steps 2w, 2w + 1)
#define HYPIC_PUBLISH()                                                                             \
    do {                                                                                            \
        _Pragma("unroll") for (int half = 0; half < 2; ++half) {                                    \
            bf16x8 bh_, bl_;                                                                        \
            acc_to_b2(st, half, bh_, bl_);                                                          \
            xs.f[2 * w + half][0][l] = __builtin_bit_cast(u32x4, bh_);                              \
            xs.f[2 * w + half][1][l] = __builtin_bit_cast(u32x4, bl_);                              \
        }                                                                                           \
    } while (0)
    // compute wave, one step: state <- e^{ell_c} P_c state + S_c, then publish it
#define HYPIC_CSTEP(SV, EL, PAR)                                                                    \
    do {                                                                                            \
        chain_refill(cs, a, c_lo, c_hi, c, head, th, NT_SL);                                        \
        lds_barrier();                                                                              \
        u32x4 bh_[8], bl_[8];                                                                       \
        _Pragma("unroll") for (int kb = 0; kb < 8; ++kb) {                                          \
            bh_[kb] = xs.f[kb][0][l];                                                               \
            bl_[kb] = xs.f[kb][1][l];                                                               \
        }                                                                                           \
        const bool more_ = c + 2 < c_hi;                                                            \
        const float le_ = EL;                                                                       \
        EL = chain_ell(cs, c_lo, more_ ? c + 2 : c);                                                \
        lds_barrier();                                                                              \
        f32x16 acc_ = {}, acc1_ = {};                                                               \
        _Pragma("unroll") for (int kb = 0; kb < 8; ++kb) {                                          \
            const int f_ = (w * 8 + kb) * FRAG_U32 + lane_slot(l32, h);                             \
            const bf16x8 ah_ = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&xp.hi[PAR][f_])); \
            const bf16x8 al_ = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(&xp.lo[PAR][f_])); \
            const bf16x8 b0_ = __builtin_bit_cast(bf16x8, bh_[kb]);                                 \
            const bf16x8 b1_ = __builtin_bit_cast(bf16x8, bl_[kb]);                                 \
            acc_ = mfma(ah_, b0_, acc_);                                                            \
            acc1_ = mfma(ah_, b1_, acc1_);                                                          \
            acc1_ = mfma(al_, b0_, acc1_);                                                          \
        }                                                                                           \
        acc_ += acc1_;                                                                              \
        {                                                                                           \
            const float sc_ = expf(le_);                                                            \
            _Pragma("unroll") for (int q = 0; q < 16; ++q) st[q] = sc_ * acc_[q] + SV[q];           \
        }                                                                                           \
        HYPIC_SFETCH(SV, more_ ? c + 2 : c);                                                        \
        ell += (double)le_;                                                                         \
        HYPIC_PUBLISH();                                                                            \
    } while (0)
    // split wave, one step: stage P_{c+1} from PN into the other buffer (on the last
    // step PN holds a repeat of an earlier record: staged, never read), then refetch
    // PN with P_{c+3}
#define HYPIC_SSTEP(PN, PAR)                                                                        \
    do {                                                                                            \
        chain_refill(cs, a, c_lo, c_hi, c, head, th, NT_SL);                                        \
        lds_barrier();                                                                              \
        const float *pn_ = HYPIC_PROW(c + 3 < c_hi ? c + 3 : c);                                    \
        lds_barrier();                                                                              \
        HYPIC_PSTAGE(PN, (PAR) ^ 1);                                                                \
        HYPIC_PFETCH(PN, pn_);    /* unconditional (the last steps reload P_c): no phi copies */    \
    } while (0)

    if (!splitter) {
        HYPIC_PUBLISH();
        if (c < c_hi) {
            HYPIC_SFETCH(sa, c);
            ea = chain_ell(cs, c_lo, c);
        }
        if (c + 1 < c_hi) {
            HYPIC_SFETCH(sb, c + 1);
            eb = chain_ell(cs, c_lo, c + 1);
        }
        // even steps use sa and fragment buffer 0, odd steps sb and buffer 1
        while (c < c_hi) {
            HYPIC_CSTEP(sa, ea, 0);
            if (++c >= c_hi) break;
            HYPIC_CSTEP(sb, eb, 1);
            ++c;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) out[(int64_t)(32 * w + acc_row(q, h)) * D + col] = st[q];
        if (a.out_ell && th == 0 && sl == 0) a.out_ell[orec] = (float)ell;
    } else {
        // P_c staged into buffer 0, P_{c+1} in pb and P_{c+2} in pa (clamped to the
        // chain's last record where the chain is shorter)
        if (c < c_hi) {
            HYPIC_PFETCH(pa, HYPIC_PROW(c));
            HYPIC_PFETCH(pb, HYPIC_PROW(c + 1 < c_hi ? c + 1 : c));
            HYPIC_PSTAGE(pa, 0);
            HYPIC_PFETCH(pa, HYPIC_PROW(c + 2 < c_hi ? c + 2 : c));
        }
        // the same step count and barriers as the compute waves
        while (c < c_hi) {
            HYPIC_SSTEP(pb, 0);
            if (++c >= c_hi) break;
            HYPIC_SSTEP(pa, 1);
            ++c;
        }
    }
#undef HYPIC_CSTEP
#undef HYPIC_SSTEP
#undef HYPIC_PUBLISH
#undef HYPIC_PSTAGE
#undef HYPIC_PFETCH
#undef HYPIC_PROW
#undef HYPIC_SFETCH
}

}  // namespace

hipError_t launch_compose_mfma(const ComposeArgs &a, hipStream_t stream, bool *taken) {
    *taken = false;
    // (KDA records are (ell = 0, P = T_C): the same fold)
    if ((a.family != HYPIC_GDN && a.family != HYPIC_KDA) || a.dk != 128 || a.dv != 128) return hipSuccess;
    *taken = true;
    const int64_t units = (int64_t)a.num_requests * a.H;
    if (units <= 512) {
        // few chains: four workgroups per chain, one per 32-column slice of the state
        const dim3 grid((unsigned)((units + 7) / 8 * 8 * NSL));
        hipLaunchKernelGGL(compose_sliced_mfma_kernel, grid, dim3(NT_SL), 0, stream, a);
    } else {
        hipLaunchKernelGGL((compose_dense_mfma_kernel<false, false>), dim3((unsigned)units), dim3(NT), 0, stream, a);
    }
    // the composed operator: one workgroup per chain, so that the whole product can be
    // renormalised at once (it writes out_ell after the state launch)
    if (a.out_P)
        hipLaunchKernelGGL((compose_dense_mfma_kernel<true, false>), dim3((unsigned)units), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

// Chains with head tokens (GDN, d_k = d_v = 128, no composed operator): one workgroup
// per (request, head) whatever the count.
hipError_t launch_compose_heads_mfma(const ComposeArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)a.num_requests * a.H;
    hipLaunchKernelGGL((compose_dense_mfma_kernel<false, true>), dim3((unsigned)units), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace hypic
