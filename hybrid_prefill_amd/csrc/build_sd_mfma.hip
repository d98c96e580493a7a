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
// i.e. one 128 x 128 x 64 contraction per chunk.  The scalar family needs no
// per-chunk rescale at all: over a block of up to 2048 tokens with total G_b,
//     S <- e^{G_b} S + sum_t beta_t e^{G_b - L_t} k_t v_t^T
// (L_t cumulative from the block start), so the weights of a whole block are
// computed once, before its chunks, into an LDS table, and each chunk only
// reads them.  The arithmetic intensity is
// 64 FLOP/B (scalar) and 32 FLOP/B (diagonal, whose fp32 gates double the
// bytes), so the build is bound by HBM; the contraction runs on bf16 MFMA so
// that the VALU is free for the scale factors.
//
// Work split: NSPLIT workgroups per (segment, head) of four compute waves and
// four loading waves.  Scalar family: workgroup q keeps value columns
// [128 q / NSPLIT, 128 (q + 1) / NSPLIT) and compute wave w rows [32w, 32w + 32)
// of S.  Diagonal family (NSPLIT = 2): workgroup q keeps key channels (rows of S)
// [64 q, 64 q + 64), so it stages only its half of the keys and of the fp32
// gates, and compute wave w the 32 rows 64 q + 32 (w / 2) + 0..31 by value
// columns 64 (w % 2) + 0..63.  Every tile is an fp32 32x32 accumulator.  Keys
// and values arrive token-major; both families read the K^T and V^T operand
// fragments straight from the token-major tiles with gfx950's transposing LDS
// read (ds_read_b64_tr_b16) and put the weights on the K^T fragment (scalar:
// beta_t e^{G_b - L_t} per token; diagonal: beta_t e^{G_i - L_{t,i}} per token
// and key channel), so a chunk is four MFMAs per value block.  Operand reads are
// issued before the first product that uses them.
//
// Streaming: four more waves load: keys, values (and the diagonal family's gates
// and beta) go from HBM straight into LDS (global_load_lds), NBUF chunks deep, so
// the compute waves never stall on the load queue (a single wave cannot issue a
// chunk's loads as fast as the compute waves use it); one workgroup barrier per
// chunk.  For the diagonal family the loading waves also bring each chunk's gates
// and beta, in a ring of their own one chunk further ahead than the keys and values;
// four factor waves (a third role, diagonal family only: 768-thread workgroups)
// turn them into the per-(token, channel) factors and the chunk decay one chunk
// ahead of use (factor wave f the workgroup's key channels 16f .. 16f + 15, while
// the compute waves run the current chunk's products), into parity-buffered LDS
// tiles that all four compute waves then read.  Tail rows past the segment
// repeat its last row and are masked at use (beta and log alpha of those tokens
// read as 0).
#include "hypic_internal.h"

namespace hypic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int CH = 64;
constexpr int D = 128;
constexpr int NWC = 4;           // compute waves
constexpr int NLW = 4;           // loading waves (one wave alone cannot issue loads fast enough)
constexpr int NFW = 4;           // diagonal family: factor waves
constexpr int NT = 64 * (NWC + NLW);
constexpr int NT_DIAG = 64 * (NWC + NLW + NFW);

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 pack8(const f32x16 &c, int half) {
    const int o = 8 * half;
    return __builtin_convertvector((f32x8){c[o], c[o + 1], c[o + 2], c[o + 3], c[o + 4], c[o + 5], c[o + 6], c[o + 7]},
                                   bf16x8);
}
__device__ __forceinline__ bf16x8 lds8(const u16 *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ds_read_b64_tr_b16: in each 16-lane group, lane 4a + b gives the address of four
// consecutive b16 of row a of a row-major tile (columns 4b .. 4b + 3 of the group's 16);
// lane j receives column j of those four rows.  Two reads give the 8-element operand
// fragment of one lane: 8 consecutive rows of one column.
__device__ __forceinline__ bf16x8 tr_pair(const u16 *p0, const u16 *p1) {
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// b16 fragment times eight fp32 factors, repacked (rounded to nearest even)
__device__ __forceinline__ bf16x8 scale8(bf16x8 x, float4 f0, float4 f1) {
    const f32x8 v = __builtin_convertvector(x, f32x8);
    const f32x8 s = {v[0] * f0.x, v[1] * f0.y, v[2] * f0.z, v[3] * f0.w, v[4] * f1.x, v[5] * f1.y, v[6] * f1.z,
                     v[7] * f1.w};
    return __builtin_convertvector(s, bf16x8);
}

// global_load_lds through inline asm (lds_dma16 / lds_dma4): the kernel counts its
// own loads (every wave issues the same number per chunk, and loads complete in
// issue order).
__device__ __forceinline__ void gll16(const void *src, void *dst) { lds_dma16(src, dst); }
// an operand every split of the (segment, head) reads (scalar: the keys; diagonal: the
// values): cached, so that the workgroups after the first find it in the XCD's L2
__device__ __forceinline__ void gll16s(const void *src, void *dst) { lds_dma16_shared(src, dst); }
__device__ __forceinline__ void gll4(const void *src, void *dst) { lds_dma4(src, dst); }

// a lane's value from another lane by a DPP control (gfx9 encoding), in registers
template <int CTRL> __device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

#define HYPIC_DPP_ADD(X, CTRL, ROWMASK) \
    X += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(X), CTRL, ROWMASK, 0xf, true))
// inclusive prefix sum over the 64 lanes of a wave (DPP row shifts, then row broadcasts)
__device__ __forceinline__ float wave_prefix_sum(float x) {
    HYPIC_DPP_ADD(x, 0x111, 0xf);
    HYPIC_DPP_ADD(x, 0x112, 0xf);
    HYPIC_DPP_ADD(x, 0x114, 0xf);
    HYPIC_DPP_ADD(x, 0x118, 0xf);
    HYPIC_DPP_ADD(x, 0x142, 0xa);
    HYPIC_DPP_ADD(x, 0x143, 0xc);
    return x;
}
#undef HYPIC_DPP_ADD

// One staged chunk.  Row r of Km holds 16 granules of 8 channels; granule g sits in
// slot g ^ (r % 16).  Vm rows hold the workgroup's 32 NJB value columns (4 NJB
// granules); granule g sits in slot g ^ ((r >> SH) % (4 NJB)), SH = 2, 1, 0 for
// NJB = 1, 2, 4.  Either way the 16 rows one operand read touches hit distinct
// bank groups, and global_load_lds can fill whole rows.
// Diagonal family: Km holds the workgroup's 64 key channels (8 granules a row,
// granule g in slot g ^ ((r >> 1) % 8)), Vm all 128 value columns (as the
// scalar Km).
constexpr int DKC = 64;                  // diagonal: key channels per workgroup
template <bool DIAG, int NJB>
struct __align__(16) SdBuf {
    u16 Km[DIAG ? CH * DKC : CH * D];
    u16 Vm[DIAG ? CH * D : CH * 32 * NJB];
};
// Diagonal family only (the scalar family reads its gates once per table block): a
// chunk's gates and beta, in a ring of their own (loaded one chunk further ahead than
// the keys and values).  Loading wave lw's share of the gates is channels
// 16 lw .. 16 lw + 15 of the workgroup's 64 for all 64 tokens (the channels compute
// wave lw turns into factors), in global_load_lds order: instruction j, lane l holds
// token 16 j + l / 4, channels 16 lw + 4 (l % 4) .. + 3.  Every loading wave loads a
// copy of beta (so that all of them issue the same instructions and count their
// loads alike); the compute waves read the first.
struct __align__(16) GateBuf {
    float gate[CH * DKC];
    float beta[NLW][CH];
};
constexpr int NBG = 3;                   // gate ring depth
__device__ __forceinline__ int gate_idx(int t, int ci) {   // token t, workgroup key channel ci
    return ((((ci >> 4) << 2) + (t >> 4)) * 64 + 4 * (t & 15) + ((ci & 15) >> 2)) * 4 + (ci & 3);
}
// factor tiles: row = workgroup key channel (64 floats), 16-byte granule g at slot g ^ (row % 16)
__device__ __forceinline__ int fac_idx(int ci, int g) { return ci * CH + ((g ^ (ci & 15)) << 2); }

constexpr int TBT = 2048;                // tokens per scalar weight table

template <bool DIAG, int NJB, int NBUF>
struct __align__(16) SdSmem {
    SdBuf<DIAG, NJB> buf[NBUF];
    GateBuf gbuf[DIAG ? NBG : 0];
    // (every array read with 16-byte loads starts 16-byte aligned)
    __align__(16) float fac[DIAG ? 2 : 1][DIAG ? DKC * CH : 4];   // diagonal, by chunk parity: beta_t e^{G_i - L_{t,i}}
    __align__(16) float eg[DIAG ? 2 : 1][DIAG ? DKC : 4];         // diagonal, by chunk parity: e^{G_i} of the chunk
    __align__(16) float wt[DIAG ? 4 : TBT];   // scalar: beta_t e^{G_b - L_t} of the current table block
    float wtot[NWC];                     // scalar: per-wave sums while a table is built
    double ellw[4];                      // scalar: per-wave ell
    int64_t t0, n;
    int32_t slot, state;
};

__device__ __forceinline__ int kmo(int r, int g) { return r * D + ((g ^ (r & 15)) << 3); }
__device__ __forceinline__ int kmo_half(int r, int g) { return r * DKC + ((g ^ ((r >> 1) & 7)) << 3); }
template <int NJB>
__device__ __forceinline__ int vmo(int r, int g) {
    constexpr int SH = NJB == 1 ? 2 : NJB == 2 ? 1 : 0;
    return r * 32 * NJB + ((g ^ ((r >> SH) & (4 * NJB - 1))) << 3);
}

// s_waitcnt vmcnt(k LPW) for a wave-uniform k <= K (the count must be an immediate;
// the counter's limit of 63 makes the wait at most a little stricter)
template <int LPW, int K>
__device__ __forceinline__ void wait_chunks(int k) {
    if constexpr (K == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        if (k >= K) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K * LPW < 63 ? K * LPW : 63) : "memory");
        else wait_chunks<LPW, K - 1>(k);
    }
}

// s_waitcnt vmcnt(k) for a wave-uniform k (rounded down to an immediate <= K; a
// smaller count only waits longer)
template <int K>
__device__ __forceinline__ void vm_wait(int k) {
    static_assert(K <= 63, "vmcnt limit");
    if constexpr (K == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
        if (k >= K) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(K) : "memory");
        else vm_wait<K - 1>(k);
    }
}

template <int FAM, int NSPLIT>
__global__ __launch_bounds__(FAM == HYPIC_DIAGONAL ? NT_DIAG : NT, (FAM == HYPIC_SCALAR && NSPLIT == 4) ? 2 : 1)
void sd_build_mfma_kernel(BuildArgs a) {
    constexpr bool DIAG = FAM == HYPIC_DIAGONAL;
    constexpr int NJB = 4 / NSPLIT;                    // 32-column value blocks per workgroup
    static_assert(!DIAG || NSPLIT == 2, "the diagonal family splits the key channels in two");
    // chunks staged: as many as fit beside the other workgroup on the CU (value
    // split 4: two per CU) or alone
    constexpr int NBUF = NSPLIT == 4 || DIAG ? 3 : NSPLIT == 2 ? 6 : 4;
    constexpr int DIST = NBUF - 1;                     // prefetch distance in chunks
    // global_load_lds instructions of each loading wave per chunk: its share of the
    // keys, values, and for the diagonal family gates, plus one dword row (beta or a
    // dummy)
    constexpr int NKI = (DIAG ? 8 : 16) / NLW, NVI = (DIAG ? 16 : 4 * NJB) / NLW, NGI = DIAG ? 16 / NLW : 0;
    static_assert(8 % NLW == 0 && (4 * NJB) % NLW == 0 && 16 % NLW == 0, "load shares");
    constexpr int LPW = NKI + NVI;                     // keys and values (the diagonal gates are counted apart)
    constexpr int LPG = NGI + 1;                       // diagonal: gates and beta
    constexpr int TBC = TBT / CH;                      // chunks per scalar weight table
    // with two value blocks per workgroup the scalar compute waves read a chunk's
    // operands one chunk ahead (two register sets fit beside the state), so at the
    // top of chunk c the loading waves have waited for chunk c + 1
    constexpr int AHEAD = (!DIAG && NJB == 2) ? 1 : 0;
    __shared__ SdSmem<DIAG, NJB, NBUF> sm;

    const int th = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(th >> 6);
    const int l = th & 63, h = l >> 5, l32 = l & 31;
    const int b = blockIdx.x;
    const int q = (b >> 3) % NSPLIT;
    const int unit = (b / (8 * NSPLIT)) * 8 + (b & 7);
    const int head = unit % a.H;
    const int seg = unit / a.H;
    const int jc0 = DIAG ? 0 : 32 * NJB * q;  // first value column of this workgroup
    const int kc0 = DIAG ? DKC * q : 0;       // first key channel of this workgroup (diagonal)
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
    const int nc = (int)((n + CH - 1) / CH);   // 32 bits: a segment whose keys fit in memory has far fewer chunks

    const u16 *kh = static_cast<const u16 *>(a.k) + t0 * a.k_st + head * a.k_sh + kc0;
    const u16 *vh = static_cast<const u16 *>(a.v) + t0 * a.v_st + head * a.v_sh + jc0;
    const float *gh = a.log_alpha ? a.log_alpha + t0 * a.la_st + head * a.la_sh + kc0 : nullptr;
    const float *bh = a.beta ? a.beta + t0 * a.b_st + head * a.b_sh : nullptr;

    // Loading wave: chunk C's loads into buffer C % NBUF, LPW instructions in a fixed
    // order (so vmcnt can count chunks).  Full chunks use per-lane element offsets
    // fixed for the segment; the tail chunk clamps rows (finite values; masked at use).
    constexpr int GR = 4 * NJB, RPI = 64 / GR, VSH = NJB == 1 ? 2 : NJB == 2 ? 1 : 0;
    int64_t mst = a.k_st > a.v_st ? a.k_st : a.v_st;
    if (a.la_st > mst) mst = a.la_st;
    if (a.b_st > mst) mst = a.b_st;
    const bool small_st = (int64_t)CH * mst < (1LL << 30);
    // Row geometry of one global_load_lds (64 lanes x 16 bytes): keys KR rows of KG
    // granules (scalar: all 128 channels; diagonal: the workgroup's 64), values VR rows
    // of VG granules (scalar: the workgroup's columns; diagonal: all 128), gates
    // (diagonal) 4 rows of 64 floats.  kswz / vswz: the LDS slot of granule g of row r.
    constexpr int KR = DIAG ? 8 : 4, KG = DIAG ? 8 : 16, KW = DIAG ? DKC : D;
    constexpr int VR = DIAG ? 4 : RPI, VG = DIAG ? 16 : GR, VW = DIAG ? D : 32 * NJB;
    auto kswz = [](int r, int g) { return DIAG ? g ^ ((r >> 1) & 7) : g ^ (r & 15); };
    auto vswz = [](int r, int g) { return DIAG ? g ^ (r & 15) : g ^ ((r >> VSH) & (GR - 1)); };
    // the operand every split of a (segment, head) reads goes through the L2 (cached);
    // the split's own operand and the gates are streamed (non-temporal)
    constexpr bool SHARED_K = !DIAG && NSPLIT > 1, SHARED_V = DIAG;
    auto gll16k = [](const void *src, void *dst) { if constexpr (SHARED_K) gll16s(src, dst); else gll16(src, dst); };
    auto gll16v = [](const void *src, void *dst) { if constexpr (SHARED_V) gll16s(src, dst); else gll16(src, dst); };
    auto issue = [&](int C, int lw, const uint32_t *ko, const uint32_t *vo, const uint32_t *go) {
        const int bi = (int)(C % NBUF);
        const int64_t base = (int64_t)C * CH, rem = n - base;
        SdBuf<DIAG, NJB> &Bf = sm.buf[bi];
        if (rem >= CH && small_st) {
            const u16 *kc = kh + base * a.k_st, *vc = vh + base * a.v_st;
#pragma unroll
            for (int j = 0; j < NKI; ++j) gll16k(kc + ko[j], &Bf.Km[KR * (lw + NLW * j) * KW]);
#pragma unroll
            for (int j = 0; j < NVI; ++j) gll16v(vc + vo[j], &Bf.Vm[VR * (lw + NLW * j) * VW]);
        } else {
            const int cl = rem < CH ? (int)rem : CH;
            int ll = l;
            asm volatile("" : "+v"(ll));
            // instruction u covers rows KR u .. KR u + KR - 1 (lane: row KR u + ll / KG, slot ll % KG)
#pragma unroll
            for (int j = 0; j < NKI; ++j) {
                const int u = lw + NLW * j, r = KR * u + ll / KG, rs = r < cl ? r : cl - 1;
                gll16k(kh + (base + rs) * a.k_st + 8 * kswz(r, ll % KG), &Bf.Km[KR * u * KW]);
            }
#pragma unroll
            for (int j = 0; j < NVI; ++j) {
                const int u = lw + NLW * j, r = VR * u + ll / VG, rs = r < cl ? r : cl - 1;
                gll16v(vh + (base + rs) * a.v_st + 8 * vswz(r, ll % VG), &Bf.Vm[VR * u * VW]);
            }
        }
    };
    // diagonal: chunk C's gates and beta (LPG instructions per loading wave)
    auto issue_g = [&](int C, int lw, const uint32_t *go) {
        if constexpr (DIAG) {
            GateBuf &Gf = sm.gbuf[C % NBG];
            const int64_t base = (int64_t)C * CH, rem = n - base;
            if (rem >= CH && small_st) {
#pragma unroll
                for (int j = 0; j < NGI; ++j)
                    gll16(gh ? gh + base * a.la_st + go[j] : (const float *)a.k, &Gf.gate[(4 * lw + j) * 256]);
                gll4(bh ? bh + base * a.b_st + go[NGI] : (const float *)a.k, Gf.beta[lw]);
            } else {
                const int cl = rem < CH ? (int)rem : CH;
                int ll = l;
                asm volatile("" : "+v"(ll));
#pragma unroll
                for (int j = 0; j < NGI; ++j) {
                    const int r = 16 * j + (ll >> 2), rs = r < cl ? r : cl - 1;
                    gll16(gh ? gh + (base + rs) * a.la_st + 4 * (4 * lw + (ll & 3)) : (const float *)a.k,
                          &Gf.gate[(4 * lw + j) * 256]);
                }
                const int rs = ll < cl ? ll : cl - 1;
                gll4(bh ? bh + (base + rs) * a.b_st : (const float *)a.k, Gf.beta[lw]);
            }
        }
    };

    f32x16 st[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st[jb][r] = 0.f;
    double ell = 0.0;   // scalar: this thread's table tokens; diagonal: this lane's tokens of channel 32w + l32
    // scalar family: K^T and V^T fragments straight from the token-major tiles with the
    // transposing read.  Lane l (16-lane group g16 = l / 16, lane j = l % 16 in it, read
    // row a = j / 4, column piece b = j % 4) addresses token 8 (g16 / 2) + 4r + a of the
    // k-step's 16 (read r = 0, 1) and channel 32w + 16 (g16 % 2) + 4b (value column
    // 32 jb + 16 (g16 % 2) + 4b); the swizzle terms do not depend on the k-step, whose
    // offset is added per read.  Output: lane l's fragment of channel (column) l % 32,
    // tokens 16 ks + 8h + 0..7.
    // diagonal family: the same fragments from its half-width key rows (kmo_half) and
    // full-width value rows (kmo); wave w: key block w / 2, value blocks 2 (w % 2) + jb
    int dkofs[2], dvofs[2][NJB];
    {
        const int g16 = l >> 4, j = l & 15, ra = j >> 2, rb = j & 3;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int t = 8 * (g16 >> 1) + 4 * r + ra;
            const int ch = 32 * (w >> 1) + 16 * (g16 & 1) + 4 * rb;
            dkofs[r] = kmo_half(t, ch >> 3) + (ch & 7);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int cv = 32 * (2 * (w & 1) + jb) + 16 * (g16 & 1) + 4 * rb;
                dvofs[r][jb] = kmo(t, cv >> 3) + (cv & 7);
            }
        }
    }
    int kofs[2], vofs[2][NJB];
    {
        const int g16 = l >> 4, j = l & 15, ra = j >> 2, rb = j & 3;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int t = 8 * (g16 >> 1) + 4 * r + ra;
            const int ch = 32 * w + 16 * (g16 & 1) + 4 * rb;
            kofs[r] = kmo(t, ch >> 3) + (ch & 7);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const int cv = 32 * jb + 16 * (g16 & 1) + 4 * rb;
                vofs[r][jb] = vmo<NJB>(t, cv >> 3) + (cv & 7);
            }
        }
    }

    // Scalar family: the weight table of tokens [tb0, min(tb0 + TBT, n)); compute
    // thread th takes tokens tb0 + 8 th + 0..7 (inclusive prefix in the thread, then
    // over the wave with DPP, then over the waves through LDS).  Returns the block's
    // G_b and adds the thread's log alphas into ell.  Every compute wave calls it; the
    // loading waves pass its two barriers.
    auto make_table = [&](int64_t tb0) -> float {
        if constexpr (DIAG) return 0.0f;
        const int64_t tb1 = tb0 + TBT < n ? tb0 + TBT : n;
        float la8[8], b8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t t = tb0 + 8 * th + e;
            const bool ok = t < tb1;
            la8[e] = (ok && gh) ? gh[t * a.la_st] : 0.0f;
            b8[e] = ok ? (bh ? bh[t * a.b_st] : 1.0f) : 0.0f;
        }
        float run = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ell += (double)la8[e];
            run += la8[e];
            la8[e] = run;
        }
        const float incl = wave_prefix_sum(run);
        if (l == 63) sm.wtot[w] = incl;
        lds_barrier();
        float woff = 0.0f, G = 0.0f;
#pragma unroll
        for (int u = 0; u < NWC; ++u) {
            const float x = sm.wtot[u];
            woff += u < w ? x : 0.0f;
            G += x;
        }
        const float base = woff + incl - run;         // cumulative before this thread's tokens
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.wt[8 * th + e] = b8[e] * __expf(G - (base + la8[e]));
        lds_barrier();                                // table visible; wtot free again
        return G;
    };

    // Diagonal family: the factors of chunk C for the workgroup key channels ch0 .. ch0 + 15,
    // computed by factor wave f (ch0 = 16 f) one chunk ahead of their use.  Lane l takes
    // channel ch0 + l / 4 and the tokens 16 (l % 4) .. + 15 (the channel's four lanes form
    // a quad):
    //   L_t (inclusive cumulative log decay of the channel), G = L_63,
    //   fac[ci][t] = beta_t e^{G - L_t},  eg[ci] = e^G,
    // written to the parity-C tiles; ell_acc collects the lane's log decays.  The gates
    // were loaded by the loading waves, each of which waited for its own before the
    // barrier that starts the chunk these factors are computed in.
    // (in two parts: the gate and beta reads, all issued before the arithmetic)
    struct FacIn { float x[16], bt[16]; };
    auto factors16_read = [&](int C, int ch0, FacIn &fi) {
        if constexpr (DIAG) {
            const GateBuf &Bf = sm.gbuf[C % NBG];
            const int cc = l >> 2, q4 = l & 3, ci = ch0 + cc, t0 = 16 * q4;
#pragma unroll
            for (int j = 0; j < 16; ++j) fi.x[j] = Bf.gate[gate_idx(t0 + j, ci)];
            // the lane's sixteen betas, read before any factor is stored (the stores could
            // alias them for all the compiler knows, which would serialise the reads)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 b4 = *reinterpret_cast<const float4 *>(&Bf.beta[0][t0 + 4 * g]);
                fi.bt[4 * g] = b4.x; fi.bt[4 * g + 1] = b4.y; fi.bt[4 * g + 2] = b4.z; fi.bt[4 * g + 3] = b4.w;
            }
        }
    };
    auto factors16 = [&](int C, int ch0, FacIn &fi, double &ell_acc) {
        if constexpr (DIAG) {
            const int64_t rem = n - (int64_t)C * CH;
            const int cl = rem < CH ? (int)rem : CH;
            const int cc = l >> 2, q4 = l & 3, ci = ch0 + cc, t0 = 16 * q4;
            float *x = fi.x;
            const float *bt = fi.bt;
            float run = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                run += (t0 + j < cl && a.log_alpha) ? x[j] : 0.0f;
                x[j] = run;
            }
            ell_acc += (double)run;
            // over the quad, in registers: inclusive scan by lane shifts of 1 and 2, total
            // by two pairwise exchanges
            float incl = run;
            {
                const float y1 = dpp_f32<0x90>(incl);           // quad_perm [0, 0, 1, 2]
                if (q4 >= 1) incl += y1;
                const float y2 = dpp_f32<0x40>(incl);           // quad_perm [0, 0, 0, 1]
                if (q4 >= 2) incl += y2;
            }
            float G = run + dpp_f32<0xB1>(run);                 // quad_perm [1, 0, 3, 2]
            G += dpp_f32<0x4E>(G);                              // quad_perm [2, 3, 0, 1]
            const float off = incl - run;
            const int par = (int)(C & 1);
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                float f[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = t0 + 4 * gq + e;
                    const float b = t < cl ? (a.beta ? bt[4 * gq + e] : 1.0f) : 0.0f;
                    f[e] = b * __expf(G - (off + x[4 * gq + e]));
                }
                *reinterpret_cast<float4 *>(&sm.fac[par][fac_idx(ci, 4 * q4 + gq)]) = make_float4(f[0], f[1], f[2], f[3]);
            }
            if (q4 == 0) sm.eg[par][ci] = __expf(G);
        }
    };
    // the record's ell of those channels: the sum of the channel's four lanes
    auto write_ell16 = [&](double ell_acc, int ch0) {
        if constexpr (DIAG) {
            ell_acc += __shfl_xor(ell_acc, 1);
            ell_acc += __shfl_xor(ell_acc, 2);
            if ((l & 3) == 0)
                a.pool_ell[((int64_t)slot * a.H + head) * D + kc0 + ch0 + (l >> 2)] =
                    state == 2 ? __int_as_float(0x7fc00000) : (float)ell_acc;
        }
    };

    if constexpr (DIAG) {
        if (w >= NWC + NLW) {
            // ================= factor waves (diagonal): during chunk c, the factors and
            // decay of chunk c + 1 from its gates (which the loading waves waited for
            // before the barrier that starts chunk c), into the parity-(c + 1) tiles that
            // the compute waves last read in chunk c - 1; the same barriers as the others
            const int fw = w - NWC - NLW;
            double ell16 = 0.0;
            FacIn fi;
            lds_barrier();                            // gates of chunk 0 visible
            if (nc > 0) {
                factors16_read(0, 16 * fw, fi);
                factors16(0, 16 * fw, fi, ell16);
            }
            for (int c = 0; c < nc; ++c) {
                lds_barrier();                        // gates of chunk c + 1 visible; chunk c's factors published
                if (c + 1 < nc) {
                    factors16_read(c + 1, 16 * fw, fi);
                    factors16(c + 1, 16 * fw, fi, ell16);
                }
            }
            write_ell16(ell16, 16 * fw);
            return;
        }
    }
    if (w >= NWC) {
        // ================= loading waves: the same barriers as the compute waves
        const int lw = w - NWC;
        uint32_t ko[NKI], vo[NVI], go[NGI + 1];
#pragma unroll
        for (int j = 0; j < NKI; ++j) {
            const int r = KR * (lw + NLW * j) + l / KG;
            ko[j] = small_st ? (uint32_t)(r * a.k_st + 8 * kswz(r, l % KG)) : 0u;
        }
#pragma unroll
        for (int j = 0; j < NVI; ++j) {
            const int r = VR * (lw + NLW * j) + l / VG;
            vo[j] = small_st ? (uint32_t)(r * a.v_st + 8 * vswz(r, l % VG)) : 0u;
        }
#pragma unroll
        for (int j = 0; j < NGI; ++j) {
            const int r = 16 * j + (l >> 2);
            go[j] = small_st ? (uint32_t)(r * a.la_st + 4 * (4 * lw + (l & 3))) : 0u;
        }
        go[NGI] = small_st ? (uint32_t)(l * a.b_st) : 0u;
        if (!DIAG)
            for (int c = 0; c < DIST && c < nc; ++c) issue(c, lw, ko, vo, go);
        if constexpr (DIAG) {
            // Issue order: "step" j >= -3 issues the gates of chunk j + 3, then the keys and
            // values of chunk j + 2 (those that exist); steps -3 .. -1 run before the loop,
            // step c after the barrier of chunk c.  A wait names how many of this wave's
            // loads were issued after the one it waits for.  Before the barrier that starts
            // chunk c every loading wave has waited for its gates of chunk c + 1, which the
            // compute waves turn into factors during chunk c.
            auto nG = [&](int m) { return m < nc ? LPG : 0; };
            auto nKV = [&](int m) { return m < nc ? LPW : 0; };
            for (int j = -3; j < 0; ++j) {
                if (j + 3 < nc) issue_g(j + 3, lw, go);
                if (j + 2 >= 0 && j + 2 < nc) issue(j + 2, lw, ko, vo, go);
            }
            vm_wait<2 * LPG + 3 * LPW>(nG(1) + nKV(0) + nG(2) + nKV(1));   // gates of chunk 0
            lds_barrier();                                                  // ... visible to all
            vm_wait<2 * LPG + 3 * LPW>(nG(2) + nKV(1));                    // gates 1, keys, values 0
            for (int c = 0; c < nc; ++c) {
                lds_barrier();                            // chunk c (and its factors) visible
                if (c + 3 < nc) issue_g(c + 3, lw, go);
                if (c + 2 < nc) issue(c + 2, lw, ko, vo, go);
                vm_wait<2 * LPG + 3 * LPW>(nG(c + 3) + nKV(c + 2));       // gates c + 2, keys, values c + 1
            }
            return;
        }
        // make_table's two barriers (these waves have no tokens, and no load to wait for)
        if (!DIAG) {
            lds_barrier();
            lds_barrier();
            if (AHEAD) {
                if (nc > 0) {
                    // chunk 0 landed: the compute waves read its operands before their loop
                    const int issued = (DIST - 1 < nc - 1 ? DIST - 1 : nc - 1);
                    wait_chunks<LPW, DIST - 1>((int)issued);
                }
                lds_barrier();
            }
        }
        for (int c = 0; c < nc; ++c) {
            // chunk c + AHEAD has landed once at most the later chunks' loads remain
            {
                const int issued = c + DIST - 1 < nc - 1 ? c + DIST - 1 : nc - 1;
                const int need = c + AHEAD < nc - 1 ? c + AHEAD : nc - 1;
                wait_chunks<LPW, DIST - 1>((int)(issued - need));
            }
            lds_barrier();                            // chunk c + AHEAD visible; chunk c - 1's buffer free
            if (c + DIST < nc) issue(c + DIST, lw, ko, vo, go);
            if (!DIAG && c > 0 && c % TBC == 0) {
                lds_barrier();
                lds_barrier();
            }
        }
        return;
    }

    // ================= compute waves
    if constexpr (!DIAG) {
        // ---- S += K^T diag(w) V with the table's weights, 16 tokens per k-step; the
        //      weights go onto the K^T fragment (one scaling serves every value block).
        //      With AHEAD, a chunk's K^T and V fragments are read during the previous
        //      chunk's products (two register sets, the loop unrolled by two).
        struct Ops {
            bf16x8 kr[4], vb[4][NJB];
        };
        auto load_ops = [&](int cc, Ops &o) {
            const SdBuf<DIAG, NJB> &B = sm.buf[cc % NBUF];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                o.kr[ks] = tr_pair(&B.Km[kofs[0] + 16 * ks * D], &B.Km[kofs[1] + 16 * ks * D]);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
                    o.vb[ks][jb] = tr_pair(&B.Vm[vofs[0][jb] + 16 * ks * 32 * NJB],
                                           &B.Vm[vofs[1][jb] + 16 * ks * 32 * NJB]);
            }
        };
        auto step = [&](int cc, Ops &cur, Ops &nxt) {
            lds_barrier();                            // chunk cc + AHEAD visible; chunk cc - 1's buffer free
            if (cc > 0 && cc % TBC == 0) {
                // a new table block: carry the state into it (every wave is past chunk cc - 1)
                const float eG = __expf(make_table((int64_t)cc * CH));
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) st[jb][r] *= eG;
            }
            if (!AHEAD) load_ops(cc, cur);
            else if (cc + 1 < nc) load_ops(cc + 1, nxt);
            const float *wrow = &sm.wt[CH * (int)(cc % TBC)];
            float4 w0[4], w1[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                w0[ks] = *reinterpret_cast<const float4 *>(&wrow[16 * ks + 8 * h]);
                w1[ks] = *reinterpret_cast<const float4 *>(&wrow[16 * ks + 8 * h + 4]);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 ka = scale8(cur.kr[ks], w0[ks], w1[ks]);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) st[jb] = mfma(ka, cur.vb[ks][jb], st[jb]);
            }
        };
        make_table(0);
        Ops oa, ob;
        if constexpr (AHEAD) {
            lds_barrier();                            // chunk 0 visible
            if (nc > 0) load_ops(0, oa);
            for (int c = 0; c < nc; c += 2) {
                step(c, oa, ob);
                if (c + 1 < nc) step(c + 1, ob, oa);
            }
        } else {
            for (int c = 0; c < nc; ++c) step(c, oa, oa);
        }
    } else {
    // the chunk's factors (computed by the factor waves one chunk ahead): decay, scale, multiply
    const int i = 32 * (w >> 1) + l32;                // this lane's key channel (of the workgroup's 64)
    lds_barrier();                                    // gates of chunk 0 visible
    for (int c = 0; c < nc; ++c) {
        lds_barrier();                                // chunk c and its factors visible; chunk c - 1's buffer free
        const SdBuf<DIAG, NJB> &B = sm.buf[c % NBUF];
        const int par = (int)(c & 1);
        // ---- operand reads: K^T and V^T fragments (transposing read), the factors of
        //      this lane's K^T fragment tokens 16 ks + 8 h + 0..7, the rows' chunk decay
        bf16x8 kr[4], vb[4][NJB];
        float4 f0[4], f1[4], g4[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            kr[ks] = tr_pair(&B.Km[dkofs[0] + 16 * ks * DKC], &B.Km[dkofs[1] + 16 * ks * DKC]);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
                vb[ks][jb] = tr_pair(&B.Vm[dvofs[0][jb] + 16 * ks * D], &B.Vm[dvofs[1][jb] + 16 * ks * D]);
            f0[ks] = *reinterpret_cast<const float4 *>(&sm.fac[par][fac_idx(i, 4 * ks + 2 * h)]);
            f1[ks] = *reinterpret_cast<const float4 *>(&sm.fac[par][fac_idx(i, 4 * ks + 2 * h + 1)]);
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
            g4[qq] = *reinterpret_cast<const float4 *>(&sm.eg[par][32 * (w >> 1) + 8 * qq + 4 * h]);
        // ---- decay of the carried state: row (key channel) r of a tile by e^{G_r}
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const float f[4] = {g4[qq].x, g4[qq].y, g4[qq].z, g4[qq].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) st[jb][4 * qq + e] *= f[e];
        }
        // ---- S += (W . K)^T V, W[t][i] = beta_t e^{G_i - L_{t,i}} on the K^T fragment
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 ka = scale8(kr[ks], f0[ks], f1[ks]);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) st[jb] = mfma(ka, vb[ks][jb], st[jb]);
        }
    }
    }
    // ---- record
    const float nanv = __int_as_float(0x7fc00000);
    const bool bad = state == 2;
    const int64_t rec = slot * a.H + head;
    float *dst = a.pool_S + rec * D * D;
    // rows (key channels) and first column of this wave's tiles
    const int row0 = DIAG ? kc0 + 32 * (w >> 1) : 32 * w;
    const int col0 = DIAG ? 64 * (w & 1) : jc0;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            dst[(int64_t)(row0 + acc_row(r, h)) * D + col0 + 32 * jb + l32] = bad ? nanv : st[jb][r];
    if (DIAG) {
        // (the loading waves wrote the channels' ell)
    } else {
        if (q != 0) return;
        // every thread summed its table tokens
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ell += __shfl_xor(ell, o);
        if (l == 0) sm.ellw[w] = ell;
        lds_barrier();
        if (th == 0) a.pool_ell[rec] = bad ? nanv : (float)(sm.ellw[0] + sm.ellw[1] + sm.ellw[2] + sm.ellw[3]);
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
    // (the diagonal family always splits in two: its whole state plus the per-channel
    // gate work does not fit the registers a wave has beside the loading wave; the
    // scalar family stages all keys in every split, so it splits only below 256 units)
    const bool diag = a.family == HYPIC_DIAGONAL;
    const int nsplit = diag ? 2 : (units >= 256 ? 1 : units >= 128 ? 2 : 4);
    const int64_t padded = (units + 7) / 8 * 8;
    const dim3 grid((unsigned)(padded * nsplit));
#define HYPIC_SD_LAUNCH(FAM_, NS_) \
    hipLaunchKernelGGL((sd_build_mfma_kernel<FAM_, NS_>), grid, dim3(FAM_ == HYPIC_DIAGONAL ? NT_DIAG : NT), 0, stream, a)
    if (a.family == HYPIC_SCALAR) {
        if (nsplit == 1) HYPIC_SD_LAUNCH(HYPIC_SCALAR, 1);
        else if (nsplit == 2) HYPIC_SD_LAUNCH(HYPIC_SCALAR, 2);
        else HYPIC_SD_LAUNCH(HYPIC_SCALAR, 4);
    } else {
        HYPIC_SD_LAUNCH(HYPIC_DIAGONAL, 2);
    }
#undef HYPIC_SD_LAUNCH
    return hipGetLastError();
}

}  // namespace hypic
