// Segment-record build on MFMA: GDN family, d_k = d_v = 128, bf16 k/v,
// fp32 records.  bf16 MFMA operands, fp32 accumulation, fp64 ell.
//
// What it computes (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4; agihunt summary, "Core Approach"): the record (ell, P, S) of
// every (segment, head), T_C = e^ell P, for A_t = alpha_t (I - beta_t k_t k_t^T)
// (Gated Delta Networks, podcast companion page, reference 7).
//
// Chunked WY/UT form, chunk = 64 tokens, g = in-chunk cumulative log decay,
// G = chunk total (the plain-arithmetic statement is in build_ref.hip):
//   A0 = strictlower(beta_t k_t.k_s),   A = A0 . e^{g_t - g_s}
//   P columns X:  Y = (I + A0)^{-1} (beta . (K X));                X <- X - K^T Y
//   S columns X:  Y = (I + A )^{-1} (beta . (V - e^g . (K X)));    X <- e^G X + K^T (e^{G-g} . Y)
// The P update uses the ungated system, so no decay factor can overflow it.
// With 32-token blocks, T_ii = (I + A_ii)^{-1} and A = diag(beta) H (H: the
// block of k_t.k_s, with e^{g_t - g_s} for S, without beta),
//     Y_1 = (T_11 diag beta_1) W_1,    Y_2 = (T_22 diag beta_2) (W_2 - H_21 Y_1),
// so each system needs two 32x32 inverse factors and H_21 per chunk.
//
// Work split: 512-thread workgroups, each taking every G-th (segment, head) unit
// (G: the grid, a multiple of the CU count; at most TMAX units per workgroup) and
// running their chunks as one stream, so that one unit's last chunk, its record
// write and the next unit's first chunk overlap as any two chunks do.  At set-up
// each thread reads one unit's offsets and slot: units with an out-of-range slot
// raise the flag, empty units and units with bad offsets get their identity or NaN
// record written by the whole workgroup, and the rest go into an LDS table in order.
// Every wave then walks the same chunk stream through that table.  Two roles:
//  * State waves 0-3 each own 32 columns of P and the same 32 columns of S
//    as eight fp32 32x32 accumulator tiles that stay in registers for the
//    whole unit (so the four waves do identical work).  Per chunk: W = K X
//    (and V - e^g . W for S), the block solve against the factors (three
//    dependent products), and the update; after a unit's last chunk, its record
//    and the reset of the accumulators to (I, 0).
//  * Prep waves 4-7 build the next chunk's factors meanwhile: the decay
//    prefix, the Gram blocks (A11, A22 in fp32, H_21 in bf16); the inverses
//    of the 32x32 diagonal blocks (4x4 forward substitution and fp32 merges
//    up to 16, one 16 -> 32 merge on the MFMA), written as T diag(beta) in
//    bf16 by each level as it finishes.  Wave 4 also loads keys and values
//    into LDS and computes the decay factors; waves 5 and 7 invert the two
//    diagonal blocks; waves 4 and 6 turn K^T around for the update in phase b.
// Two workgroup barriers per chunk: in phase a the state waves finish chunk
// c - 1 (solve, update) while the prep waves compute A of chunk c; in phase b
// the state waves form W of chunk c while the prep waves invert.
//
// Layout facts used throughout (v_mfma_f32_32x32x16_bf16): the accumulator
// and the B operand both put one column per lane, so an accumulator tile is
// the B operand of the next product after a bf16 pack (acc_to_b); the pack
// feeds contraction indices 16 half + 4h + 0..3 and 16 half + 8 + 4h + 0..3 from
// lane half h.  The rows of every state-side accumulator are kept in swizzled
// order (physical row p holds index swz(p), bits 2 and 3 swapped) so that
// those indices become 16 half + 8h + 0..7: every A operand is then one
// 16-byte LDS read from a plain row-major tile, at row swz(lane).
// X . I on the MFMA moves a token-major tile into the accumulator layout
// (one column per lane); that gives K^T and the V term of W.
#include "gdn_mfma_common.h"

namespace hypic {
namespace {

constexpr int NT = 512;    // 4 state waves + 4 prep waves
constexpr int TMAX = 512;  // units per workgroup: one per thread at set-up

struct __align__(16) Smem {
    static constexpr bool kWithP = true;
    static constexpr int kTmax = TMAX;
    static constexpr int kS = 1;
    u16 Km[2][CH * KML];       // keys, token-major, double-buffered by chunk parity
    u16 Vm[2][CH * KML];       // values, token-major, double-buffered by chunk parity
    u16 Kt[D * KTL];           // keys, channel-major
    u16 TB[2][2][2][32 * TBL]; // [chunk parity][system]: T_11 diag(beta_1), T_22 diag(beta_2) (negated for P)
    u16 H21[2][2][32 * TBL];   // [chunk parity][system]: H_21 (P), -H_21 (S), row t, column s
    float Af[2][32 * AFL];     // diagonal blocks of A0 (P system), inverted in place
    float pv[4][2][CH];        // per prep wave: g, beta of the chunk being prepared
    float inv_tmp[4][128];     // per prep wave: products inside the blocked inversion
    float egs[2][CH];          // -e^{g_t} sigma_c: the K X factor of W (S columns)
    float egrs[2][CH];         // e^{G - g_t} / sigma_{c+1}: the update factor (S columns)
    float bsv[CH];             // beta_t e^{G - g_t} / sigma_{c+1} (wave 7): the S factor of block 2
    float rs[2];               // sigma_c e^G when the scale is folded back into the state, else 1
    float sig_fin[2];          // sigma after the chunk of that parity (S = sigma X at a unit's end)
    UnitEnt units[TMAX];       // the stream's units from the front, set-up records from the back
    int64_t wsum[8];           // set-up: per wave, chunks of its valid units
    int32_t wcnt[8][2];        // set-up: per wave, valid units and set-up records
    int32_t steps;             // chunks in the stream (a workgroup's units fit in memory: far below 2^31)
    int32_t nvalid, nspecial;
};

__global__ __launch_bounds__(NT, 1) void gdn_build_mfma_kernel(BuildArgs a) {
    __shared__ Smem sm;

    const int th = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(th >> 6);
    const int lane = th & 63;

    // ---- set-up: the workgroup's units tabled, the records of empty units and bad
    //      offsets written (the launch keeps the unit count within TMAX = NT)
    // the upper triangles of the T diag(beta) tiles stay zero for the whole launch
    for (int e = th; e < (int)(sizeof(sm.TB) / 16); e += NT) reinterpret_cast<u32x4 *>(&sm.TB[0][0][0][0])[e] = u32x4{};
    stream_setup<Smem, NT>(sm, a, true);
    const int nvalid = uni32(sm.nvalid);
    const int steps = uni32(sm.steps);
    stream_special_records<Smem, NT>(sm, a);

    if (w < 4) {
        // =============================== state waves ===============================
        // column block 0: P columns 32w .. 32w + 31; column block 1: the same S columns
        const int col = 32 * w;
        f32x16 st[2][4];                          // [column block][row block], rows swizzled
        bf16x8 wb[2][2][2];                       // W of the chunk in flight as B operands [cb][tb][half]
        // (P, S) = (I, 0), the state before a unit's first chunk
#define HYPIC_STATE_RESET(HH, L32)                                                                   \
    _Pragma("unroll") for (int cb_ = 0; cb_ < 2; ++cb_)                                              \
        _Pragma("unroll") for (int mb_ = 0; mb_ < 4; ++mb_)                                          \
            _Pragma("unroll") for (int r_ = 0; r_ < 16; ++r_)                                        \
                st[cb_][mb_][r_] = (cb_ == 0 && swz(32 * mb_ + acc_row(r_, (HH))) == col + (L32)) ? 1.0f : 0.0f
        HYPIC_STATE_RESET(lane >> 5, lane & 31);
        __syncthreads();                                            // prologue: chunk 0 staged
        Cursor cs = cursor_first(sm, nvalid);                      // chunk i (phase b)
        for (int i = 0; i <= steps; ++i) {
            int thv = th;
            asm volatile("" : "+v"(thv));
            const int h = (thv & 63) >> 5, l32 = thv & 31;
            // ---- phase a: solve and update of chunk i - 1
            if (i >= 1) {
                const int b = (int)((i - 1) & 1);
                const int rr = swz(l32) * TBL + 8 * h;
                {
                    const float rsc = sm.rs[b];
                    if (rsc != 1.0f) {
                        // the pending decay sigma_c e^G is folded into the S state (rare)
#pragma unroll
                        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) st[1][mb][r] *= rsc;
                    }
                }
                // factor operands [system][k-step]: T_11 diag b_1 and H_21 read up front
                bf16x8 f0[2][2], fh[2][2], f1[2][2];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        f0[cb][half] = lds8(&sm.TB[b][cb][0][rr + 16 * half]);
                        fh[cb][half] = lds8(&sm.H21[b][cb][rr + 16 * half]);
                    }
                f32x16 y1[2], y2[2];     // [column block = system]
                bf16x8 yb[4][2];         // B operands of the update, [k-step][system]
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    y1[cb] = mfma(f0[cb][0], wb[cb][0][0], f32x16{});
                    y1[cb] = mfma(f0[cb][1], wb[cb][0][1], y1[cb]);
                }
                // W_2 - H_21 Y_1 (H21 carries the sign that makes this a sum for both
                // systems; P's factors and Y are negated), accumulated onto W_2 itself: a
                // B operand pack holds the registers of its accumulator in order
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const f32x8 w0 = __builtin_convertvector(wb[cb][1][0], f32x8);
                    const f32x8 w1 = __builtin_convertvector(wb[cb][1][1], f32x8);
                    y2[cb] = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
                    yb[0][cb] = acc_to_b(y1[cb], 0);
                    yb[1][cb] = acc_to_b(y1[cb], 1);
                    y2[cb] = mfma(fh[cb][0], yb[0][cb], y2[cb]);
                    y2[cb] = mfma(fh[cb][1], yb[1][cb], y2[cb]);
                }
                // S: Y_1 times e^{G - g} / sigma for the update
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 e0 = tok4(sm.egrs[b], 0, q, h);
                    y1[1][4 * q] *= e0.x; y1[1][4 * q + 1] *= e0.y;
                    y1[1][4 * q + 2] *= e0.z; y1[1][4 * q + 3] *= e0.w;
                }
                yb[0][1] = acc_to_b(y1[1], 0);
                yb[1][1] = acc_to_b(y1[1], 1);
                // T_22 diag b_2, read while the first half of the update runs
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int half = 0; half < 2; ++half) f1[cb][half] = lds8(&sm.TB[b][cb][1][rr + 16 * half]);
                // X += K^T Y (the P factors are stored negated): A operand = Kt rows (channels)
                // swz(32 mb + lane); token steps 0, 1 need only Y_1, so they overlap the
                // Y_2 chain below
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    bf16x8 kt[4];
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) kt[mb] = lds8(&sm.Kt[swz(32 * mb + l32) * KTL + 16 * s2 + 8 * h]);
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                        for (int cb = 0; cb < 2; ++cb) st[cb][mb] = mfma(kt[mb], yb[s2][cb], st[cb][mb]);
                }
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const bf16x8 u0 = acc_to_b(y2[cb], 0), u1 = acc_to_b(y2[cb], 1);
                    y2[cb] = mfma(f1[cb][0], u0, f32x16{});
                    y2[cb] = mfma(f1[cb][1], u1, y2[cb]);
                }
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    yb[2][cb] = acc_to_b(y2[cb], 0);
                    yb[3][cb] = acc_to_b(y2[cb], 1);
                }
#pragma unroll
                for (int s2 = 2; s2 < 4; ++s2) {
                    bf16x8 kt[4];
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb) kt[mb] = lds8(&sm.Kt[swz(32 * mb + l32) * KTL + 16 * s2 + 8 * h]);
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                        for (int cb = 0; cb < 2; ++cb) st[cb][mb] = mfma(kt[mb], yb[s2][cb], st[cb][mb]);
                }
            }
            lds_barrier();                                          // a -> b
            // ---- phase b: W of chunk i; the record of the unit that ended with chunk i - 1
            //      (physical row p of a tile holds channel swz(p); S = sigma X), then the
            //      state of the next unit
            const bool pend = i >= 1 && cs.c == 0;
#define HYPIC_RECORD()                                                                               \
    do {                                                                                             \
        const int64_t rec_ = uni32(sm.units[cs.q - 1].rec);                                          \
        const float sfin_ = sm.sig_fin[(int)((i - 1) & 1)];                                          \
        /* tile row swz(32 mb + acc_row(r, h)) = 8 h + 32 mb + 16 (r >> 3) + 4 ((r >> 2) & 1) + (r & 3): \
           one lane offset for every store, the row's constant part in the scalar offset */         \
        const int lo_ = 4 * (8 * h * D + col + l32);                                                 \
        _Pragma("unroll") for (int cb_ = 0; cb_ < 2; ++cb_) {                                        \
            const __amdgpu_buffer_rsrc_t rs_ = __builtin_amdgcn_make_buffer_rsrc(                    \
                (cb_ == 0 ? a.pool_P : a.pool_S) + rec_ * D * D, (short)0, D * D * 4, RSRC_WORD3);   \
            const float sc_ = cb_ == 0 ? 1.0f : sfin_;                                               \
            _Pragma("unroll") for (int mb_ = 0; mb_ < 4; ++mb_)                                      \
                _Pragma("unroll") for (int r_ = 0; r_ < 16; ++r_)                                    \
                    __builtin_amdgcn_raw_buffer_store_b32(                                           \
                        __float_as_uint(st[cb_][mb_][r_] * sc_), rs_, lo_,                           \
                        4 * D * (32 * mb_ + 16 * (r_ >> 3) + 4 * ((r_ >> 2) & 1) + (r_ & 3)), 0);     \
        }                                                                                            \
    } while (0)
            if (i < steps) {
                const int b = (int)(i & 1);
                f32x16 z[2][2];                   // [column block][token block], rows swizzled
                if (cs.c == 0) {
                    // a unit's first chunk: the previous unit's record goes out first (its
                    // stores drain while the products below run); with X = (I, 0), W =
                    // (K X_P, V) is this wave's columns of K and V, turned around on the MFMA
                    if (pend) {
                        HYPIC_RECORD();
                        HYPIC_STATE_RESET(h, l32);
                    }
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const bf16x8 eye = eye_b(ks, h, l32);
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb) {
                            const int o = kmo(swz(32 * mb + l32), 4 * w + 2 * ks + h);
                            z[0][mb] = mfma(lds8(&sm.Km[b][o]), eye, ks == 0 ? f32x16{} : z[0][mb]);
                            z[1][mb] = mfma(lds8(&sm.Vm[b][o]), eye, ks == 0 ? f32x16{} : z[1][mb]);
                        }
                    }
                } else {
                    // K X: A operand = Km rows (tokens) swz(32 mb + lane), B = state rows in swizzled order
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) {
                        bf16x8 sb[2];
#pragma unroll
                        for (int cb = 0; cb < 2; ++cb) sb[cb] = acc_to_b(st[cb][kb >> 1], kb & 1);
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb) {
                            const bf16x8 km = lds8(&sm.Km[b][kmo(swz(32 * mb + l32), 2 * kb + h)]);
#pragma unroll
                            for (int cb = 0; cb < 2; ++cb)
                                z[cb][mb] = mfma(km, sb[cb], kb == 0 ? f32x16{} : z[cb][mb]);
                        }
                    }
                    {
                        // S block: W = V - e^g . (K X): scale, then add V turned around on the MFMA
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const float4 e4 = tok4(sm.egs[b], mb, q, h);
                                z[1][mb][4 * q] *= e4.x; z[1][mb][4 * q + 1] *= e4.y;
                                z[1][mb][4 * q + 2] *= e4.z; z[1][mb][4 * q + 3] *= e4.w;
                            }
#pragma unroll
                        for (int ks = 0; ks < 2; ++ks) {
                            const bf16x8 eye = eye_b(ks, h, l32);
#pragma unroll
                            for (int mb = 0; mb < 2; ++mb)
                                z[1][mb] = mfma(lds8(&sm.Vm[b][kmo(swz(32 * mb + l32), 4 * w + 2 * ks + h)]), eye, z[1][mb]);
                        }
                    }
                }
                // kept across the barrier as bf16 B operands: half the registers of W
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int half = 0; half < 2; ++half) wb[cb][mb][half] = acc_to_b(z[cb][mb], half);
            } else if (pend) {
                HYPIC_RECORD();                                     // the last unit
            }
            __syncthreads();                                        // b -> next a
            cursor_next(sm, nvalid, cs);
        }
#undef HYPIC_RECORD
#undef HYPIC_STATE_RESET
    } else {
        // =============================== prep waves ===============================
        // Their work is a chain of short dependent steps that shares each SIMD with a
        // state wave's long MFMA stream: issue priority keeps the chain moving.
        __builtin_amdgcn_s_setprio(3);
        const int pw = w - 4;
        const int pl = th & 63;
        // every prep wave loads la and beta of a chunk itself (lane = token)
        float lar = 0.f, br = 0.f;
#define HYPIC_FETCH_G(DESC)                                                                          \
    do {                                                                                             \
        const StepDesc d_ = (DESC);                                                                  \
        const int64_t tk_ = d_.tok + pl;                                                             \
        br = pl < d_.cl ? (a.beta ? a.beta[tk_ * a.b_st + d_.head * a.b_sh] : 1.0f) : 0.0f;          \
        lar = (pl < d_.cl && a.log_alpha) ? a.log_alpha[tk_ * a.la_st + d_.head * a.la_sh] : 0.0f;   \
    } while (0)
        Cursor nxt = cursor_first(sm, nvalid);                     // chunk i + 1 (chunk 0 here)
        if (steps > 0) HYPIC_FETCH_G(step_desc(nxt));
        if (pw == 0) {
            // ---- wave 4: loads keys and values, the decay factors and ell in phase a;
            //      turns K^T around for tokens 0-31 of the chunk in phase b.
            // Keys and values go straight from HBM into Km/Vm (global_load_lds): the
            // instruction for rows 4u .. 4u + 3 lands lane l's 16 bytes in row 4u + l / 16,
            // slot l % 16, so the lane loads the granule that kmo puts there.  Rows past
            // the unit repeat its last row (finite values; their beta is zero).
            const u16 *kp = static_cast<const u16 *>(a.k), *vp = static_cast<const u16 *>(a.v);
            // full chunks (the common case): element offsets of this lane's sixteen
            // pieces, relative to the chunk's first row, fixed for the whole launch
            const bool small_st = (int64_t)CH * (a.k_st > a.v_st ? a.k_st : a.v_st) < (1LL << 30);
            uint32_t ko[16], vo[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int t = 4 * u + (pl >> 4), g = (pl & 15) ^ (t & 15);
                ko[u] = small_st ? (uint32_t)(t * a.k_st + 8 * g) : 0u;
                vo[u] = small_st ? (uint32_t)(t * a.v_st + 8 * g) : 0u;
            }
#define HYPIC_LOAD_KV(DESC, BUF)                                                                     \
    do {                                                                                             \
        const StepDesc d_ = (DESC);                                                                  \
        const u16 *kc_ = kp + d_.tok * a.k_st + d_.head * a.k_sh;                                    \
        const u16 *vc_ = vp + d_.tok * a.v_st + d_.head * a.v_sh;                                    \
        if (d_.cl == CH && small_st) {                                                               \
            _Pragma("unroll") for (int u_ = 0; u_ < 16; ++u_) {                                      \
                __builtin_amdgcn_global_load_lds(kc_ + ko[u_], &sm.Km[BUF][4 * u_ * KML], 16, 0, kLoadNT); \
                __builtin_amdgcn_global_load_lds(vc_ + vo[u_], &sm.Vm[BUF][4 * u_ * KML], 16, 0, kLoadNT); \
            }                                                                                        \
        } else {                                                                                     \
            const int cl_ = d_.cl;                                                                   \
            int l_ = pl;                                                                             \
            asm volatile("" : "+v"(l_));                                                             \
            const int r_ = l_ >> 4, p_ = l_ & 15;                                                    \
            _Pragma("unroll") for (int u_ = 0; u_ < 16; ++u_) {                                      \
                const int t_ = 4 * u_ + r_, ts_ = t_ < cl_ ? t_ : cl_ - 1;                           \
                const int g_ = p_ ^ (t_ & 15);                                                       \
                __builtin_amdgcn_global_load_lds(kc_ + ts_ * a.k_st + 8 * g_,                        \
                                                 &sm.Km[BUF][4 * u_ * KML], 16, 0, kLoadNT);         \
                __builtin_amdgcn_global_load_lds(vc_ + ts_ * a.v_st + 8 * g_,                        \
                                                 &sm.Vm[BUF][4 * u_ * KML], 16, 0, kLoadNT);         \
            }                                                                                        \
        }                                                                                            \
    } while (0)
            double ell = 0.0;     // this lane's tokens of the unit; summed over the wave at its end
            // S = sigma X for the S columns: the decay e^G of each chunk is carried in
            // sigma and folded into X only when sigma would drop below 2^-60, so the
            // state waves do not rescale X every chunk.
            float sig = 1.0f;
            if (steps > 0) {
                HYPIC_LOAD_KV(step_desc(nxt), 0);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            // chunk i: its unit, its index in the unit and the unit's chunk count
            int cq = nxt.q, cc = nxt.c, cnc = nxt.nc;
            cursor_next(sm, nvalid, nxt);
            __syncthreads();                                        // prologue: chunk 0 staged
            for (int i = 0; i <= steps; ++i) {
                int thv = th;
                asm volatile("" : "+v"(thv));
                const int l = thv & 63;
                // ---- phase a: decay factors of chunk i; keys and values of chunk i + 1 start
                if (i < steps) {
                    const int b = (int)(i & 1);
                    const float la_i = lar, b_i = br;
                    if (i + 1 < steps) HYPIC_LOAD_KV(step_desc(nxt), b ^ 1);   // lands during this chunk
                    if (cc == 0) sig = 1.0f;
                    const float gv = wave_prefix_sum(la_i);
                    sm.pv[0][0][l] = gv;
                    sm.pv[0][1][l] = b_i;
                    const float gt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 63));
                    const float sp = sig * __expf(gt);
                    const bool fold = sp < 0x1p-60f;
                    const float inv = fold ? 1.0f : 1.0f / sp;
                    sm.egs[b][l] = -__expf(gv) * sig;
                    sm.egrs[b][l] = __expf(gt - gv) * inv;
                    if (l == 63) {
                        sm.rs[b] = fold ? sp : 1.0f;
                        sm.sig_fin[b] = fold ? 1.0f : sp;
                    }
                    sig = fold ? 1.0f : sp;
                    ell += (double)la_i;
                    if (cc == cnc - 1) {
                        // the unit's ell
#pragma unroll
                        for (int o = 32; o >= 1; o >>= 1) ell += __shfl_xor(ell, o);
                        if (l == 0) a.pool_ell[uni32(sm.units[cq].rec)] = (float)ell;
                        ell = 0.0;
                    }
                }
                lds_barrier();                                      // a -> b
                // ---- phase b: keys and values of chunk i + 1 land in the other buffers;
                //      gates of chunk i + 1 (read in phase b, so that their wait falls at
                //      its end); factors of block 0 of the P system
                if (i + 1 < steps) HYPIC_FETCH_G(step_desc(nxt));
                if (i < steps) prep_kt(sm, (int)(i & 1), 0, l);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // chunk i + 1 has landed
                __syncthreads();                                    // b -> next a
                cq = nxt.q;
                cc = nxt.c;
                cnc = nxt.nc;
                cursor_next(sm, nvalid, nxt);
            }
#undef HYPIC_LOAD_KV
        } else {
            // ---- waves 5-7: a Gram block in phase a (waves 5 and 7 the diagonal blocks,
            //      which they also start inverting; wave 6 H_21); in phase b waves 5 and 7
            //      finish their block's inverse, wave 6 turns K^T around for tokens 32-63.
            // Wave 7 writes block 2's S factor already scaled by the update factor:
            // e^{G - g_r} / sigma' times D T0 D^{-1} diag(beta), row r, is T0 diag(bs) with
            // bs_c = beta_c e^{G - g_c} / sigma', because e^{G - g_r} / sigma' e^{g_r} is the
            // same for every row; so Y_2 of the S columns comes out ready for the update, and
            // the S factor needs no exponential per entry.  It keeps its own copy of sigma
            // (the same recurrence, from the same gates, as wave 4's).
            int cc = nxt.c;                                         // chunk i's index in its unit
            float sig = 1.0f;
            cursor_next(sm, nvalid, nxt);                           // chunk 1
            __syncthreads();                                        // prologue: chunk 0 staged
            for (int i = 0; i <= steps; ++i) {
                int thv = th;
                asm volatile("" : "+v"(thv));
                const int l = thv & 63;
                if (i < steps) {
                    const int b = (int)(i & 1);
                    const float la_i = lar, b_i = br;
                    const float gv = wave_prefix_sum(la_i);
                    sm.pv[pw][0][l] = gv;
                    sm.pv[pw][1][l] = b_i;
                    if (pw == 3) {
                        if (cc == 0) sig = 1.0f;
                        const float gt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gv), 63));
                        const float sp = sig * __expf(gt);
                        const bool fold = sp < 0x1p-60f;
                        const float inv = fold ? 1.0f : 1.0f / sp;
                        sm.bsv[l] = b_i * (__expf(gt - gv) * inv);
                        sig = fold ? 1.0f : sp;
                    }
                    wave_lds_sync();
                    prep_gram(sm, b, pw, l);
                    if (pw != 2) {
                        wave_lds_sync();
                        prep_invert1<true>(inv_ctx(sm, b, pw >> 1, pw, pw == 3 ? &sm.bsv[32] : nullptr), l);
                    }
                }
                lds_barrier();                                      // a -> b
                if (i + 1 < steps) HYPIC_FETCH_G(step_desc(nxt));   // gates of chunk i + 1
                if (i < steps && pw != 2)
                    prep_invert2<true>(inv_ctx(sm, (int)(i & 1), pw >> 1, pw, pw == 3 ? &sm.bsv[32] : nullptr), l);
                if (i < steps && pw == 2) prep_kt(sm, (int)(i & 1), 1, l);
                __syncthreads();                                    // b -> next a
                cc = nxt.c;
                cursor_next(sm, nvalid, nxt);
            }
        }
#undef HYPIC_FETCH_G
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_build_mfma(const BuildArgs &a, hipStream_t stream, bool *taken) {
    *taken = false;
    if (a.family != HYPIC_GDN || a.kv_dtype != HYPIC_BF16 || a.dk != 128 || a.dv != 128) return hipSuccess;
    if (!aligned16(a.k) || !aligned16(a.v) || (a.k_st % 8) || (a.k_sh % 8) || (a.v_st % 8) || (a.v_sh % 8))
        return hipSuccess;
    if (a.num_slots * a.H > 0x7fffffffLL) return hipSuccess;   // record index kept in 32 bits
    *taken = true;
    const int64_t G = stream_grid((int64_t)a.num_segments * a.H, TMAX);
    hipLaunchKernelGGL(gdn_build_mfma_kernel, dim3((unsigned)G), dim3(NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace hypic
