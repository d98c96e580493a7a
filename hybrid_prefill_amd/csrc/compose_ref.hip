// Composition of pool records along request chains, fp32 LDS-tiled kernel.
//
// What it computes (besthub article "Cut First-Token Latency by 3.25x ...",
// paragraph 4: reuse composes T_C2*S(C1)+S(C2); podcast companion page,
// "Composition law, step by step"): for every request r and head h, over the
// chain's slots in prompt order
//     S <- e^{ell_i} (P_i S) + S_i           (GDN; T_i = e^{ell_i} P_i)
//     S <- e^{ell_i} S + S_i                 (scalar)
//     S <- diag(e^{ell_i}) S + S_i           (diagonal)
// and optionally the composed operator ell <- ell + ell_i, P <- P_i P.
//
// GDN work split: one workgroup per (request, head, 64-column slab of S).  The
// slab stays in LDS across the chain; P_i streams through LDS in 32-column blocks.
// The composed P runs in a launch of its own, one workgroup per (request, head)
// holding the whole product, so that it can be renormalised as a whole.  Scalar and diagonal
// families: 1024 state elements per workgroup, four per thread in registers (or,
// for unaligned buffers, one workgroup per (request, head)).
#include "hypic_internal.h"

namespace hypic {
namespace {

constexpr int NT = 256;
constexpr int NSL = 64;
constexpr int KB = 32;

// Check a request's chain; returns 0 ok, 1 slot out of range, 2 bad offsets.
__device__ int check_chain(const ComposeArgs &a, int r, int64_t &c_lo, int64_t &c_hi, int *sh_bad) {
    if (threadIdx.x == 0) {
        const int64_t lo = a.chain_offsets[r], hi = a.chain_offsets[r + 1];
        *sh_bad = (lo < 0 || hi < lo || hi > a.num_chain_slots) ? 2 : 0;
    }
    __syncthreads();
    c_lo = a.chain_offsets[r];
    c_hi = a.chain_offsets[r + 1];
    if (*sh_bad) return *sh_bad;
    __syncthreads();
    for (int64_t c = c_lo + threadIdx.x; c < c_hi; c += blockDim.x) {
        const int32_t s = a.chain_slots[c];
        if (s < 0 || s >= a.num_slots) *sh_bad = 1;   // benign race: every writer stores 1
    }
    __syncthreads();
    return *sh_bad;
}

template <int DK, int DV>
__global__ __launch_bounds__(NT) void compose_dense_ref_kernel(ComposeArgs a) {
    __shared__ float St[DK][NSL + 1];
    __shared__ float Pt[DK][KB + 1];
    __shared__ int sh_bad;

    const int tid = threadIdx.x;
    constexpr int nslab = DV / NSL;
    const int slab = blockIdx.x % nslab;
    const int unit = blockIdx.x / nslab;
    const int h = unit % a.H;
    const int r = unit / a.H;
    const int c0 = slab * NSL;
    constexpr int ldo = DV;
    float *out = a.out_S + ((int64_t)r * a.H + h) * DK * DV;

    int64_t lo, hi;
    const int bad = check_chain(a, r, lo, hi, &sh_bad);
    if (bad) {
        if (tid == 0 && slab == 0)
            raise_flag(a.err_flag, bad == 1 ? HYPIC_EFLAG_SLOT_OUT_OF_RANGE : HYPIC_EFLAG_BAD_OFFSETS);
        const float nanv = __int_as_float(0x7fc00000);
        for (int e = tid; e < DK * NSL; e += NT) out[(int64_t)(e / NSL) * ldo + c0 + e % NSL] = nanv;
        if (slab == 0 && a.out_ell && tid == 0) a.out_ell[(int64_t)r * a.H + h] = nanv;
        return;
    }

    for (int e = tid; e < DK * NSL; e += NT) {
        const int i = e / NSL, c = e % NSL;
        St[i][c] = a.init_S ? a.init_S[((int64_t)r * a.H + h) * DK * DV + (int64_t)i * DV + c0 + c] : 0.0f;
    }
    double ell = 0.0;
    const int tr = tid / 16, tc = tid % 16;
    constexpr int RP = DK / 16;

    for (int64_t ci = lo; ci < hi; ++ci) {
        const int64_t rec = (int64_t)a.chain_slots[ci] * a.H + h;
        const float *Pi = a.pool_P + rec * DK * DK;
        const float le = a.pool_ell[rec];
        ell += (double)le;
        const float sc = expf(le);
        float acc[RP][4];
#pragma unroll
        for (int p = 0; p < RP; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[p][q] = 0.f;
        for (int kb = 0; kb < DK; kb += KB) {
            __syncthreads();
            for (int e = tid; e < DK * KB; e += NT) {
                const int i = e / KB, k = e % KB;
                Pt[i][k] = Pi[(int64_t)i * DK + kb + k];
            }
            __syncthreads();
            for (int k = 0; k < KB; ++k) {
                float pv[RP], sv[4];
#pragma unroll
                for (int p = 0; p < RP; ++p) pv[p] = Pt[tr + 16 * p][k];
#pragma unroll
                for (int q = 0; q < 4; ++q) sv[q] = St[kb + k][tc + 16 * q];
#pragma unroll
                for (int p = 0; p < RP; ++p)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[p][q] += pv[p] * sv[q];
            }
        }
        __syncthreads();   // everyone is done reading the old slab
        const float *Si = a.pool_S + rec * DK * DV;
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            const int i = tr + 16 * p;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = tc + 16 * q;
                St[i][c] = sc * acc[p][q] + Si[(int64_t)i * DV + c0 + c];
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < DK * NSL; e += NT) {
        const int i = e / NSL, c = e % NSL;
        out[(int64_t)i * ldo + c0 + c] = St[i][c];
    }
    if (slab == 0 && a.out_ell && tid == 0) a.out_ell[(int64_t)r * a.H + h] = (float)ell;
}

// The composed operator of a GDN / KDA chain, P <- P_i P from P = I, one workgroup
// per (request, head) holding the whole product in LDS.  A product of contracting
// records drifts toward the fp32 subnormals (a GDN record's P shrinks by about
// e^-4 per 2048 tokens at unit keys and beta = sigmoid(N(0,1))), so whenever the
// largest |entry| falls below 2^-32 the product is scaled back to [1, 2) by a power
// of two, which is exact, and the exponent goes into ell: (out_ell, out_P) stays a
// record of the chain, T = e^ell P.  Runs after the state launch, which has raised
// the error flag and written ell for bad chains; here only P is NaN-filled.
template <int DK>
__global__ __launch_bounds__(NT) void compose_P_ref_kernel(ComposeArgs a) {
    __shared__ float Xs[DK][DK + 1];
    __shared__ float Pt[DK][KB + 1];
    __shared__ float red[NT / 64];
    __shared__ int sh_bad;

    const int tid = threadIdx.x;
    const int h = blockIdx.x % a.H;
    const int r = blockIdx.x / a.H;
    float *out = a.out_P + ((int64_t)r * a.H + h) * DK * DK;
    int64_t lo, hi;
    if (check_chain(a, r, lo, hi, &sh_bad)) {
        const float nanv = __int_as_float(0x7fc00000);
        for (int e = tid; e < DK * DK; e += NT) out[e] = nanv;
        return;
    }
    for (int e = tid; e < DK * DK; e += NT) Xs[e / DK][e % DK] = (e / DK == e % DK) ? 1.0f : 0.0f;
    double ell = 0.0;
    int pexp = 0;                       // the product is 2^pexp Xs
    // thread (tr, tc) owns rows tr + 16 p and columns tc + 16 q of the product
    constexpr int RP = DK / 16;
    const int tr = tid / 16, tc = tid % 16;
    for (int64_t ci = lo; ci < hi; ++ci) {
        const int64_t rec = (int64_t)a.chain_slots[ci] * a.H + h;
        const float *Pi = a.pool_P + rec * DK * DK;
        ell += (double)a.pool_ell[rec];
        float acc[RP][RP];
#pragma unroll
        for (int p = 0; p < RP; ++p)
#pragma unroll
            for (int q = 0; q < RP; ++q) acc[p][q] = 0.f;
        for (int kb = 0; kb < DK; kb += KB) {
            __syncthreads();
            for (int e = tid; e < DK * KB; e += NT) {
                const int i = e / KB, k = e % KB;
                Pt[i][k] = Pi[(int64_t)i * DK + kb + k];
            }
            __syncthreads();
            for (int k = 0; k < KB; ++k) {
                float pv[RP], xv[RP];
#pragma unroll
                for (int p = 0; p < RP; ++p) pv[p] = Pt[tr + 16 * p][k];
#pragma unroll
                for (int q = 0; q < RP; ++q) xv[q] = Xs[kb + k][tc + 16 * q];
#pragma unroll
                for (int p = 0; p < RP; ++p)
#pragma unroll
                    for (int q = 0; q < RP; ++q) acc[p][q] += pv[p] * xv[q];
            }
        }
        __syncthreads();    // every read of the old product is done
        float m = 0.f;
#pragma unroll
        for (int p = 0; p < RP; ++p)
#pragma unroll
            for (int q = 0; q < RP; ++q) {
                Xs[tr + 16 * p][tc + 16 * q] = acc[p][q];
                m = fmaxf(m, fabsf(acc[p][q]));
            }
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        if ((tid & 63) == 0) red[tid >> 6] = m;
        __syncthreads();
        float mx = 0.f;
#pragma unroll
        for (int wv = 0; wv < NT / 64; ++wv) mx = fmaxf(mx, red[wv]);
        if (mx < 0x1p-32f && mx > 0.f) {
            const int sft = -ilogbf(mx);
#pragma unroll
            for (int p = 0; p < RP; ++p)
#pragma unroll
                for (int q = 0; q < RP; ++q)
                    Xs[tr + 16 * p][tc + 16 * q] = ldexpf(Xs[tr + 16 * p][tc + 16 * q], sft);
            pexp -= sft;
        }
    }
    __syncthreads();
    for (int e = tid; e < DK * DK; e += NT) out[e] = Xs[e / DK][e % DK];
    if (a.out_ell && tid == 0) a.out_ell[(int64_t)r * a.H + h] = (float)(ell + (double)pexp * 0.69314718055994530942);
}

// Scalar / diagonal: elementwise, one workgroup per (request, head).
template <int FAM, int DK, int DV>
__global__ __launch_bounds__(NT) void compose_sd_kernel(ComposeArgs a) {
    constexpr int PER = DK * DV / NT;
    __shared__ int sh_bad;
    const int tid = threadIdx.x;
    const int h = blockIdx.x % a.H;
    const int r = blockIdx.x / a.H;
    const int64_t orec = (int64_t)r * a.H + h;
    float *out = a.out_S + orec * DK * DV;
    int64_t lo, hi;
    const int bad = check_chain(a, r, lo, hi, &sh_bad);
    if (bad) {
        if (tid == 0) raise_flag(a.err_flag, bad == 1 ? HYPIC_EFLAG_SLOT_OUT_OF_RANGE : HYPIC_EFLAG_BAD_OFFSETS);
        const float nanv = __int_as_float(0x7fc00000);
        for (int e = tid; e < DK * DV; e += NT) out[e] = nanv;
        if (a.out_ell) {
            if (FAM == HYPIC_DIAGONAL) { if (tid < DK) a.out_ell[orec * DK + tid] = nanv; }
            else if (tid == 0) a.out_ell[orec] = nanv;
        }
        return;
    }
    float s[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) s[q] = a.init_S ? a.init_S[orec * DK * DV + tid + q * NT] : 0.0f;
    double ell = 0.0;   // thread i < DK keeps channel i (diagonal), thread 0 the scalar
    for (int64_t ci = lo; ci < hi; ++ci) {
        const int64_t rec = (int64_t)a.chain_slots[ci] * a.H + h;
        const float *Si = a.pool_S + rec * DK * DV;
        if (FAM == HYPIC_DIAGONAL) {
            const float *le = a.pool_ell + rec * DK;
            if (tid < DK) ell += (double)le[tid];
#pragma unroll
            for (int q = 0; q < PER; ++q) {
                const int e = tid + q * NT;
                s[q] = expf(le[e / DV]) * s[q] + Si[e];
            }
        } else {
            const float le = a.pool_ell[rec];
            ell += (double)le;
            const float sc = expf(le);
#pragma unroll
            for (int q = 0; q < PER; ++q) s[q] = sc * s[q] + Si[tid + q * NT];
        }
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) out[tid + q * NT] = s[q];
    if (a.out_ell) {
        if (FAM == HYPIC_DIAGONAL) { if (tid < DK) a.out_ell[orec * DK + tid] = (float)ell; }
        else if (tid == 0) a.out_ell[orec] = (float)ell;
    }
}

// Scalar / diagonal, wide: the fold is elementwise, so the record is spread over
// DK DV / 1024 workgroups per (request, head) and each thread keeps four consecutive
// elements of one row (16-byte loads and stores).  The chain is folded eight steps at
// a time: the eight slots (wave-uniform), then every step's gate and S_i piece are
// loaded before the first is used, so one batch costs about two load latencies
// instead of eight dependent round trips.
constexpr int WE = 4 * NT;               // elements per workgroup
constexpr int CB = 8;                    // chain steps per batch
template <int FAM, int DK, int DV>
__global__ __launch_bounds__(NT) void compose_sd_wide_kernel(ComposeArgs a) {
    constexpr int NBLK = DK * DV / WE;
    __shared__ int sh_bad;
    const int tid = threadIdx.x;
    const int blk = blockIdx.x % NBLK;
    const int unit = blockIdx.x / NBLK;
    const int h = unit % a.H;
    const int r = unit / a.H;
    const int64_t orec = (int64_t)r * a.H + h;
    const int e0 = blk * WE + 4 * tid;       // first of this thread's four elements
    const int row = e0 / DV;                 // DV % 4 == 0: the four share a row
    const bool row_lead = (e0 % DV) == 0;
    float *out = a.out_S + orec * DK * DV + e0;
    int64_t lo, hi;
    const int bad = check_chain(a, r, lo, hi, &sh_bad);
    if (bad) {
        if (blk == 0 && tid == 0) raise_flag(a.err_flag, bad == 1 ? HYPIC_EFLAG_SLOT_OUT_OF_RANGE : HYPIC_EFLAG_BAD_OFFSETS);
        const float nanv = __int_as_float(0x7fc00000);
        *reinterpret_cast<float4 *>(out) = make_float4(nanv, nanv, nanv, nanv);
        if (a.out_ell) {
            if (FAM == HYPIC_DIAGONAL) { if (row_lead) a.out_ell[orec * DK + row] = nanv; }
            else if (blk == 0 && tid == 0) a.out_ell[orec] = nanv;
        }
        return;
    }
    float4 s = a.init_S ? *reinterpret_cast<const float4 *>(a.init_S + orec * DK * DV + e0)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    double ell = 0.0;
    for (int64_t base = lo; base < hi; base += CB) {
        const int nb = hi - base < CB ? (int)(hi - base) : CB;
        int64_t rec[CB];
#pragma unroll
        for (int k = 0; k < CB; ++k) rec[k] = (int64_t)a.chain_slots[k < nb ? base + k : base] * a.H + h;
        float4 si[CB];
        float le[CB];
#pragma unroll
        for (int k = 0; k < CB; ++k) {
            si[k] = *reinterpret_cast<const float4 *>(a.pool_S + rec[k] * DK * DV + e0);
            le[k] = FAM == HYPIC_DIAGONAL ? a.pool_ell[rec[k] * DK + row] : a.pool_ell[rec[k]];
        }
#pragma unroll
        for (int k = 0; k < CB; ++k) {
            if (k < nb) {
                const float sc = expf(le[k]);
                s.x = sc * s.x + si[k].x;
                s.y = sc * s.y + si[k].y;
                s.z = sc * s.z + si[k].z;
                s.w = sc * s.w + si[k].w;
                ell += (double)le[k];
            }
        }
    }
    *reinterpret_cast<float4 *>(out) = s;
    if (a.out_ell) {
        if (FAM == HYPIC_DIAGONAL) { if (row_lead) a.out_ell[orec * DK + row] = (float)ell; }
        else if (blk == 0 && tid == 0) a.out_ell[orec] = (float)ell;
    }
}

__host__ bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

template <int DK, int DV>
hipError_t launch_dims(const ComposeArgs &a, hipStream_t stream) {
    const int64_t units = (int64_t)a.num_requests * a.H;
    if (a.family == HYPIC_GDN || a.family == HYPIC_KDA) {      // (KDA: ell = 0, P = T_C)
        hipLaunchKernelGGL((compose_dense_ref_kernel<DK, DV>), dim3((unsigned)(units * (DV / NSL))), dim3(NT), 0, stream, a);
        if (a.out_P) hipLaunchKernelGGL((compose_P_ref_kernel<DK>), dim3((unsigned)units), dim3(NT), 0, stream, a);
    } else if (aligned16(a.pool_S) && aligned16(a.out_S) && (!a.init_S || aligned16(a.init_S))) {
        const dim3 grid((unsigned)(units * (DK * DV / WE)));
        if (a.family == HYPIC_SCALAR)
            hipLaunchKernelGGL((compose_sd_wide_kernel<HYPIC_SCALAR, DK, DV>), grid, dim3(NT), 0, stream, a);
        else
            hipLaunchKernelGGL((compose_sd_wide_kernel<HYPIC_DIAGONAL, DK, DV>), grid, dim3(NT), 0, stream, a);
    } else if (a.family == HYPIC_SCALAR) {
        hipLaunchKernelGGL((compose_sd_kernel<HYPIC_SCALAR, DK, DV>), dim3((unsigned)units), dim3(NT), 0, stream, a);
    } else {
        hipLaunchKernelGGL((compose_sd_kernel<HYPIC_DIAGONAL, DK, DV>), dim3((unsigned)units), dim3(NT), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_compose_ref(const ComposeArgs &a, hipStream_t stream) {
    if (a.dk == 64 && a.dv == 64) return launch_dims<64, 64>(a, stream);
    if (a.dk == 64 && a.dv == 128) return launch_dims<64, 128>(a, stream);
    if (a.dk == 128 && a.dv == 64) return launch_dims<128, 64>(a, stream);
    return launch_dims<128, 128>(a, stream);
}

}  // namespace hypic
