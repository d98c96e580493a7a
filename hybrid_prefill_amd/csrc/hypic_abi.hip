// C ABI entry points of libhypic: synchronous argument validation, then one
// asynchronous launch on the caller's stream.  Validation touches no HIP API,
// so a bad call is rejected the same way with or without a GPU.
#include <string.h>

#include "hypic_internal.h"

namespace hypic {
hipError_t launch_build_ref(const BuildArgs &a, hipStream_t stream);
hipError_t launch_build_mfma(const BuildArgs &a, hipStream_t stream, bool *taken);
hipError_t launch_build_sd_mfma(const BuildArgs &a, hipStream_t stream, bool *taken);
hipError_t launch_build_kda(const BuildArgs &a, hipStream_t stream);
hipError_t launch_compose_ref(const ComposeArgs &a, hipStream_t stream);
hipError_t launch_compose_mfma(const ComposeArgs &a, hipStream_t stream, bool *taken);
hipError_t launch_compose_heads_mfma(const ComposeArgs &a, hipStream_t stream);
}  // namespace hypic

using namespace hypic;

namespace {

bool head_size_ok(int32_t d) { return d == 64 || d == 128; }
bool family_ok(int32_t f) { return f == HYPIC_SCALAR || f == HYPIC_DIAGONAL || f == HYPIC_GDN || f == HYPIC_KDA; }
bool has_P(int32_t f) { return f == HYPIC_GDN || f == HYPIC_KDA; }
bool dtype_ok(int32_t t) { return t == HYPIC_F32 || t == HYPIC_BF16; }

hypic_status check_pool(const hypic_pool *pool) {
    if (!pool) return HYPIC_ERR_INVALID_ARG;
    if (!family_ok(pool->family)) return HYPIC_ERR_UNSUPPORTED;
    if (pool->num_heads <= 0 || pool->num_slots < 0) return HYPIC_ERR_INVALID_ARG;
    if (!head_size_ok(pool->d_k) || !head_size_ok(pool->d_v)) return HYPIC_ERR_UNSUPPORTED;
    if (!pool->S || !pool->log_scale) return HYPIC_ERR_INVALID_ARG;
    if (has_P(pool->family) != (pool->P != nullptr)) return HYPIC_ERR_INVALID_ARG;
    return HYPIC_OK;
}

}  // namespace

extern "C" {

int32_t hypic_abi_version(void) { return HYPIC_ABI_VERSION; }

const char *hypic_status_string(int32_t s) {
    switch (s) {
    case HYPIC_OK: return "ok";
    case HYPIC_ERR_INVALID_ARG: return "invalid argument";
    case HYPIC_ERR_UNSUPPORTED: return "unsupported configuration";
    case HYPIC_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

hypic_status hypic_build_segment(const hypic_segments *in, const hypic_pool *pool,
                                 const int32_t *dst_slots, uint32_t *err_flag, void *stream) {
    if (!in) return HYPIC_ERR_INVALID_ARG;
    const hypic_status ps = check_pool(pool);
    if (ps != HYPIC_OK) return ps;
    if (!family_ok(in->family) || !dtype_ok(in->kv_dtype)) return HYPIC_ERR_UNSUPPORTED;
    if (in->family != pool->family || in->num_heads != pool->num_heads || in->d_k != pool->d_k ||
        in->d_v != pool->d_v)
        return HYPIC_ERR_INVALID_ARG;
    if (in->num_segments < 0 || in->num_tokens < 0) return HYPIC_ERR_INVALID_ARG;
    if (in->num_segments == 0) return HYPIC_OK;
    if (!in->seg_offsets || !dst_slots) return HYPIC_ERR_INVALID_ARG;
    if (in->num_tokens > 0 && (!in->k || !in->v)) return HYPIC_ERR_INVALID_ARG;
    if (in->k_stride_t < 0 || in->k_stride_h < 0 || in->v_stride_t < 0 || in->v_stride_h < 0 ||
        in->beta_stride_t < 0 || in->beta_stride_h < 0 || in->la_stride_t < 0 || in->la_stride_h < 0)
        return HYPIC_ERR_INVALID_ARG;
    if ((int64_t)in->num_segments * in->num_heads * 4 > 0x7fffffffLL) return HYPIC_ERR_UNSUPPORTED;

    BuildArgs a;
    memset(&a, 0, sizeof(a));
    a.family = in->family; a.H = in->num_heads; a.dk = in->d_k; a.dv = in->d_v;
    a.num_segments = in->num_segments; a.kv_dtype = in->kv_dtype; a.num_tokens = in->num_tokens;
    a.seg_offsets = in->seg_offsets;
    a.k = in->k; a.k_st = in->k_stride_t; a.k_sh = in->k_stride_h;
    a.v = in->v; a.v_st = in->v_stride_t; a.v_sh = in->v_stride_h;
    a.beta = in->beta; a.b_st = in->beta_stride_t; a.b_sh = in->beta_stride_h;
    a.log_alpha = in->log_alpha; a.la_st = in->la_stride_t; a.la_sh = in->la_stride_h;
    a.dst_slots = dst_slots; a.num_slots = pool->num_slots;
    a.pool_ell = pool->log_scale; a.pool_P = pool->P; a.pool_S = pool->S;
    a.err_flag = err_flag;

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (a.family == HYPIC_KDA) return launch_build_kda(a, st) == hipSuccess ? HYPIC_OK : HYPIC_ERR_HIP;
    bool taken = false;
    hipError_t e = launch_build_mfma(a, st, &taken);
    if (!taken) e = launch_build_sd_mfma(a, st, &taken);
    if (!taken) e = launch_build_ref(a, st);
    return e == hipSuccess ? HYPIC_OK : HYPIC_ERR_HIP;
}

hypic_status hypic_prefill_segment(const hypic_segments *in, const void *q, int64_t q_stride_t,
                                   int64_t q_stride_h, void *o, int64_t o_stride_t, int64_t o_stride_h,
                                   int32_t o_dtype, const hypic_pool *pool, const int32_t *dst_slots,
                                   uint32_t *err_flag, void *stream) {
    if (!in) return HYPIC_ERR_INVALID_ARG;
    if (!family_ok(in->family) || !dtype_ok(in->kv_dtype)) return HYPIC_ERR_UNSUPPORTED;
    if (in->family != HYPIC_GDN || in->kv_dtype != HYPIC_BF16 || in->d_k != 128 || in->d_v != 128)
        return HYPIC_ERR_UNSUPPORTED;
    if (in->num_heads <= 0 || in->num_segments < 0 || in->num_tokens < 0) return HYPIC_ERR_INVALID_ARG;
    if (!pool && !o) return HYPIC_ERR_INVALID_ARG;          // nothing asked for
    if (pool) {
        const hypic_status ps = check_pool(pool);
        if (ps != HYPIC_OK) return ps;
        if (pool->family != in->family || pool->num_heads != in->num_heads || pool->d_k != in->d_k ||
            pool->d_v != in->d_v)
            return HYPIC_ERR_INVALID_ARG;
    }
    if (o) {
        if (!dtype_ok(o_dtype)) return HYPIC_ERR_UNSUPPORTED;
        if (!q || q_stride_t < 0 || q_stride_h < 0 || o_stride_t < 0 || o_stride_h < 0) return HYPIC_ERR_INVALID_ARG;
    }
    if (in->num_segments == 0) return HYPIC_OK;
    if (!in->seg_offsets || (pool && !dst_slots)) return HYPIC_ERR_INVALID_ARG;
    if (in->num_tokens > 0 && (!in->k || !in->v)) return HYPIC_ERR_INVALID_ARG;
    if (in->k_stride_t < 0 || in->k_stride_h < 0 || in->v_stride_t < 0 || in->v_stride_h < 0 ||
        in->beta_stride_t < 0 || in->beta_stride_h < 0 || in->la_stride_t < 0 || in->la_stride_h < 0)
        return HYPIC_ERR_INVALID_ARG;
    if ((int64_t)in->num_segments * in->num_heads > 0x7fffffffLL) return HYPIC_ERR_UNSUPPORTED;

    BuildArgs a;
    memset(&a, 0, sizeof(a));
    a.family = in->family; a.H = in->num_heads; a.dk = in->d_k; a.dv = in->d_v;
    a.num_segments = in->num_segments; a.kv_dtype = in->kv_dtype; a.num_tokens = in->num_tokens;
    a.seg_offsets = in->seg_offsets;
    a.k = in->k; a.k_st = in->k_stride_t; a.k_sh = in->k_stride_h;
    a.v = in->v; a.v_st = in->v_stride_t; a.v_sh = in->v_stride_h;
    a.beta = in->beta; a.b_st = in->beta_stride_t; a.b_sh = in->beta_stride_h;
    a.log_alpha = in->log_alpha; a.la_st = in->la_stride_t; a.la_sh = in->la_stride_h;
    if (pool) {
        a.dst_slots = dst_slots; a.num_slots = pool->num_slots;
        a.pool_ell = pool->log_scale; a.pool_P = pool->P; a.pool_S = pool->S;
    }
    a.err_flag = err_flag;
    FwdIO io;
    memset(&io, 0, sizeof(io));
    io.q = q; io.q_st = q_stride_t; io.q_sh = q_stride_h;
    io.o = o; io.o_st = o_stride_t; io.o_sh = o_stride_h; io.o_bf16 = o_dtype == HYPIC_BF16;

    bool taken = false;
    const hipError_t e = launch_chunk_mfma(a, io, pool != nullptr, o != nullptr, static_cast<hipStream_t>(stream),
                                           &taken);
    if (!taken) return HYPIC_ERR_UNSUPPORTED;                 // unaligned rows or strides
    return e == hipSuccess ? HYPIC_OK : HYPIC_ERR_HIP;
}

hypic_status hypic_compose_chain(const hypic_pool *pool, int32_t num_requests,
                                 const int64_t *chain_offsets, const int32_t *chain_slots,
                                 int64_t num_chain_slots,
                                 const float *init_S, float *out_S, float *out_log_scale,
                                 float *out_P, uint32_t *err_flag, void *stream) {
    const hypic_status ps = check_pool(pool);
    if (ps != HYPIC_OK) return ps;
    if (num_requests < 0 || num_chain_slots < 0) return HYPIC_ERR_INVALID_ARG;
    if (num_requests == 0) return HYPIC_OK;
    if (!chain_offsets || !out_S) return HYPIC_ERR_INVALID_ARG;
    if (num_chain_slots > 0 && !chain_slots) return HYPIC_ERR_INVALID_ARG;
    if (out_P && !has_P(pool->family)) return HYPIC_ERR_INVALID_ARG;
    // the composed operator may be renormalised into ell: both or neither
    if (out_P && !out_log_scale) return HYPIC_ERR_INVALID_ARG;
    if ((int64_t)num_requests * pool->num_heads * 4 > 0x7fffffffLL) return HYPIC_ERR_UNSUPPORTED;

    ComposeArgs a;
    memset(&a, 0, sizeof(a));
    a.family = pool->family; a.H = pool->num_heads; a.dk = pool->d_k; a.dv = pool->d_v;
    a.num_requests = num_requests; a.num_slots = pool->num_slots; a.num_chain_slots = num_chain_slots;
    a.pool_ell = pool->log_scale; a.pool_P = pool->P; a.pool_S = pool->S;
    a.chain_offsets = chain_offsets; a.chain_slots = chain_slots;
    a.init_S = init_S; a.out_S = out_S; a.out_ell = out_log_scale; a.out_P = out_P;
    a.err_flag = err_flag;

    hipStream_t st = static_cast<hipStream_t>(stream);
    bool taken = false;
    hipError_t e = launch_compose_mfma(a, st, &taken);
    if (!taken) e = launch_compose_ref(a, st);
    return e == hipSuccess ? HYPIC_OK : HYPIC_ERR_HIP;
}

hypic_status hypic_compose_chain_heads(const hypic_pool *pool, int32_t num_requests,
                                       const int64_t *chain_offsets, const int32_t *chain_slots,
                                       int64_t num_chain_slots, const int64_t *head_offsets,
                                       int64_t num_head_tokens, const float *head_k, const float *head_v,
                                       const float *head_beta, const float *head_log_alpha,
                                       const float *init_S, float *out_S, float *out_log_scale,
                                       uint32_t *err_flag, void *stream) {
    const hypic_status ps = check_pool(pool);
    if (ps != HYPIC_OK) return ps;
    if (num_requests < 0 || num_chain_slots < 0 || num_head_tokens < 0) return HYPIC_ERR_INVALID_ARG;
    if (pool->family != HYPIC_GDN || pool->d_k != 128 || pool->d_v != 128) return HYPIC_ERR_UNSUPPORTED;
    if (num_head_tokens >= (1LL << 27)) return HYPIC_ERR_UNSUPPORTED;
    if (num_requests == 0) return HYPIC_OK;
    if (!chain_offsets || !out_S || !head_offsets) return HYPIC_ERR_INVALID_ARG;
    if (num_chain_slots > 0 && !chain_slots) return HYPIC_ERR_INVALID_ARG;
    if (num_head_tokens == 0) {       // no head tokens at all: the plain chain
        if (head_k || head_v || head_beta || head_log_alpha) return HYPIC_ERR_INVALID_ARG;
        return hypic_compose_chain(pool, num_requests, chain_offsets, chain_slots, num_chain_slots, init_S,
                                   out_S, out_log_scale, nullptr, err_flag, stream);
    }
    if (!head_k || !head_v || !head_beta || !head_log_alpha) return HYPIC_ERR_INVALID_ARG;
    if ((int64_t)num_requests * pool->num_heads > 0x7fffffffLL) return HYPIC_ERR_UNSUPPORTED;

    ComposeArgs a;
    memset(&a, 0, sizeof(a));
    a.family = pool->family; a.H = pool->num_heads; a.dk = pool->d_k; a.dv = pool->d_v;
    a.num_requests = num_requests; a.num_slots = pool->num_slots; a.num_chain_slots = num_chain_slots;
    a.pool_ell = pool->log_scale; a.pool_P = pool->P; a.pool_S = pool->S;
    a.chain_offsets = chain_offsets; a.chain_slots = chain_slots;
    a.init_S = init_S; a.out_S = out_S; a.out_ell = out_log_scale;
    a.err_flag = err_flag;
    a.head_offsets = head_offsets; a.num_head_tokens = num_head_tokens;
    a.head_k = head_k; a.head_v = head_v; a.head_beta = head_beta; a.head_la = head_log_alpha;
    const hipError_t e = launch_compose_heads_mfma(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HYPIC_OK : HYPIC_ERR_HIP;
}

hypic_status hypic_conv_warmup(int32_t num_boundaries, int32_t channels, int32_t kernel_size,
                               int32_t x_dtype,
                               const void *tails, int64_t num_tails, const int32_t *tail_index,
                               const void *heads, int64_t num_heads, const int32_t *head_index,
                               const float *weight, const float *bias, int32_t activation,
                               float *out, uint32_t *err_flag, void *stream) {
    if (num_boundaries < 0 || channels <= 0 || num_tails < 0 || num_heads < 0) return HYPIC_ERR_INVALID_ARG;
    if (kernel_size < 2 || kernel_size > 8 || !dtype_ok(x_dtype)) return HYPIC_ERR_UNSUPPORTED;
    if (activation != 0 && activation != 1) return HYPIC_ERR_UNSUPPORTED;
    if (num_boundaries == 0) return HYPIC_OK;
    if (!tails || !heads || !weight || !out) return HYPIC_ERR_INVALID_ARG;
    if (!tail_index && num_tails < num_boundaries) return HYPIC_ERR_INVALID_ARG;
    if (!head_index && num_heads < num_boundaries) return HYPIC_ERR_INVALID_ARG;

    ConvArgs a;
    memset(&a, 0, sizeof(a));
    a.num_boundaries = num_boundaries; a.channels = channels; a.ksize = kernel_size;
    a.x_dtype = x_dtype; a.activation = activation;
    a.tails = tails; a.num_tails = num_tails; a.tail_index = tail_index;
    a.heads = heads; a.num_heads = num_heads; a.head_index = head_index;
    a.weight = weight; a.bias = bias; a.out = out; a.err_flag = err_flag;
    const hipError_t e = launch_conv_warmup(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HYPIC_OK : HYPIC_ERR_HIP;
}

hypic_status hypic_conv_kv(int32_t num_tokens, int32_t num_heads, int32_t d_k, int32_t d_v, int32_t kernel_size,
                           int32_t x_dtype, const void *x, int64_t num_rows, const int32_t *window,
                           const float *weight, const float *bias, int32_t activation, int32_t normalize_k,
                           int32_t out_dtype, void *k_out, void *v_out,
                           const int32_t *src_token, int64_t num_src_tokens, const float *beta,
                           const float *log_alpha, float *beta_out, float *la_out,
                           uint32_t *err_flag, void *stream) {
    if (num_tokens < 0 || num_heads <= 0 || d_k <= 0 || d_v <= 0 || num_rows < 0 || num_src_tokens < 0)
        return HYPIC_ERR_INVALID_ARG;
    if (kernel_size < 1 || kernel_size > 8 || !dtype_ok(x_dtype) || !dtype_ok(out_dtype))
        return HYPIC_ERR_UNSUPPORTED;
    if (activation != 0 && activation != 1) return HYPIC_ERR_UNSUPPORTED;
    if ((int64_t)num_heads * (d_k + d_v) > 16384) return HYPIC_ERR_UNSUPPORTED;   // LDS row of the conv
    if (num_tokens == 0) return HYPIC_OK;
    if (!x || !window || !weight || !k_out || !v_out) return HYPIC_ERR_INVALID_ARG;
    if (src_token && (!beta_out || !la_out)) return HYPIC_ERR_INVALID_ARG;

    ConvKvArgs a;
    memset(&a, 0, sizeof(a));
    a.num_tokens = num_tokens; a.H = num_heads; a.dk = d_k; a.dv = d_v; a.ksize = kernel_size;
    a.x_dtype = x_dtype; a.activation = activation; a.normalize_k = normalize_k != 0; a.out_dtype = out_dtype;
    a.x = x; a.num_rows = num_rows; a.window = window; a.weight = weight; a.bias = bias;
    a.k_out = k_out; a.v_out = v_out;
    a.src_token = src_token; a.num_src_tokens = num_src_tokens; a.beta = beta; a.log_alpha = log_alpha;
    a.beta_out = beta_out; a.la_out = la_out; a.err_flag = err_flag;
    const hipError_t e = launch_conv_kv(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? HYPIC_OK : HYPIC_ERR_HIP;
}

}  // extern "C"
