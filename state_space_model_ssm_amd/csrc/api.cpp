// C ABI of the gfx950 Mamba-2 SSM core: argument validation, dispatch to the
// HIP kernels on the caller's stream, and the host-side slot allocator.
// Nothing here allocates device memory, synchronises or memsets.
#include "../../include/mamba2.h"
#include "../../include/mamba1.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <new>
#include <cstdio>
#include <string>
#include <vector>

#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return MAMBA2_OK;
}

bool valid_dtype(int d) { return d == MAMBA2_F32 || d == MAMBA2_BF16; }
size_t dtype_bytes(int d) { return d == MAMBA2_BF16 ? 2 : 4; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dims_basic(const mamba2_dims *d) {
    if (!d) return fail(MAMBA2_ERR_INVALID_ARG, "dims is NULL");
    if (d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0 || d->conv_width <= 0 ||
        d->chunk_size <= 0)
        return fail(MAMBA2_ERR_INVALID_ARG, "dims must be positive (H=%d P=%d N=%d G=%d W=%d Q=%d)", d->nheads,
                    d->headdim, d->dstate, d->ngroups, d->conv_width, d->chunk_size);
    if (d->nheads % d->ngroups != 0)
        return fail(MAMBA2_ERR_INVALID_ARG, "nheads (%d) must be a multiple of ngroups (%d)", d->nheads, d->ngroups);
    if (!valid_dtype(d->act_dtype) || !valid_dtype(d->xbc_dtype) || !valid_dtype(d->state_dtype) ||
        !valid_dtype(d->out_dtype))
        return fail(MAMBA2_ERR_INVALID_ARG, "unknown dtype code");
    return MAMBA2_OK;
}

m2::LayerShape shape_of(const mamba2_dims *d) {
    m2::LayerShape s;
    s.H = d->nheads; s.P = d->headdim; s.N = d->dstate; s.G = d->ngroups; s.W = d->conv_width; s.Q = d->chunk_size;
    s.act_dt = d->act_dtype; s.xbc_dt = d->xbc_dtype; s.state_dt = d->state_dtype; s.out_dt = d->out_dtype;
    return s;
}

int check_conv(const mamba2_dims *d) {
    int st = check_dims_basic(d);
    if (st) return st;
    if (!m2::conv_supported(shape_of(d)))
        return fail(MAMBA2_ERR_UNSUPPORTED, "conv1d supports conv_width 2..4 and Cdim %% 8 == 0 (W=%d, Cdim=%lld)",
                    d->conv_width, (long long)shape_of(d).cdim());
    return MAMBA2_OK;
}

int check_state_update(const mamba2_dims *d) {
    int st = check_dims_basic(d);
    if (st) return st;
    const m2::LayerShape s = shape_of(d);
    if (!m2::state_update_supported(s) || s.cdim() % 8 != 0 || s.P % 4 != 0)
        return fail(MAMBA2_ERR_UNSUPPORTED, "state update supports dstate in {16, 64, 128}, headdim %% 4 == 0 (N=%d)",
                    d->dstate);
    // (the update kernels address a token's row and a head's state tile by 32-bit byte offsets)
    if (s.cdim() > (1 << 24) || (int64_t)s.P * s.N > (1 << 24))
        return fail(MAMBA2_ERR_UNSUPPORTED, "state update supports Cdim and headdim * dstate up to 2^24 (Cdim=%lld)",
                    (long long)s.cdim());
    return MAMBA2_OK;
}

int check_scan(const mamba2_dims *d) {
    int st = check_dims_basic(d);
    if (st) return st;
    if (!m2::scan_supported(shape_of(d)))
        return fail(MAMBA2_ERR_UNSUPPORTED,
                    "chunk scan supports (headdim, dstate, chunk) in {(16,16,16|32|64), (64,128,64|128)}; got (%d,%d,%d)",
                    d->headdim, d->dstate, d->chunk_size);
    return MAMBA2_OK;
}

#define REQUIRE_PTR(p) \
    do { if (!(p)) return fail(MAMBA2_ERR_INVALID_ARG, "%s is NULL", #p); \
         if (!aligned16(p)) return fail(MAMBA2_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); } while (0)
#define OPT_PTR(p) \
    do { if ((p) && !aligned16(p)) return fail(MAMBA2_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); } while (0)
#define REQUIRE_IDX(p) \
    do { if (!(p)) return fail(MAMBA2_ERR_INVALID_ARG, "%s is NULL", #p); \
         if (reinterpret_cast<uintptr_t>(p) & 3u) return fail(MAMBA2_ERR_INVALID_ARG, "%s is not 4-byte aligned", #p); } while (0)

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MAMBA2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// The device word (current device) in which kernels count the pool indices >= num_slots
// that they skip; looked up right before a launch.
int slot_word(unsigned **err) {
    const hipError_t e = m2::slot_error_word(err);
    if (e != hipSuccess) return fail(MAMBA2_ERR_HIP, "slot error word: %s", hipGetErrorString(e));
    return MAMBA2_OK;
}

#define SLOT_WORD(err)             \
    unsigned *err = nullptr;       \
    do {                           \
        int st_ = slot_word(&err); \
        if (st_) return st_;       \
    } while (0)

}  // namespace

extern "C" {

int mamba2_check_dims(const mamba2_dims *d) {
    int st = check_conv(d);
    if (st) return st;
    st = check_state_update(d);
    if (st) return st;
    st = check_scan(d);
    if (st) return st;
    return ok();
}

size_t mamba2_ssm_slot_bytes(const mamba2_dims *d) {
    if (check_dims_basic(d)) return 0;
    return (size_t)d->nheads * d->headdim * d->dstate * dtype_bytes(d->state_dtype);
}

size_t mamba2_conv_slot_bytes(const mamba2_dims *d) {
    if (check_dims_basic(d)) return 0;
    return (size_t)(d->conv_width - 1) * (size_t)shape_of(d).cdim() * dtype_bytes(d->state_dtype);
}

int mamba2_chunk_scan_workspace_bytes(const mamba2_dims *d, int64_t total_tokens, int32_t nseq, size_t *bytes) {
    int st = check_scan(d);
    if (st) return st;
    if (!bytes) return fail(MAMBA2_ERR_INVALID_ARG, "bytes is NULL");
    if (total_tokens < 0 || nseq < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative size");
    const m2::LayerShape s = shape_of(d);
    *bytes = m2::chunk_scan_blocks_supported(s) ? (size_t)m2::fused_workspace_bytes(s, total_tokens) : 0;
    return ok();
}

int mamba2_conv1d_fwd(const mamba2_dims *d, const void *xbc, const float *conv_w, const float *conv_b, void *xbc_out,
                      void *conv_pool, int32_t num_slots, const int32_t *cu_seqlens, int32_t nseq,
                      int64_t total_tokens, const int32_t *state_indices, const uint8_t *has_initial_state,
                      void *stream) {
    int st = check_conv(d);
    if (st) return st;
    if (num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be >= 0 (got %d)", num_slots);
    if (nseq < 0 || total_tokens < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative nseq or total_tokens");
    if (total_tokens > INT32_MAX)  // (cu_seqlens are int32)
        return fail(MAMBA2_ERR_INVALID_ARG, "total_tokens %lld beyond the int32 range of cu_seqlens", (long long)total_tokens);
    if (nseq == 0) {
        if (total_tokens != 0) return fail(MAMBA2_ERR_INVALID_ARG, "tokens without sequences");
        return ok();
    }
    REQUIRE_PTR(conv_w); OPT_PTR(conv_b); REQUIRE_PTR(conv_pool);
    REQUIRE_IDX(cu_seqlens); REQUIRE_IDX(state_indices);
    if (total_tokens > 0) { REQUIRE_PTR(xbc); REQUIRE_PTR(xbc_out); }
    if (xbc && xbc == xbc_out) return fail(MAMBA2_ERR_INVALID_ARG, "xbc_out must not alias xbc");
    SLOT_WORD(err);
    m2::ConvFwdArgs a{xbc, conv_w, conv_b, xbc_out, conv_pool, cu_seqlens, state_indices, has_initial_state, nseq,
                      total_tokens, num_slots, err};
    return hip_status(m2::launch_conv_fwd(shape_of(d), a, static_cast<hipStream_t>(stream)), "conv1d_fwd launch");
}

int mamba2_conv1d_update(const mamba2_dims *d, const void *xbc, const float *conv_w, const float *conv_b,
                         void *xbc_out, void *conv_pool, int32_t num_slots, const int32_t *state_indices,
                         int32_t batch, void *stream) {
    int st = check_conv(d);
    if (st) return st;
    if (num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be >= 0 (got %d)", num_slots);
    if (batch < 0) return fail(MAMBA2_ERR_INVALID_ARG, "batch < 0");
    if (batch == 0) return ok();
    REQUIRE_PTR(xbc); REQUIRE_PTR(conv_w); OPT_PTR(conv_b); REQUIRE_PTR(xbc_out); REQUIRE_PTR(conv_pool);
    REQUIRE_IDX(state_indices);
    if (xbc == xbc_out) return fail(MAMBA2_ERR_INVALID_ARG, "xbc_out must not alias xbc");
    SLOT_WORD(err);
    m2::ConvUpdateArgs a{xbc, conv_w, conv_b, xbc_out, conv_pool, state_indices, batch, num_slots, err};
    return hip_status(m2::launch_conv_update(shape_of(d), a, static_cast<hipStream_t>(stream)), "conv1d_update launch");
}

int mamba2_chunk_scan_fwd(const mamba2_dims *d, const void *xbc, const void *dt_raw, const float *A_log,
                          const float *dt_bias, const float *D, const void *z, void *y, void *ssm_pool,
                          int32_t num_slots, const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens,
                          const int32_t *state_indices, const uint8_t *has_initial_state, void *workspace,
                          size_t workspace_bytes, void *stream) {
    int st = check_scan(d);
    if (st) return st;
    if (num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be >= 0 (got %d)", num_slots);
    if (nseq < 0 || total_tokens < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative nseq or total_tokens");
    if (total_tokens > INT32_MAX)  // (cu_seqlens are int32)
        return fail(MAMBA2_ERR_INVALID_ARG, "total_tokens %lld beyond the int32 range of cu_seqlens", (long long)total_tokens);
    if (nseq == 0) {
        if (total_tokens != 0) return fail(MAMBA2_ERR_INVALID_ARG, "tokens without sequences");
        return ok();
    }
    REQUIRE_PTR(A_log); REQUIRE_PTR(dt_bias); REQUIRE_PTR(D); REQUIRE_PTR(ssm_pool);
    REQUIRE_IDX(cu_seqlens); REQUIRE_IDX(state_indices);
    if (total_tokens > 0) { REQUIRE_PTR(xbc); REQUIRE_PTR(dt_raw); REQUIRE_PTR(y); OPT_PTR(z); }
    const m2::LayerShape s = shape_of(d);
    if (workspace && total_tokens > 0 && m2::chunk_scan_blocks_supported(s)) {
        // 32-token blocks with B/C operand planes in the workspace; without one, the chunk kernel
        const size_t need = (size_t)m2::fused_workspace_bytes(s, total_tokens);
        if (workspace_bytes < need)
            return fail(MAMBA2_ERR_WORKSPACE, "chunk scan needs %zu workspace bytes, got %zu", need, workspace_bytes);
        OPT_PTR(workspace);
        if (workspace == xbc || workspace == y) return fail(MAMBA2_ERR_INVALID_ARG, "xbc, y and workspace must not alias");
        SLOT_WORD(err);
        m2::FusedArgs fa{xbc, nullptr, nullptr, nullptr, dt_raw, A_log, dt_bias, D, z, y, ssm_pool, cu_seqlens,
                         state_indices, has_initial_state, nseq, total_tokens, nullptr, nullptr, nullptr};
        fa.num_slots = num_slots;
        fa.err = err;
        return hip_status(m2::launch_block_scan(s, fa, workspace, static_cast<hipStream_t>(stream)),
                          "chunk_scan launch");
    }
    SLOT_WORD(err);
    m2::ScanArgs a{xbc,   dt_raw, A_log, dt_bias,      D,         z,   y, ssm_pool, cu_seqlens, state_indices,
                   has_initial_state, nseq, total_tokens, num_slots, err};
    return hip_status(m2::launch_chunk_scan(s, a, static_cast<hipStream_t>(stream)), "chunk_scan launch");
}

int mamba2_state_update(const mamba2_dims *d, const void *xbc, const void *dt_raw, const float *A_log,
                        const float *dt_bias, const float *D, const void *z, void *y, void *ssm_pool,
                        int32_t num_slots, const int32_t *state_indices, int32_t batch, void *stream) {
    int st = check_state_update(d);
    if (st) return st;
    if (num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be >= 0 (got %d)", num_slots);
    if (batch < 0) return fail(MAMBA2_ERR_INVALID_ARG, "batch < 0");
    if (batch == 0) return ok();
    REQUIRE_PTR(xbc); REQUIRE_PTR(dt_raw); REQUIRE_PTR(A_log); REQUIRE_PTR(dt_bias); REQUIRE_PTR(D);
    OPT_PTR(z); REQUIRE_PTR(y); REQUIRE_PTR(ssm_pool); REQUIRE_IDX(state_indices);
    SLOT_WORD(err);
    m2::StateUpdateArgs a{xbc, dt_raw, A_log, dt_bias, D, z, y, ssm_pool, state_indices, batch, num_slots, err};
    return hip_status(m2::launch_state_update(shape_of(d), a, static_cast<hipStream_t>(stream)), "state_update launch");
}

int mamba2_conv1d_update_multi(const mamba2_dims *d, const void *xbc, const float *conv_w, const float *conv_b,
                               void *xbc_out, void *conv_pool, int32_t num_slots, const int32_t *src_indices,
                               const int32_t *dst_indices, int32_t batch, int32_t tokens, void *stream) {
    int st = check_conv(d);
    if (st) return st;
    if (num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be >= 0 (got %d)", num_slots);
    if (batch < 0 || tokens < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative batch or tokens");
    if (batch == 0 || tokens == 0) return ok();
    REQUIRE_PTR(xbc); REQUIRE_PTR(conv_w); OPT_PTR(conv_b); REQUIRE_PTR(xbc_out); REQUIRE_PTR(conv_pool);
    REQUIRE_IDX(src_indices);
    if (dst_indices && (reinterpret_cast<uintptr_t>(dst_indices) & 3u))
        return fail(MAMBA2_ERR_INVALID_ARG, "dst_indices is not 4-byte aligned");
    if (xbc == xbc_out) return fail(MAMBA2_ERR_INVALID_ARG, "xbc_out must not alias xbc");
    SLOT_WORD(err);
    m2::ConvMultiArgs a{xbc, conv_w, conv_b, xbc_out, conv_pool, src_indices, dst_indices, batch, tokens, num_slots, err};
    return hip_status(m2::launch_conv_update_multi(shape_of(d), a, static_cast<hipStream_t>(stream)),
                      "conv1d_update_multi launch");
}

int mamba2_state_update_multi(const mamba2_dims *d, const void *xbc, const void *dt_raw, const float *A_log,
                              const float *dt_bias, const float *D, const void *z, void *y, void *ssm_pool,
                              int32_t num_slots, const int32_t *src_indices, const int32_t *dst_indices,
                              int32_t batch, int32_t tokens, void *stream) {
    int st = check_state_update(d);
    if (st) return st;
    if (num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be >= 0 (got %d)", num_slots);
    if (batch < 0 || tokens < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative batch or tokens");
    if (batch == 0 || tokens == 0) return ok();
    // (a row's T tokens are addressed by 32-bit byte offsets from the row's start)
    if ((int64_t)tokens * shape_of(d).cdim() * 4 > (int64_t)UINT32_MAX)
        return fail(MAMBA2_ERR_UNSUPPORTED, "tokens x Cdim x 4 bytes beyond 2^32 (tokens=%d, Cdim=%lld)", tokens,
                    (long long)shape_of(d).cdim());
    REQUIRE_PTR(xbc); REQUIRE_PTR(dt_raw); REQUIRE_PTR(A_log); REQUIRE_PTR(dt_bias); REQUIRE_PTR(D);
    OPT_PTR(z); REQUIRE_PTR(y); REQUIRE_PTR(ssm_pool); REQUIRE_IDX(src_indices);
    if (dst_indices && (reinterpret_cast<uintptr_t>(dst_indices) & 3u))
        return fail(MAMBA2_ERR_INVALID_ARG, "dst_indices is not 4-byte aligned");
    SLOT_WORD(err);
    m2::MultiStepArgs a{xbc,         dt_raw,      A_log, dt_bias, D,         z, y, ssm_pool, src_indices,
                        dst_indices, batch, tokens, num_slots, err};
    return hip_status(m2::launch_state_update_multi(shape_of(d), a, static_cast<hipStream_t>(stream)),
                      "state_update_multi launch");
}

int mamba2_mixed_fwd(const mamba2_dims *d, const void *xbc, const void *dt_raw, const void *z, const float *conv_w,
                     const float *conv_b, const float *A_log, const float *dt_bias, const float *D, void *xbc_post,
                     void *y, void *ssm_pool, void *conv_pool, int32_t num_slots, const int32_t *cu_seqlens, int32_t nseq,
                     int64_t total_tokens, const int32_t *prefill_indices, const uint8_t *has_initial_state,
                     const int32_t *decode_indices, int32_t decode_batch, void *workspace, size_t workspace_bytes,
                     void *stream) {
    int st = mamba2_check_dims(d);
    if (st) return st;
    if (nseq < 0 || total_tokens < 0 || decode_batch < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative size");
    if (total_tokens > INT32_MAX)  // (cu_seqlens are int32)
        return fail(MAMBA2_ERR_INVALID_ARG, "total_tokens %lld beyond the int32 range of cu_seqlens", (long long)total_tokens);
    const m2::LayerShape s = shape_of(d);
    const int64_t cdim = s.cdim(), hp = (int64_t)s.H * s.P;
    const size_t ab = dtype_bytes(d->act_dtype), xb = dtype_bytes(d->xbc_dtype), ob = dtype_bytes(d->out_dtype);
    if (nseq > 0) {
        size_t need = 0;
        st = mamba2_prefill_workspace_bytes(d, total_tokens, &need);
        if (st) return st;
        if (workspace && workspace_bytes >= need && total_tokens > 0) {
            // whole prefill in one call (fused for the Nemotron head shape); xbc_post rows of the
            // prefill segment are not written
            st = mamba2_prefill_fwd(d, xbc, dt_raw, z, conv_w, conv_b, A_log, dt_bias, D, nullptr, 0.0f, 0, y,
                                    ssm_pool, conv_pool, num_slots, cu_seqlens, nseq, total_tokens, prefill_indices,
                                    has_initial_state, workspace, workspace_bytes, stream);
            if (st) return st;
        } else {
            st = mamba2_conv1d_fwd(d, xbc, conv_w, conv_b, xbc_post, conv_pool, num_slots, cu_seqlens, nseq,
                                   total_tokens, prefill_indices, has_initial_state, stream);
            if (st) return st;
            st = mamba2_chunk_scan_fwd(d, xbc_post, dt_raw, A_log, dt_bias, D, z, y, ssm_pool, num_slots, cu_seqlens,
                                       nseq, total_tokens, prefill_indices, has_initial_state, nullptr, 0, stream);
            if (st) return st;
        }
    }
    if (decode_batch > 0) {
        REQUIRE_PTR(xbc); REQUIRE_PTR(dt_raw); REQUIRE_PTR(xbc_post); REQUIRE_PTR(y);
        const char *xin = static_cast<const char *>(xbc) + total_tokens * cdim * ab;
        char *xpost = static_cast<char *>(xbc_post) + total_tokens * cdim * xb;
        const char *dtd = static_cast<const char *>(dt_raw) + total_tokens * s.H * ab;
        const char *zd = z ? static_cast<const char *>(z) + total_tokens * hp * ab : nullptr;
        char *yd = static_cast<char *>(y) + total_tokens * hp * ob;
        st = mamba2_conv1d_update(d, xin, conv_w, conv_b, xpost, conv_pool, num_slots, decode_indices, decode_batch,
                                  stream);
        if (st) return st;
        st = mamba2_state_update(d, xpost, dtd, A_log, dt_bias, D, zd, yd, ssm_pool, num_slots, decode_indices,
                                 decode_batch, stream);
        if (st) return st;
    }
    return ok();
}

// ------------------------------------------------------------ fused prefill + gated norm
namespace {

bool fused_path(const mamba2_dims *d) { return m2::prefill_fused_supported(shape_of(d)); }

int norm_group_of(const mamba2_dims *d, int32_t group) {
    return group > 0 ? group : (d->nheads * d->headdim) / d->ngroups;
}

int check_norm(const mamba2_dims *d, int32_t group) {
    const int64_t width = (int64_t)d->nheads * d->headdim;
    const int gs = norm_group_of(d, group);
    if (group < 0) return fail(MAMBA2_ERR_INVALID_ARG, "norm group size must be >= 0 (0 = H*P/G)");
    if (!m2::gated_norm_supported(width, gs))
        return fail(MAMBA2_ERR_UNSUPPORTED, "gated norm needs a group size dividing H*P, a multiple of 4, <= 4096 (%d)",
                    gs);
    return MAMBA2_OK;
}

}  // namespace

int mamba2_prefill_workspace_bytes(const mamba2_dims *d, int64_t total_tokens, size_t *bytes) {
    int st = check_conv(d);
    if (st) return st;
    st = check_scan(d);
    if (st) return st;
    if (!bytes) return fail(MAMBA2_ERR_INVALID_ARG, "bytes is NULL");
    if (total_tokens < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative total_tokens");
    const m2::LayerShape s = shape_of(d);
    *bytes = fused_path(d) ? (size_t)m2::fused_workspace_bytes(s, total_tokens)
                           : (size_t)s.cdim() * dtype_bytes(d->xbc_dtype) * (size_t)total_tokens;
    return ok();
}

int mamba2_gated_rmsnorm(const mamba2_dims *d, const void *y, const void *z, const float *norm_w, float eps,
                         int32_t group_size, void *out, int64_t rows, void *stream) {
    int st = check_dims_basic(d);
    if (st) return st;
    st = check_norm(d, group_size);
    if (st) return st;
    if (rows < 0) return fail(MAMBA2_ERR_INVALID_ARG, "rows < 0");
    if (!(eps >= 0.0f)) return fail(MAMBA2_ERR_INVALID_ARG, "eps must be >= 0");
    if (rows == 0) return ok();
    REQUIRE_PTR(y); OPT_PTR(z); REQUIRE_PTR(norm_w); REQUIRE_PTR(out);
    if (z && z == out) return fail(MAMBA2_ERR_INVALID_ARG, "out must not alias z");
    m2::NormArgs a{y, z, norm_w, out, eps, rows};
    return hip_status(m2::launch_gated_norm(a, d->out_dtype, d->act_dtype, (int64_t)d->nheads * d->headdim,
                                            norm_group_of(d, group_size), static_cast<hipStream_t>(stream)),
                      "gated_rmsnorm launch");
}

int mamba2_prefill_fwd(const mamba2_dims *d, const void *xbc, const void *dt_raw, const void *z, const float *conv_w,
                       const float *conv_b, const float *A_log, const float *dt_bias, const float *D,
                       const float *norm_w, float norm_eps, int32_t norm_group, void *y, void *ssm_pool,
                       void *conv_pool, int32_t num_slots, const int32_t *cu_seqlens, int32_t nseq,
                       int64_t total_tokens, const int32_t *state_indices, const uint8_t *has_initial_state,
                       void *workspace, size_t workspace_bytes, void *stream) {
    int st = check_conv(d);
    if (st) return st;
    st = check_scan(d);
    if (st) return st;
    if (num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be >= 0 (got %d)", num_slots);
    if (norm_w) {
        st = check_norm(d, norm_group);
        if (st) return st;
        if (!(norm_eps >= 0.0f)) return fail(MAMBA2_ERR_INVALID_ARG, "norm_eps must be >= 0");
    }
    if (nseq < 0 || total_tokens < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative nseq or total_tokens");
    if (total_tokens > INT32_MAX)  // (cu_seqlens are int32)
        return fail(MAMBA2_ERR_INVALID_ARG, "total_tokens %lld beyond the int32 range of cu_seqlens", (long long)total_tokens);
    if (nseq == 0) {
        if (total_tokens != 0) return fail(MAMBA2_ERR_INVALID_ARG, "tokens without sequences");
        return ok();
    }
    size_t need = 0;
    st = mamba2_prefill_workspace_bytes(d, total_tokens, &need);
    if (st) return st;
    if (workspace_bytes < need)
        return fail(MAMBA2_ERR_WORKSPACE, "prefill needs %zu workspace bytes, got %zu", need, workspace_bytes);
    REQUIRE_PTR(conv_w); OPT_PTR(conv_b); REQUIRE_PTR(A_log); REQUIRE_PTR(dt_bias); REQUIRE_PTR(D);
    REQUIRE_PTR(ssm_pool); REQUIRE_PTR(conv_pool); REQUIRE_IDX(cu_seqlens); REQUIRE_IDX(state_indices);
    if (total_tokens > 0) {
        REQUIRE_PTR(xbc); REQUIRE_PTR(dt_raw); REQUIRE_PTR(y); OPT_PTR(z); REQUIRE_PTR(workspace);
        if (xbc == y || workspace == xbc || workspace == y)
            return fail(MAMBA2_ERR_INVALID_ARG, "xbc, y and workspace must not alias");
    }
    hipStream_t strm = static_cast<hipStream_t>(stream);
    const m2::LayerShape s = shape_of(d);
    // with a norm, the gate is applied by the norm pass (the scan writes ungated y)
    const void *scan_z = norm_w ? nullptr : z;
    SLOT_WORD(err);
    m2::ConvFwdArgs ca{xbc,  conv_w,       conv_b, workspace, conv_pool, cu_seqlens, state_indices, has_initial_state,
                       nseq, total_tokens, num_slots, err};
    if (fused_path(d)) {
        m2::FusedArgs fa{xbc, conv_w, conv_b, conv_pool, dt_raw, A_log, dt_bias, D, scan_z, y, ssm_pool,
                         cu_seqlens, state_indices, has_initial_state, nseq, total_tokens, nullptr, nullptr, nullptr};
        fa.num_slots = num_slots;
        fa.err = err;
        st = hip_status(m2::launch_fused_prefill(s, fa, total_tokens > 0 ? workspace : nullptr, strm), "prefill launch");
        if (st) return st;
        st = hip_status(m2::launch_conv_state(s, ca, strm), "prefill conv state launch");
        if (st) return st;
    } else {
        st = mamba2_conv1d_fwd(d, xbc, conv_w, conv_b, workspace, conv_pool, num_slots, cu_seqlens, nseq,
                               total_tokens, state_indices, has_initial_state, stream);
        if (st) return st;
        st = mamba2_chunk_scan_fwd(d, workspace, dt_raw, A_log, dt_bias, D, scan_z, y, ssm_pool, num_slots,
                                   cu_seqlens, nseq, total_tokens, state_indices, has_initial_state, nullptr, 0, stream);
        if (st) return st;
    }
    if (norm_w && total_tokens > 0)
        return mamba2_gated_rmsnorm(d, y, z, norm_w, norm_eps, norm_group, y, total_tokens, stream);
    return ok();
}

int mamba2_prefill_fwd_noalloc(const mamba2_dims *d, const void *xbc, const void *dt_raw, const void *z,
                               const float *conv_w, const float *conv_b, const float *A_log, const float *dt_bias,
                               const float *D, const float *norm_w, float norm_eps, int32_t norm_group, void *y,
                               void *ssm_pool, void *conv_pool, int32_t num_slots, const int32_t *cu_seqlens,
                               int32_t nseq, int64_t total_tokens, const int32_t *state_indices,
                               const uint8_t *has_initial_state, void *stream) {
    size_t need = 0;
    int st = mamba2_prefill_workspace_bytes(d, total_tokens, &need);
    if (st) return st;
    if (need > MAMBA2_STATIC_SCRATCH_BYTES)
        return fail(MAMBA2_ERR_WORKSPACE,
                    "prefill of %lld tokens needs %zu workspace bytes, more than the %u-byte static scratch; "
                    "split it into smaller chunks or use mamba2_prefill_fwd with a workspace",
                    (long long)total_tokens, need, (unsigned)MAMBA2_STATIC_SCRATCH_BYTES);
    void *scratch = nullptr;
    size_t bytes = 0;
    if (nseq > 0 && total_tokens > 0) {
        st = hip_status(m2::static_scratch(&scratch, &bytes), "static scratch lookup");
        if (st) return st;
    }
    return mamba2_prefill_fwd(d, xbc, dt_raw, z, conv_w, conv_b, A_log, dt_bias, D, norm_w, norm_eps, norm_group, y,
                              ssm_pool, conv_pool, num_slots, cu_seqlens, nseq, total_tokens, state_indices,
                              has_initial_state, scratch, bytes, stream);
}

// ------------------------------------------------------------ Mamba-1 selective scan
namespace {

int check_sel(const mamba1_dims *d) {
    if (!d) return fail(MAMBA2_ERR_INVALID_ARG, "dims is NULL");
    if (d->dim <= 0 || d->dstate <= 0 || d->ngroups <= 0)
        return fail(MAMBA2_ERR_INVALID_ARG, "dims must be positive (Dc=%d N=%d G=%d)", d->dim, d->dstate, d->ngroups);
    if (d->dim % d->ngroups != 0)
        return fail(MAMBA2_ERR_INVALID_ARG, "dim (%d) must be a multiple of ngroups (%d)", d->dim, d->ngroups);
    if (!valid_dtype(d->act_dtype) || !valid_dtype(d->state_dtype) || !valid_dtype(d->out_dtype))
        return fail(MAMBA2_ERR_INVALID_ARG, "unknown dtype code");
    m2::SelShape s{d->dim, d->dstate, d->ngroups, d->act_dtype, d->state_dtype, d->out_dtype};
    if (!m2::selective_scan_supported(s))
        return fail(MAMBA2_ERR_UNSUPPORTED,
                    "selective scan supports dstate in {4, 8, 16} with dim/ngroups a multiple of 64/128/256 (Dc=%d "
                    "N=%d G=%d)", d->dim, d->dstate, d->ngroups);
    return MAMBA2_OK;
}

}  // namespace

size_t mamba1_ssm_slot_bytes(const mamba1_dims *d) {
    if (!d || d->dim <= 0 || d->dstate <= 0 || !valid_dtype(d->state_dtype)) return 0;
    return (size_t)d->dim * d->dstate * dtype_bytes(d->state_dtype);
}

int mamba1_selective_scan_fwd(const mamba1_dims *d, const void *u, const void *delta_raw, const float *A,
                              const void *B, const void *C, const float *D, const void *z, const float *delta_bias,
                              int32_t delta_softplus, void *y, void *ssm_pool, int32_t num_slots,
                              const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens,
                              const int32_t *state_indices, const uint8_t *has_initial_state, void *stream) {
    int st = check_sel(d);
    if (st) return st;
    if (num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be >= 0 (got %d)", num_slots);
    if (nseq < 0 || total_tokens < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative nseq or total_tokens");
    if (total_tokens > INT32_MAX)  // (cu_seqlens are int32)
        return fail(MAMBA2_ERR_INVALID_ARG, "total_tokens %lld beyond the int32 range of cu_seqlens", (long long)total_tokens);
    if (nseq == 0) {
        if (total_tokens != 0) return fail(MAMBA2_ERR_INVALID_ARG, "tokens without sequences");
        return ok();
    }
    REQUIRE_PTR(A); OPT_PTR(D); OPT_PTR(delta_bias); REQUIRE_PTR(ssm_pool);
    REQUIRE_IDX(cu_seqlens); REQUIRE_IDX(state_indices);
    if (total_tokens > 0) {
        REQUIRE_PTR(u); REQUIRE_PTR(delta_raw); REQUIRE_PTR(B); REQUIRE_PTR(C); OPT_PTR(z); REQUIRE_PTR(y);
        if (y == u || y == delta_raw || (z && y == z)) return fail(MAMBA2_ERR_INVALID_ARG, "y must not alias inputs");
    }
    m2::SelShape s{d->dim, d->dstate, d->ngroups, d->act_dtype, d->state_dtype, d->out_dtype};
    SLOT_WORD(err);
    m2::SelScanArgs a{u, delta_raw, A, B, C, D, z, delta_bias, delta_softplus ? 1 : 0, y, ssm_pool, cu_seqlens,
                      state_indices, has_initial_state, nseq, total_tokens, num_slots, err};
    return hip_status(m2::launch_selective_scan(s, a, static_cast<hipStream_t>(stream)), "selective_scan launch");
}

int mamba1_selective_state_update(const mamba1_dims *d, const void *u, const void *delta_raw, const float *A,
                                  const void *B, const void *C, const float *D, const void *z,
                                  const float *delta_bias, int32_t delta_softplus, void *y, void *ssm_pool,
                                  int32_t num_slots, const int32_t *state_indices, int32_t batch, void *stream) {
    int st = check_sel(d);
    if (st) return st;
    if (num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be >= 0 (got %d)", num_slots);
    if (batch < 0) return fail(MAMBA2_ERR_INVALID_ARG, "batch < 0");
    if (batch == 0) return ok();
    REQUIRE_PTR(u); REQUIRE_PTR(delta_raw); REQUIRE_PTR(A); REQUIRE_PTR(B); REQUIRE_PTR(C); OPT_PTR(D); OPT_PTR(z);
    OPT_PTR(delta_bias); REQUIRE_PTR(y); REQUIRE_PTR(ssm_pool); REQUIRE_IDX(state_indices);
    if (y == u || y == delta_raw || (z && y == z)) return fail(MAMBA2_ERR_INVALID_ARG, "y must not alias inputs");
    m2::SelShape s{d->dim, d->dstate, d->ngroups, d->act_dtype, d->state_dtype, d->out_dtype};
    SLOT_WORD(err);
    m2::SelUpdateArgs a{u, delta_raw, A, B, C, D, z, delta_bias, delta_softplus ? 1 : 0, y, ssm_pool, state_indices,
                        batch, num_slots, err};
    return hip_status(m2::launch_selective_update(s, a, static_cast<hipStream_t>(stream)),
                      "selective_state_update launch");
}

// ------------------------------------------------------------ slot allocator
struct mamba2_slots {
    std::vector<int32_t> free_list;  // stack of free slot ids
    std::vector<uint8_t> in_use;
};

int mamba2_slots_create(int32_t num_slots, mamba2_slots **out) {
    if (!out) return fail(MAMBA2_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (num_slots <= 0) return fail(MAMBA2_ERR_INVALID_ARG, "num_slots must be positive");
    auto *s = new (std::nothrow) mamba2_slots;
    if (!s) return fail(MAMBA2_ERR_NO_SLOT, "out of host memory for %d slots", num_slots);
    try {  // no exception may cross the C ABI
        s->free_list.reserve(num_slots);
        for (int32_t i = num_slots - 1; i >= 0; --i) s->free_list.push_back(i);  // slot 0 is handed out first
        s->in_use.assign(num_slots, 0);
    } catch (...) {
        delete s;
        return fail(MAMBA2_ERR_NO_SLOT, "out of host memory for %d slots", num_slots);
    }
    *out = s;
    return ok();
}

int mamba2_slot_alloc(mamba2_slots *s, int32_t *slot) {
    if (!s || !slot) return fail(MAMBA2_ERR_INVALID_ARG, "NULL argument");
    if (s->free_list.empty()) return fail(MAMBA2_ERR_NO_SLOT, "all %zu slots are in use", s->in_use.size());
    *slot = s->free_list.back();
    s->free_list.pop_back();
    s->in_use[*slot] = 1;
    return ok();
}

int mamba2_slot_free(mamba2_slots *s, int32_t slot) {
    if (!s) return fail(MAMBA2_ERR_INVALID_ARG, "NULL allocator");
    if (slot < 0 || (size_t)slot >= s->in_use.size() || !s->in_use[slot])
        return fail(MAMBA2_ERR_NO_SLOT, "slot %d is not allocated", slot);
    s->in_use[slot] = 0;
    s->free_list.push_back(slot);
    return ok();
}

int32_t mamba2_slots_in_use(const mamba2_slots *s) {
    return s ? (int32_t)(s->in_use.size() - s->free_list.size()) : 0;
}

void mamba2_slots_destroy(mamba2_slots *s) { delete s; }

const char *mamba2_status_string(int status) {
    switch (status) {
        case MAMBA2_OK: return "ok";
        case MAMBA2_ERR_INVALID_ARG: return "invalid argument";
        case MAMBA2_ERR_UNSUPPORTED: return "unsupported dims or dtype";
        case MAMBA2_ERR_WORKSPACE: return "workspace too small";
        case MAMBA2_ERR_HIP: return "HIP error";
        case MAMBA2_ERR_NO_SLOT: return "no slot";
        default: return "unknown status";
    }
}

const char *mamba2_last_error(void) { return g_last_error.c_str(); }

int mamba2_read_slot_errors(uint32_t *count, int32_t reset, void *stream) {
    REQUIRE_IDX(count);
    return hip_status(m2::launch_read_slot_errors(count, reset ? 1 : 0, static_cast<hipStream_t>(stream)),
                      "read_slot_errors launch");
}

int mamba2_check_slot_indices(const int32_t *indices, int32_t n, int32_t num_slots, uint32_t *result, void *stream) {
    if (n < 0 || num_slots < 0) return fail(MAMBA2_ERR_INVALID_ARG, "negative n or num_slots");
    REQUIRE_PTR(result);
    if (n > 0) REQUIRE_IDX(indices);
    return hip_status(m2::launch_check_slots(indices, n, num_slots, result, static_cast<hipStream_t>(stream)),
                      "check_slot_indices launch");
}

const char *mamba2_version(void) { return "mamba2-gfx950 0.1"; }

}  // extern "C"
