/*
 * mamba1.h -- C ABI of the gfx950 (MI355X) Mamba-1 selective scan, in the same
 * library as mamba2.h (libmamba2.so).
 *
 * Source on the pages: the trace page "Hybrid Mamba-Transformer MoEs hide their
 * stalls..." names selective_scan_fwd among the kernels of Mamba layers and
 * cites the Mamba paper for the layer; the record page lists Mamba-1 model
 * classes (MambaForCausalLM, FalconMambaForCausalLM) among the hybrid/SSM rows.
 *
 * Math (per sequence, tokens in order; g(d) = d / (Dc/G)):
 *   delta_t[d] = softplus(delta_raw_t[d] + delta_bias[d])   (delta_softplus = 1)
 *              = delta_raw_t[d] + delta_bias[d]             (delta_softplus = 0)
 *   h_t[d][n]  = exp(delta_t[d] * A[d][n]) * h_{t-1}[d][n] + delta_t[d] * B_t[g][n] * u_t[d]
 *   y_t[d]     = sum_n C_t[g][n] * h_t[d][n] + D[d] * u_t[d]   (times SiLU(z_t[d]) when z is given)
 * A is the (negative) decay matrix itself, as the kernel takes it (a model
 * storing A_log passes -exp(A_log)).
 *
 * Conventions are those of mamba2.h (caller-owned 16-byte aligned device
 * memory, stream-ordered, no allocation, status codes, mamba2_last_error()).
 * Layouts: u, delta_raw, z, y [T][Dc]; B, C [T][G][N]; A [Dc][N] fp32;
 * D, delta_bias [Dc] fp32 or NULL; state pool [slots][Dc][N] (state_dtype).
 */
#ifndef MAMBA1_H
#define MAMBA1_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t dim;        /* Dc, channels (d_inner) */
    int32_t dstate;     /* N: 4, 8 or 16 */
    int32_t ngroups;    /* G: B/C groups (1 in the Mamba paper's layer) */
    int32_t act_dtype;  /* MAMBA2_F32 or MAMBA2_BF16: u, delta_raw, z, B, C */
    int32_t state_dtype;
    int32_t out_dtype;  /* y */
} mamba1_dims;

/* Bytes of one sequence's state slot: Dc * N * sizeof(state_dtype). */
size_t mamba1_ssm_slot_bytes(const mamba1_dims *dims);

/* Selective scan over packed sequences (cu_seqlens [nseq+1]). Sequence i
 * starts from ssm_pool[state_indices[i]] when has_initial_state[i] is 1 (zeros
 * otherwise; has_initial_state may be NULL) and its final state is written to
 * that slot. state_indices[i] < 0 marks a padding sequence (y = 0, no slot
 * access); num_slots is the pool's slot count, and an index >= num_slots is
 * skipped like padding and counted (see mamba2_slot_errors in mamba2.h).
 * Requires dstate in {4, 8, 16} and Dc/G a multiple of the
 * workgroup's channel count (64, 128, 256 for N = 16, 8, 4), else
 * MAMBA2_ERR_UNSUPPORTED. */
int mamba1_selective_scan_fwd(const mamba1_dims *dims, const void *u, const void *delta_raw,
                              const float *A, const void *B, const void *C, const float *D,
                              const void *z, const float *delta_bias, int32_t delta_softplus,
                              void *y, void *ssm_pool, int32_t num_slots, const int32_t *cu_seqlens,
                              int32_t nseq, int64_t total_tokens, const int32_t *state_indices,
                              const uint8_t *has_initial_state, void *stream);

/* One token per row, the state read and written in place at
 * ssm_pool[state_indices[i]] (the decode form; the in-place, index-addressed
 * update is the one the vllm.cpp page, "The divergence", asks for). Same math
 * and the same per-step arithmetic as mamba1_selective_scan_fwd, so T calls equal
 * one T-token scan. u, delta_raw, z, y [batch][Dc]; B, C [batch][G][N].
 * state_indices[i] < 0 marks a padding row (y = 0, no slot access); an index
 * >= num_slots is skipped and counted the same way; two rows on one slot race. */
int mamba1_selective_state_update(const mamba1_dims *dims, const void *u, const void *delta_raw,
                                  const float *A, const void *B, const void *C, const float *D,
                                  const void *z, const float *delta_bias, int32_t delta_softplus,
                                  void *y, void *ssm_pool, int32_t num_slots,
                                  const int32_t *state_indices, int32_t batch, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MAMBA1_H */
