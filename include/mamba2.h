/*
 * mamba2.h -- C ABI of the gfx950 (MI355X) Mamba-2 SSM core.
 *
 * The library computes the SSM core of the Mamba-2 mixer in hybrid
 * Mamba-Transformer models:
 *   - causal depthwise conv1d + SiLU over the x/B/C channels, as a prefill
 *     form and a one-token decode form;
 *   - the selective recurrence, as a chunked SSD scan for prefill and as a
 *     one-token state update for decode;
 *   - varlen (cu_seqlens) packing and mixed prefill + decode batches.
 *
 * Sources on the pages:
 *   [record]  "Nemotron-H-8B-Base-8K" -- mixer tensors (A_log, D, conv1d,
 *             dt_bias), n_groups 8, section "Recurrent state" (128 heads x
 *             headdim 64 x d_state 128; 2 MiB per layer per sequence in bf16),
 *             section "REQUIRED KERNEL CLASS" (a chunked scan kernel plus a
 *             fixed-size recurrent-state allocator);
 *   [vllm.cpp] "NemotronH runs the PREFILL mamba kernels at decode" --
 *             section "The divergence" (decode ops take state/conv-state
 *             indices and read+write the cache in place at the slot),
 *             section "Cost, at T=1, chunk_size=128, nchunks=1" (the one-step
 *             update: 1 launch, no allocation, no memset, no scratch),
 *             section "Confirm or refute" (hpg = H/G; the chunk scan must
 *             equal repeated single steps);
 *   [TRT-LLM] "Hybrid GDN (Qwen3.5-class) at high concurrency: mixed
 *             prefill+decode iterations..." -- mixed batches of context
 *             chunks and decode rows in one iteration.
 *
 * Math (per sequence, tokens in order; g(h) = h / (H/G)):
 *   conv:  v_t[c] = bias[c] + sum_k w[c][k] * u~[t-(W-1)+k][c],  x|B|C = SiLU(v)
 *          (u~ = [cached W-1 raw inputs, oldest first || new tokens];
 *           tap W-1 multiplies the current token)
 *   dt = softplus(dt_raw + dt_bias[h]), A = -exp(A_log[h]), a = exp(dt * A)
 *   h_t[h][p][n] = a * h_{t-1}[h][p][n] + dt * x_t[h][p] * B_t[g(h)][n]
 *   y_t[h][p]    = sum_n C_t[g(h)][n] * h_t[h][p][n] + D[h] * x_t[h][p]
 *                  (times SiLU(z_t[h][p]) when z is given)
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned device memory (for example torch
 *     tensors), contiguous, 16-byte aligned. The library keeps no pointer
 *     after a call returns and never allocates, frees or memsets memory.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is
 *     enqueued on it; results are valid once the stream reaches the call.
 *     No entry point synchronises the host.
 *   - Return value: MAMBA2_OK (0) or an error code. On error nothing was
 *     enqueued; mamba2_last_error() gives a thread-local message.
 *   - Layouts (N fastest in the SSM pool, channel fastest elsewhere):
 *       xBC        [T][Cdim], Cdim = H*P + 2*G*N, channels x (h*P + p) || B (g*N + n) || C (g*N + n)
 *       dt_raw     [T][H]          z, y  [T][H*P]
 *       conv w     [Cdim][W] fp32  conv bias [Cdim] fp32 or NULL
 *       A_log, dt_bias, D  [H] fp32
 *       ssm pool   [slots][H][P][N]   (state_dtype)
 *       conv pool  [slots][W-1][Cdim] (state_dtype; raw pre-conv inputs, oldest first)
 *   - Every entry point that takes a pool also takes num_slots, the number of
 *     slots the caller allocated in it (both pools of a call have that many).
 *     Slot index < 0 marks a padding row/sequence: its outputs are written as
 *     zero and no slot is read or written. An index >= num_slots is a caller
 *     error that the kernels treat the same way (outputs zero, no slot access,
 *     so nothing outside the pool is touched) and count in a per-device word
 *     that mamba2_slot_errors reads. Two rows of one call on the same slot race
 *     (undefined result); mamba2_check_slot_indices finds such duplicates.
 *   - Sizes: a call with zero rows / zero tokens is valid and enqueues nothing.
 */
#ifndef MAMBA2_H
#define MAMBA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MAMBA2_OK = 0,
    MAMBA2_ERR_INVALID_ARG = 1,  /* null pointer, misalignment, negative size, H % G != 0 ... */
    MAMBA2_ERR_UNSUPPORTED = 2,  /* dims or dtypes outside the compiled kernel set */
    MAMBA2_ERR_WORKSPACE = 3,    /* workspace missing or too small */
    MAMBA2_ERR_HIP = 4,          /* a HIP launch failed */
    MAMBA2_ERR_NO_SLOT = 5       /* slot allocator: pool exhausted or slot not allocated */
} mamba2_status;

typedef enum { MAMBA2_F32 = 0, MAMBA2_BF16 = 1 } mamba2_dtype;

/* Layer dimensions and storage dtypes.
 *   act_dtype   raw xBC, dt_raw and z
 *   xbc_dtype   post-conv xBC, written by the conv entry points and read by
 *               the scan and the state update (F32 keeps fp32-state prefill
 *               within 1e-3 of exact arithmetic)
 *   state_dtype SSM pool and conv pool
 *   out_dtype   y                                                            */
typedef struct {
    int32_t nheads, headdim, dstate, ngroups, conv_width, chunk_size;
    int32_t act_dtype, xbc_dtype, state_dtype, out_dtype;
} mamba2_dims;

/* Returns MAMBA2_OK if every entry point supports `dims`, else
 * MAMBA2_ERR_INVALID_ARG / MAMBA2_ERR_UNSUPPORTED (message in mamba2_last_error). */
int mamba2_check_dims(const mamba2_dims *dims);

/* Bytes of one SSM pool slot: H*P*N*sizeof(state). At Nemotron-H-8B dims in
 * bf16 this is 2 MiB per layer per sequence ([record], "Recurrent state").
 * Returns 0 for invalid dims. */
size_t mamba2_ssm_slot_bytes(const mamba2_dims *dims);

/* Bytes of one conv pool slot: (W-1)*Cdim*sizeof(state). 0 for invalid dims. */
size_t mamba2_conv_slot_bytes(const mamba2_dims *dims);

/* Workspace for the faster form of mamba2_chunk_scan_fwd with `total_tokens`
 * packed tokens in `nseq` sequences (written to *bytes). For headdim 64,
 * dstate 128 with bf16 act_dtype and out_dtype it is the B/C operand planes of
 * each 32-token block (the same layout and size as
 * mamba2_prefill_workspace_bytes); 0 for every other shape, whose scan keeps
 * all chunk data on chip. The workspace is optional: a call without one runs
 * the workspace-free chunk kernel. */
int mamba2_chunk_scan_workspace_bytes(const mamba2_dims *dims, int64_t total_tokens, int32_t nseq,
                                      size_t *bytes);

/* Prefill conv1d + SiLU over packed sequences ([record] conv1d tensor).
 *   xbc            [total_tokens][Cdim] act_dtype, raw inputs (not modified)
 *   xbc_out        [total_tokens][Cdim] xbc_dtype, SiLU(conv); must not alias xbc
 *   cu_seqlens     [nseq+1] int32 device, cu_seqlens[0] = 0, nondecreasing,
 *                  cu_seqlens[nseq] = total_tokens (so total_tokens <= INT32_MAX;
 *                  larger totals return MAMBA2_ERR_INVALID_ARG)
 *   state_indices  [nseq] int32 device: conv pool slot of each sequence
 *   has_initial_state [nseq] uint8 device or NULL (all 0): 1 = left context is
 *                  the slot's cached inputs, 0 = zeros
 * Afterwards each used slot holds the sequence's last W-1 raw inputs (taken
 * from the old cache for sequences shorter than W-1). Rows of padding
 * sequences (slot < 0) are written as zero. */
int mamba2_conv1d_fwd(const mamba2_dims *dims, const void *xbc, const float *conv_w,
                      const float *conv_b, void *xbc_out, void *conv_pool, int32_t num_slots,
                      const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens,
                      const int32_t *state_indices, const uint8_t *has_initial_state,
                      void *stream);

/* One-token conv1d + SiLU per row, shifting the slot's cached inputs in place
 * ([vllm.cpp], "The divergence": conv-state indices, in place at the slot).
 *   xbc [batch][Cdim] act_dtype; xbc_out [batch][Cdim] xbc_dtype (may not alias xbc);
 *   state_indices [batch] int32 device. */
int mamba2_conv1d_update(const mamba2_dims *dims, const void *xbc, const float *conv_w,
                         const float *conv_b, void *xbc_out, void *conv_pool, int32_t num_slots,
                         const int32_t *state_indices, int32_t batch, void *stream);

/* Chunked SSD scan over packed sequences ([record], "REQUIRED KERNEL CLASS").
 *   xbc   [total_tokens][Cdim] xbc_dtype, post-conv x||B||C
 *   dt_raw [total_tokens][H] act_dtype;  z [total_tokens][H*P] act_dtype or NULL
 *   y     [total_tokens][H*P] out_dtype
 *   ssm_pool: the initial state is read from slot state_indices[i] when
 *   has_initial_state[i] is 1 (zeros otherwise); the final state is written
 *   to that slot. dims->chunk_size is the SSD chunk length.
 *   workspace/workspace_bytes: NULL/0, or device memory of at least
 *   mamba2_chunk_scan_workspace_bytes (MAMBA2_ERR_WORKSPACE if smaller), not
 *   aliasing xbc or y. With one, the shapes that size it nonzero run as
 *   32-token blocks whose B/C operands are formed once per group in the
 *   workspace (the mamba2_prefill_fwd kernels with the conv left out); without
 *   one, as chunks of dims->chunk_size on chip. Both give the scan's result up
 *   to rounding order. */
int mamba2_chunk_scan_fwd(const mamba2_dims *dims, const void *xbc, const void *dt_raw,
                          const float *A_log, const float *dt_bias, const float *D, const void *z,
                          void *y, void *ssm_pool, int32_t num_slots, const int32_t *cu_seqlens,
                          int32_t nseq, int64_t total_tokens, const int32_t *state_indices,
                          const uint8_t *has_initial_state, void *workspace,
                          size_t workspace_bytes, void *stream);

/* One-token selective state update per row, reading and writing
 * ssm_pool[state_indices[i]] in place ([vllm.cpp], "The divergence" and the
 * right-hand column of "Cost, at T=1, chunk_size=128, nchunks=1": one launch,
 * no allocation, no memset, no scratch).
 *   xbc [batch][Cdim] xbc_dtype (post-conv); dt_raw [batch][H] act_dtype;
 *   z [batch][H*P] act_dtype or NULL; y [batch][H*P] out_dtype.
 *   Supported: dstate 16, 64 or 128, headdim a multiple of 4, and Cdim and
 *   headdim * dstate at most 2^24 (rows and state tiles are addressed by 32-bit
 *   byte offsets); MAMBA2_ERR_UNSUPPORTED otherwise, here and in every entry
 *   point that runs the update (multi-token, mixed). */
int mamba2_state_update(const mamba2_dims *dims, const void *xbc, const void *dt_raw,
                        const float *A_log, const float *dt_bias, const float *D, const void *z,
                        void *y, void *ssm_pool, int32_t num_slots, const int32_t *state_indices,
                        int32_t batch, void *stream);

/* Multi-token decode: `tokens` (T) consecutive tokens per row, as when a step
 * verifies drafted tokens ([TRT-LLM]: one-model MTP in the hybrid serving
 * configurations; the equivalence of one multi-token pass and T single steps is
 * the [vllm.cpp] "Confirm or refute" contract). Row i starts from the state in
 * slot src_indices[i] and takes its T tokens in order; after token t the state
 * (conv window, SSM state) is written to slot dst_indices[i*T + t] when that is
 * >= 0, a per-step snapshot the caller can resume from once it knows how many
 * tokens were accepted. dst_indices NULL: only the final state is written, back
 * to src_indices[i]. The state stays in registers between tokens, so it is
 * rounded to the pool dtype only where it is written.
 *   xbc [batch][T][Cdim] (raw for conv1d, post-conv xbc_dtype for the state
 *   update); dt_raw [batch][T][H]; z [batch][T][H*P] or NULL; y [batch][T][H*P];
 *   xbc_out [batch][T][Cdim] xbc_dtype.
 * Every source slot is read before any destination is written only within a
 * row: a destination that is another row's source (or two rows writing one
 * slot) races. src_indices[i] < 0 marks a padding row (y = 0, no slot access).
 * mamba2_state_update_multi addresses a row's tokens by 32-bit byte offsets:
 * T * Cdim * 4 above 2^32 - 1 returns MAMBA2_ERR_UNSUPPORTED (T up to 104,857
 * at Nemotron-H-8B dims). */
int mamba2_conv1d_update_multi(const mamba2_dims *dims, const void *xbc, const float *conv_w,
                               const float *conv_b, void *xbc_out, void *conv_pool, int32_t num_slots,
                               const int32_t *src_indices, const int32_t *dst_indices,
                               int32_t batch, int32_t tokens, void *stream);
int mamba2_state_update_multi(const mamba2_dims *dims, const void *xbc, const void *dt_raw,
                              const float *A_log, const float *dt_bias, const float *D,
                              const void *z, void *y, void *ssm_pool, int32_t num_slots,
                              const int32_t *src_indices, const int32_t *dst_indices, int32_t batch,
                              int32_t tokens, void *stream);

/* Mixed batch ([TRT-LLM] mixed prefill+decode iterations): the prefill
 * segment (packed by cu_seqlens) runs conv1d_fwd + chunk_scan_fwd, or
 * mamba2_prefill_fwd when `workspace` holds at least
 * mamba2_prefill_workspace_bytes(total_tokens) (then xbc_post rows
 * [0, total_tokens) are not written); the decode segment (`decode_batch`
 * rows, one token each) runs conv1d_update + state_update, all on `stream`
 * with no host synchronisation.
 *   xbc/dt_raw/z/y hold prefill tokens in rows [0, total_tokens) and decode
 *   rows in rows [total_tokens, total_tokens + decode_batch);
 *   xbc_post [total_tokens + decode_batch][Cdim] xbc_dtype receives the conv output.
 *   prefill_indices [nseq], decode_indices [decode_batch]: pool slots. */
int mamba2_mixed_fwd(const mamba2_dims *dims, const void *xbc, const void *dt_raw, const void *z,
                     const float *conv_w, const float *conv_b, const float *A_log,
                     const float *dt_bias, const float *D, void *xbc_post, void *y,
                     void *ssm_pool, void *conv_pool, int32_t num_slots, const int32_t *cu_seqlens,
                     int32_t nseq, int64_t total_tokens, const int32_t *prefill_indices,
                     const uint8_t *has_initial_state, const int32_t *decode_indices,
                     int32_t decode_batch, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Workspace that mamba2_prefill_fwd needs for `total_tokens` packed tokens.
 * For the fused shape (headdim 64, dstate 128, out_dtype bf16) it holds the
 * post-conv B/C operands of each 32-token block of the packed batch: C
 * (G*N bf16 per token), B^T as hi/lo bf16 (2*G*N per token) and C.B^T
 * (G*32 fp32 per token), each region rounded up to 256 bytes; from 2048
 * tokens on it also holds what the segment mode needs, used when few
 * sequences (nseq*H <= 256) would leave most of the GPU idle: each long
 * sequence is then cut into up to 8 segments scanned in parallel from zero
 * state and joined afterwards by linearity (512/H segment records, their
 * final states in fp32 and as bf16 MFMA operands, H*P*N*6 bytes per record
 * with the per-head decays, and one fp32 log-decay per block and head);
 * otherwise the post-conv xBC, Cdim elements of xbc_dtype per token. */
int mamba2_prefill_workspace_bytes(const mamba2_dims *dims, int64_t total_tokens, size_t *bytes);

/* Whole prefill of the mixer's SSM core over packed sequences: conv1d + SiLU,
 * chunked SSD scan, optional gate and optional gated RMSNorm ([record]: mixer
 * tensors conv1d, A_log, D, dt_bias, norm; "REQUIRED KERNEL CLASS").
 * Same results as mamba2_conv1d_fwd followed by mamba2_chunk_scan_fwd (and
 * mamba2_gated_rmsnorm when norm_w is given), but for the fused shape the x
 * channels are convolved inside the scan and never stored: only the B/C
 * channels pass through the workspace, once per group rather than per head.
 *   xbc [total_tokens][Cdim] act_dtype, raw (pre-conv); dt_raw, z as for
 *   chunk_scan_fwd; y [total_tokens][H*P] out_dtype.
 *   norm_w [H*P] fp32 or NULL (no norm): y = norm_w * g / rms_group(g) with
 *   g = y_ssm * SiLU(z) (g = y_ssm when z is NULL), groups of norm_group
 *   consecutive channels (0 = H*P/G), rms over the group plus norm_eps.
 *   conv_pool / ssm_pool: read at state_indices[i] when has_initial_state[i]
 *   is 1, then overwritten with the sequence's final conv and SSM state.
 *   workspace: device memory of at least mamba2_prefill_workspace_bytes
 *   (MAMBA2_ERR_WORKSPACE otherwise); its contents are scratch. */
int mamba2_prefill_fwd(const mamba2_dims *dims, const void *xbc, const void *dt_raw, const void *z,
                       const float *conv_w, const float *conv_b, const float *A_log,
                       const float *dt_bias, const float *D, const float *norm_w, float norm_eps,
                       int32_t norm_group, void *y, void *ssm_pool, void *conv_pool,
                       int32_t num_slots, const int32_t *cu_seqlens, int32_t nseq, int64_t total_tokens,
                       const int32_t *state_indices, const uint8_t *has_initial_state,
                       void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): mamba2_prefill_fwd with
 * the same arguments except the workspace, which is a fixed device array inside
 * the library, MAMBA2_STATIC_SCRATCH_BYTES per GPU, held from the time the
 * library's code is loaded on that GPU until the process ends. The call allocates
 * and frees nothing. A batch whose workspace (mamba2_prefill_workspace_bytes)
 * exceeds the array is refused with MAMBA2_ERR_WORKSPACE before anything is
 * enqueued (about 5,800 packed tokens at Nemotron-H-8B dims with bf16 y; split
 * longer prefills into chunks). Every call on one GPU uses the same array, which
 * keeps the last call's contents: calls that overlap on one GPU (two streams, two
 * host threads) race and must be serialised by the caller. */
#define MAMBA2_STATIC_SCRATCH_BYTES (64u * 1024u * 1024u)
int mamba2_prefill_fwd_noalloc(const mamba2_dims *dims, const void *xbc, const void *dt_raw, const void *z,
                               const float *conv_w, const float *conv_b, const float *A_log,
                               const float *dt_bias, const float *D, const float *norm_w, float norm_eps,
                               int32_t norm_group, void *y, void *ssm_pool, void *conv_pool,
                               int32_t num_slots, const int32_t *cu_seqlens, int32_t nseq,
                               int64_t total_tokens, const int32_t *state_indices,
                               const uint8_t *has_initial_state, void *stream);

/* Gated RMSNorm of mixer outputs ([record], the mixer's "norm" tensor):
 * out = norm_w * g / sqrt(mean_group(g^2) + eps), g = y * SiLU(z) (g = y when z
 * is NULL), over groups of group_size consecutive channels (0 = H*P/G).
 *   y, out [rows][H*P] out_dtype (out may equal y); z [rows][H*P] act_dtype or
 *   NULL; norm_w [H*P] fp32. group_size must divide H*P, be a multiple of 4
 *   and at most 4096 (MAMBA2_ERR_UNSUPPORTED otherwise). */
int mamba2_gated_rmsnorm(const mamba2_dims *dims, const void *y, const void *z, const float *norm_w,
                         float eps, int32_t group_size, void *out, int64_t rows, void *stream);

/* Captured decode step ([TRT-LLM], "Questions" item 1: run the decode rows of a
 * mixed iteration as a replay of the captured decode graph and only the context
 * chunk eagerly; "Corrected measurements": graphed decode replays against the
 * eager mixed pass). The decode of `nlayers` layer entries -- each
 * mamba2_conv1d_update then mamba2_state_update of `batch` rows with that
 * entry's buffers -- is recorded once into a HIP graph and replayed by
 * mamba2_decode_graph_launch with one launch. An entry is a layer at one step:
 * several steps of a stack are simply more entries. The graph keeps the
 * pointers: the caller refills the same buffers (inputs, slot indices) before a
 * replay and keeps them alive until mamba2_decode_graph_destroy.
 *   create: records on capture_stream (a created stream, not NULL); on error
 *           nothing is kept and *out is NULL. It instantiates the graph, which
 *           may allocate: call it at set-up, not per step.
 *   launch: enqueues one replay on `stream` (any stream); no allocation.
 * Messages of the graph calls: mamba2_decode_graph_last_error(). */
typedef struct {
    const void *xbc;                 /* [batch][Cdim] act_dtype, raw */
    const float *conv_w, *conv_b;    /* [Cdim][W]; [Cdim] or NULL */
    void *xbc_post;                  /* [batch][Cdim] xbc_dtype */
    void *conv_pool;                 /* [num_slots][W-1][Cdim] */
    const void *dt_raw;              /* [batch][H] */
    const float *A_log, *dt_bias, *D;
    const void *z;                   /* [batch][H*P] or NULL */
    void *y;                         /* [batch][H*P] out_dtype */
    void *ssm_pool;                  /* [num_slots][H][P][N] */
    int32_t num_slots;
    const int32_t *state_indices;    /* [batch] */
} mamba2_decode_layer;
typedef struct mamba2_decode_graph mamba2_decode_graph;
int mamba2_decode_graph_create(const mamba2_dims *dims, const mamba2_decode_layer *layers, int32_t nlayers,
                               int32_t batch, void *capture_stream, mamba2_decode_graph **out);
int mamba2_decode_graph_launch(mamba2_decode_graph *graph, void *stream);
void mamba2_decode_graph_destroy(mamba2_decode_graph *graph);
const char *mamba2_decode_graph_last_error(void);

/* Fixed-size recurrent-state slot allocator ([record], "REQUIRED KERNEL
 * CLASS": a fixed-size recurrent state allocator; "Recurrent state": the
 * cost scales with concurrency, not context). Host-only: it hands out slot
 * ids of a caller-owned pool in O(1); it never touches device memory. A new
 * sequence starts from zero state by passing has_initial_state = 0, not by
 * clearing its slot. Not thread-safe: calls on one allocator from several
 * threads need the caller's lock; distinct allocators are independent. One
 * allocator per pool. Host memory for the free list comes from the C++ heap;
 * if it runs out, mamba2_slots_create returns MAMBA2_ERR_NO_SLOT (no exception
 * crosses the ABI). */
typedef struct mamba2_slots mamba2_slots;
int mamba2_slots_create(int32_t num_slots, mamba2_slots **out);
int mamba2_slot_alloc(mamba2_slots *s, int32_t *slot);      /* MAMBA2_ERR_NO_SLOT when full */
int mamba2_slot_free(mamba2_slots *s, int32_t slot);        /* MAMBA2_ERR_NO_SLOT if not allocated */
int32_t mamba2_slots_in_use(const mamba2_slots *s);
void mamba2_slots_destroy(mamba2_slots *s);

/* Slot index safety ([vllm.cpp], "The divergence": the ops index the caller's
 * cache in place at the slot, so the library bounds every index it reads).
 * mamba2_read_slot_errors: when the stream reaches the call, count[0] (device
 * memory, one uint32) receives how many times kernels on the current device
 * skipped a row or sequence because its index was >= num_slots since the last
 * reset, and reset != 0 then sets that count to 0. A call with one bad row may
 * count it once per kernel of the call that reads the slot, so any nonzero
 * value means "a caller passed an index beyond its pool". The count lives in
 * one device word per GPU that every call on that GPU shares.
 * mamba2_check_slot_indices: a debug check of one index list on `stream`,
 * nothing else touched: result[0] = entries >= num_slots, result[1] = entries
 * in [0, num_slots) equal to an earlier entry (rows that would race); result
 * is device memory for 2 uint32, written (not accumulated) when the stream
 * reaches the call. O(n^2) compares in one workgroup: meant for debugging,
 * not for the hot path. */
int mamba2_read_slot_errors(uint32_t *count, int32_t reset, void *stream);
int mamba2_check_slot_indices(const int32_t *indices, int32_t n, int32_t num_slots, uint32_t *result,
                              void *stream);

const char *mamba2_status_string(int status);
const char *mamba2_last_error(void);
const char *mamba2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MAMBA2_H */
