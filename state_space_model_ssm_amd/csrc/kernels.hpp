// Host-side launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

struct LayerShape {
    int H, P, N, G, W, Q;
    int act_dt, xbc_dt, state_dt, out_dt;
    int64_t cdim() const { return (int64_t)H * P + 2LL * G * N; }
};

struct StateUpdateArgs {
    const void *xbc;      // [batch][Cdim] post-conv
    const void *dt_raw;   // [batch][H]
    const float *A_log, *dt_bias, *D;
    const void *z;        // [batch][H*P] or null
    void *y;              // [batch][H*P]
    void *pool;           // [slots][H][P][N]
    const int32_t *idx;   // [batch]
    int batch;
    int num_slots = 0;    // pool slots: indices >= num_slots are skipped like padding and counted in *err
    unsigned *err = nullptr;  // the library's per-device count of such indices
};

struct ConvUpdateArgs {
    const void *xbc;      // [batch][Cdim] raw
    const float *w, *b;   // [Cdim][W], [Cdim] or null
    void *out;            // [batch][Cdim]
    void *pool;           // [slots][W-1][Cdim]
    const int32_t *idx;
    int batch;
    int num_slots = 0;    // pool slots: indices >= num_slots are skipped like padding and counted in *err
    unsigned *err = nullptr;  // the library's per-device count of such indices
};

struct ConvFwdArgs {
    const void *xbc;      // [T][Cdim] raw
    const float *w, *b;
    void *out;            // [T][Cdim]
    void *pool;
    const int32_t *cu;    // [nseq+1]
    const int32_t *idx;   // [nseq]
    const uint8_t *has_init;  // [nseq] or null
    int nseq;
    int64_t T;
    int num_slots = 0;    // pool slots: indices >= num_slots are skipped like padding and counted in *err
    unsigned *err = nullptr;  // the library's per-device count of such indices
};

struct ScanArgs {
    const void *xbc;      // [T][Cdim] post-conv
    const void *dt_raw;   // [T][H]
    const float *A_log, *dt_bias, *D;
    const void *z;        // [T][H*P] or null
    void *y;              // [T][H*P]
    void *pool;           // [slots][H][P][N]
    const int32_t *cu, *idx;
    const uint8_t *has_init;
    int nseq;
    int64_t T;
    int num_slots = 0;    // pool slots: indices >= num_slots are skipped like padding and counted in *err
    unsigned *err = nullptr;  // the library's per-device count of such indices
};

// T tokens per row: activations [batch][T][...]; src [batch] (slot read before the
// first token), dst [batch][T] (slot written after each token, < 0 = skip) or
// null (final state written back to src).
struct MultiStepArgs {
    const void *xbc;      // [batch][T][Cdim] post-conv
    const void *dt_raw;   // [batch][T][H]
    const float *A_log, *dt_bias, *D;
    const void *z;        // [batch][T][H*P] or null
    void *y;              // [batch][T][H*P]
    void *pool;           // [slots][H][P][N]
    const int32_t *src, *dst;
    int batch, T;
    int num_slots = 0;    // pool slots: indices >= num_slots are skipped like padding and counted in *err
    unsigned *err = nullptr;  // the library's per-device count of such indices
};

struct ConvMultiArgs {
    const void *xbc;      // [batch][T][Cdim] raw
    const float *w, *b;
    void *out;            // [batch][T][Cdim]
    void *pool;           // [slots][W-1][Cdim]
    const int32_t *src, *dst;
    int batch, T;
    int num_slots = 0;    // pool slots: indices >= num_slots are skipped like padding and counted in *err
    unsigned *err = nullptr;  // the library's per-device count of such indices
};

// Fused prefill (fused.hip); cp / bt / cb are the workspace planes, set by
// launch_fused_prefill / launch_block_scan.
struct FusedArgs {
    const void *xbc;      // [T][Cdim]: raw (pre-conv, activation dtype) for launch_fused_prefill,
                          // post-conv (xbc dtype) for launch_block_scan
    const float *conv_w, *conv_b;  // [Cdim][W], [Cdim] or null (unused by launch_block_scan)
    const void *conv_pool;  // [slots][W-1][Cdim], read for the context before each sequence (idem)
    const void *dt_raw;   // [T][H]
    const float *A_log, *dt_bias, *D;
    const void *z;        // [T][H*P] or null
    void *y;              // [T][H*P] bf16
    void *pool;           // [slots][H][P][N]
    const int32_t *cu, *idx;
    const uint8_t *has_init;
    int nseq;
    int64_t T;
    void *cp, *bt, *cb;
    // segment mode (small batches; set by the launcher): workgroup row v takes segment v
    // of seg [nseg][4] = {start, end, sequence, flags} and, unless it is its sequence's
    // only segment, leaves its local final state and total log2 decay in seg_state /
    // seg_dec for the fix-up pass
    const int32_t *seg;
    float *seg_state;  // [nseg][H][P][N]
    float *seg_dec;    // [nseg][H]
    float *seg_lam;    // [block][H]: log2 decay from the segment's start through the block (blocks inside a segment)
    void *seg_hin;     // [nseg][H][4 waves][64 lanes][4] bf16x8: a later segment's true initial state, as MFMA operand
    int num_slots = 0;    // pool slots: indices >= num_slots are skipped like padding and counted in *err
    unsigned *err = nullptr;  // the library's per-device count of such indices
};

struct NormArgs {
    const void *y;        // [rows][width]
    const void *z;        // [rows][width] or null
    const float *w;       // [width]
    void *out;            // [rows][width] (may equal y)
    float eps;
    int64_t rows;
};

// Mamba-1 selective scan: Dc channels, N states, G groups of B/C.
struct SelShape {
    int Dc, N, G;
    int act_dt, state_dt, out_dt;
};

struct SelScanArgs {
    const void *u, *delta;       // [T][Dc] activation dtype
    const float *A;              // [Dc][N]
    const void *B, *C;           // [T][G][N] activation dtype
    const float *D;              // [Dc] or null
    const void *z;               // [T][Dc] or null
    const float *delta_bias;     // [Dc] or null
    int delta_softplus;
    void *y;                     // [T][Dc] out dtype
    void *pool;                  // [slots][Dc][N] state dtype
    const int32_t *cu, *idx;
    const uint8_t *has_init;
    int nseq;
    int64_t T;
    int num_slots = 0;    // pool slots: indices >= num_slots are skipped like padding and counted in *err
    unsigned *err = nullptr;  // the library's per-device count of such indices
};

struct SelUpdateArgs {
    const void *u, *delta;       // [batch][Dc]
    const float *A;              // [Dc][N]
    const void *B, *C;           // [batch][G][N]
    const float *D;              // [Dc] or null
    const void *z;               // [batch][Dc] or null
    const float *delta_bias;     // [Dc] or null
    int delta_softplus;
    void *y;                     // [batch][Dc]
    void *pool;                  // [slots][Dc][N]
    const int32_t *idx;          // [batch]
    int batch;
    int num_slots = 0;    // pool slots: indices >= num_slots are skipped like padding and counted in *err
    unsigned *err = nullptr;  // the library's per-device count of such indices
};

// Device address of this library's count of out-of-range slot indices on the current
// device (a file-scope device word, looked up once per device).
hipError_t slot_error_word(unsigned **out);
// Copies that count to dst (device memory) on the stream and clears it when reset != 0.
hipError_t launch_read_slot_errors(unsigned *dst, int reset, hipStream_t st);
// Debug check of one index list: result[0] = indices >= num_slots, result[1] = indices
// (>= 0) equal to an earlier one; one workgroup, result written without a prior clear.
hipError_t launch_check_slots(const int32_t *idx, int n, int num_slots, unsigned *result, hipStream_t st);

// Device address (current device) and size of the library's fixed scratch array, looked up
// once per device; the workspace of mamba2_prefill_fwd_noalloc.
hipError_t static_scratch(void **ptr, size_t *bytes);

// Each returns hipSuccess or the launch error. `supported` queries return
// false for shapes outside the compiled set (no launch happens).
bool state_update_supported(const LayerShape &s);
hipError_t launch_state_update(const LayerShape &s, const StateUpdateArgs &a, hipStream_t st);

hipError_t launch_state_update_multi(const LayerShape &s, const MultiStepArgs &a, hipStream_t st);
hipError_t launch_conv_update_multi(const LayerShape &s, const ConvMultiArgs &a, hipStream_t st);

bool conv_supported(const LayerShape &s);
hipError_t launch_conv_update(const LayerShape &s, const ConvUpdateArgs &a, hipStream_t st);
hipError_t launch_conv_fwd(const LayerShape &s, const ConvFwdArgs &a, hipStream_t st);
// B/C channels only, as bf16 planes [B hi | B lo | C] per token (a.out); no cache update
// the conv cache update of launch_conv_fwd alone
hipError_t launch_conv_state(const LayerShape &s, const ConvFwdArgs &a, hipStream_t st);

bool prefill_fused_supported(const LayerShape &s);
int64_t fused_workspace_bytes(const LayerShape &s, int64_t T);
hipError_t launch_fused_prefill(const LayerShape &s, FusedArgs a, void *workspace, hipStream_t st);
// The same 32-token-block scan on post-conv xbc (chunk_scan_fwd with a workspace of
// fused_workspace_bytes): P = 64, N = 128, bf16 activations and y.
bool chunk_scan_blocks_supported(const LayerShape &s);
hipError_t launch_block_scan(const LayerShape &s, FusedArgs a, void *workspace, hipStream_t st);

bool gated_norm_supported(int64_t width, int gs);
hipError_t launch_gated_norm(const NormArgs &a, int y_dt, int z_dt, int64_t width, int gs, hipStream_t st);

bool selective_scan_supported(const SelShape &s);
hipError_t launch_selective_scan(const SelShape &s, const SelScanArgs &a, hipStream_t st);
hipError_t launch_selective_update(const SelShape &s, const SelUpdateArgs &a, hipStream_t st);

bool scan_supported(const LayerShape &s);
hipError_t launch_chunk_scan(const LayerShape &s, const ScanArgs &a, hipStream_t st);

}  // namespace m2
