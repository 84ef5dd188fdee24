// MFMA fragment helpers and the token / head orderings shared by the chunked
// scan kernels (v_mfma_f32_16x16x32_bf16: A rows and B columns on lane & 15,
// eight consecutive k per lane starting at (lane >> 4) * 8; D columns on
// lane & 15, rows (lane >> 4) * 4 + r).
#pragma once
#include "common.hpp"

namespace m2 {

__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split8(const float *v, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const bf16 h = f32_to_bf16(v[j]);
        hi[j] = h;
        lo[j] = f32_to_bf16(v[j] - (float)h);
    }
}

__device__ __forceinline__ bf16x8 cvt8(const float *v) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = f32_to_bf16(v[j]);
    return r;
}

// Position, inside a 32-token block, of token u = 16b + 4q + r: q*8 + b*4 + r.
// A lane of quad q then reads its 8 k-values (tokens 4q..4q+3 and 16+4q..)
// as one contiguous run, matching two stacked 16x16 accumulator tiles.
__device__ __forceinline__ int perm32(int u) { return ((u >> 2) & 3) * 8 + (u >> 4) * 4 + (u & 3); }
__device__ __forceinline__ int pos_of(int s) { return (s & ~31) + perm32(s & 31); }
__device__ __forceinline__ int tok_of_slot(int q, int j) { return j < 4 ? 4 * q + j : 16 + 4 * q + (j - 4); }

// Workgroups are dispatched round-robin over the 8 XCDs by linear id, and each
// XCD has its own L2. Remap blockIdx.x so consecutive heads (which share a
// group's B/C channels) run on the same XCD: XCD x gets heads
// [x*H/8, (x+1)*H/8), i.e. whole groups at H/G = 16. Without this each group's
// B/C stream is fetched from HBM by every XCD (measured 3x the algorithmic
// read traffic of the scan).
__device__ __forceinline__ int xcd_head(int bx, int H) {
    constexpr int kXcds = 8;
    return (H % kXcds == 0) ? (bx % kXcds) * (H / kXcds) + bx / kXcds : bx;
}

__device__ __forceinline__ void ld8f(const float *p, float *v) {
    Io<float>::load(p, v);
    Io<float>::load(p + 4, v + 4);
}

// t-tile handled by wave w (i-th of its tiles). With 8 tiles on 8 waves, waves w
// and w+4 (same SIMD) take tiles whose causal work sums to a constant.
template <int TL, int NW>
__device__ __forceinline__ int ttile_of(int w, int i) {
    if constexpr (TL == 8 && NW == 8) return w < 4 ? w : 11 - w;
    return w + i * NW;
}

}  // namespace m2
