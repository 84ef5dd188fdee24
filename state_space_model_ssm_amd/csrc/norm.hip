// Gated RMSNorm of the mixer output: the "norm" tensor among the Mamba-2 mixer
// tensors of the "Nemotron-H-8B-Base-8K" record. The pages name the tensor only;
// the reading used here: with g = y * SiLU(z) (g = y without z), each group of
// `gs` consecutive channels of a row is scaled to unit root mean square,
//   out[c] = w[c] * g[c] / sqrt(mean_{c' in group} g[c']^2 + eps),
// the groups being the channels of H/G heads when gs = H*P/G.
//
// HBM bound (one read of y and z, one write): one wavefront per (row, group),
// K 4-element vectors per lane kept in registers between the sum of squares
// (a butterfly over the wavefront) and the scaling; SiLU from the hardware exp2
// and reciprocal. Rows are independent, so in-place use (out == y) is allowed.
#include "common.hpp"
#include "kernels.hpp"

namespace m2 {

template <typename YT, typename ZT, typename OT, int K, bool HasZ>
__global__ __launch_bounds__(256) void gated_norm_kernel(NormArgs a, int64_t width, int gs, int ngroups_row) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (int64_t)a.rows * ngroups_row) return;
    const int64_t row = item / ngroups_row;
    const int64_t c0 = row * width + (item % ngroups_row) * gs;
    const int cw0 = (int)((item % ngroups_row) * gs);
    // Every load (y, z and the weights) is issued before any value is used, unconditionally:
    // lanes past the group's end read its last vector and drop the values. Loads behind
    // per-lane branches were waited for one at a time.
    Raw<YT, 4> yr[K];
    Raw<ZT, 4> zr[HasZ ? K : 1];
    f32x4 wr[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = min((k * 64 + lane) * 4, gs - 4);
        yr[k].load(static_cast<const YT *>(a.y) + c0 + c);
        if constexpr (HasZ) zr[k].load(static_cast<const ZT *>(a.z) + c0 + c);
        wr[k] = *reinterpret_cast<const f32x4 *>(a.w + cw0 + c);
    }
    __builtin_amdgcn_sched_barrier(0);  // (else the compiler sinks the weight loads into the stores)
    float v[K][4];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const bool live = (k * 64 + lane) * 4 < gs;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float g = yr[k][j];
            if constexpr (HasZ) g *= silu_fast(zr[k][j]);
            v[k][j] = live ? g : 0.0f;
            ss += v[k][j] * v[k][j];
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float scale = 1.0f / sqrtf(ss / (float)gs + a.eps);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int c = (k * 64 + lane) * 4;
        if (c < gs) {
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = v[k][j] * scale * wr[k][j];
            store_k<OT, 4>(static_cast<OT *>(a.out) + c0 + c, o);
        }
    }
}

template <typename YT, typename ZT, typename OT, int K>
static void launch_gn_kz(const NormArgs &a, int64_t width, int gs, int ng, dim3 grid, hipStream_t stream) {
    if (a.z) hipLaunchKernelGGL((gated_norm_kernel<YT, ZT, OT, K, true>), grid, dim3(256), 0, stream, a, width, gs, ng);
    else hipLaunchKernelGGL((gated_norm_kernel<YT, ZT, OT, K, false>), grid, dim3(256), 0, stream, a, width, gs, ng);
}

template <typename YT, typename ZT, typename OT>
static hipError_t launch_gn_k(const NormArgs &a, int64_t width, int gs, hipStream_t stream) {
    const int ng = (int)(width / gs);
    const int64_t items = (int64_t)a.rows * ng;
    dim3 grid((unsigned)((items + 3) / 4));
    const int k = (gs + 255) / 256;
    if (k <= 1) launch_gn_kz<YT, ZT, OT, 1>(a, width, gs, ng, grid, stream);
    else if (k <= 2) launch_gn_kz<YT, ZT, OT, 2>(a, width, gs, ng, grid, stream);
    else if (k <= 4) launch_gn_kz<YT, ZT, OT, 4>(a, width, gs, ng, grid, stream);
    else if (k <= 8) launch_gn_kz<YT, ZT, OT, 8>(a, width, gs, ng, grid, stream);
    else if (k <= 16) launch_gn_kz<YT, ZT, OT, 16>(a, width, gs, ng, grid, stream);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <typename YT, typename OT>
static hipError_t launch_gn_z(const NormArgs &a, int z_dt, int64_t width, int gs, hipStream_t stream) {
    return z_dt == DT_BF16 ? launch_gn_k<YT, bf16, OT>(a, width, gs, stream)
                           : launch_gn_k<YT, float, OT>(a, width, gs, stream);
}

bool gated_norm_supported(int64_t width, int gs) {
    return gs > 0 && gs % 4 == 0 && gs <= 4096 && width % gs == 0;
}

// y and out share the output dtype; z has the activation dtype.
hipError_t launch_gated_norm(const NormArgs &a, int y_dt, int z_dt, int64_t width, int gs, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    return y_dt == DT_BF16 ? launch_gn_z<bf16, bf16>(a, z_dt, width, gs, stream)
                           : launch_gn_z<float, float>(a, z_dt, width, gs, stream);
}

}  // namespace m2
