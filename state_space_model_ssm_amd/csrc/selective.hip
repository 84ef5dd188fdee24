// Mamba-1 selective scan (the "selective_scan_fwd" kernel the trace page
// "Hybrid Mamba-Transformer MoEs hide their stalls..." names for Mamba layers;
// the recurrence is that of the Mamba paper the page cites): a diagonal state
// per (channel d, state n) with its own decay A[d][n],
//   delta = softplus(delta_raw + bias)        (or delta_raw + bias)
//   h_t[d][n] = exp(delta_t[d] A[d][n]) h_{t-1}[d][n] + delta_t[d] B_t[n] u_t[d]
//   y_t[d]    = sum_n C_t[n] h_t[d][n] + D[d] u_t[d]        (times SiLU(z_t[d]))
// with B, C shared by the channels of a group.
//
// There is no dense contraction here: per state element and token it is one
// exp and a few multiply-adds, so the bound is VALU issue (the exp runs on the
// transcendental unit), not MFMA and not HBM (u, delta, z, y are 8 bytes per
// channel and token against N = 16 state updates).
//
// Design: one workgroup per (64 channels, sequence), looping over the
// sequence's tokens in chunks (64 tokens at N = 16):
//   * staging: the chunk's u, delta, z of the workgroup's channels and B, C of
//     its group are loaded cooperatively (coalesced rows) and reduced once per
//     (token, channel) to delta, delta*u, D*u and the gate, in LDS;
//   * recurrence: each thread owns 4 states of one channel (N/4 lanes per
//     channel) in registers, A pre-scaled by log2(e) so each step is one
//     multiply, one exp2 and two fused multiply-adds per state; the partial
//     C.h sums are combined across the channel's lanes with DPP quad moves;
//   * the chunk's y tile is written to LDS and stored as coalesced rows.
// The state stays in registers for the whole sequence; only the initial and
// final states touch the pool.
#include "common.hpp"
#include "kernels.hpp"

namespace m2 {

// Sum over aligned groups of G consecutive lanes (G = 1, 2, 4), every lane of the
// group ending with the total. DPP quad permutations move values within quads of
// lanes as ordinary VALU operations (no LDS crossbar, no wait): [1,0,3,2] swaps
// neighbours, [2,3,0,1] swaps pairs.
template <int G> __device__ __forceinline__ float lane_group_sum(float v) {
    static_assert(G == 1 || G == 2 || G == 4, "lane groups of 1, 2 or 4");
    if constexpr (G >= 2)
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    if constexpr (G >= 4)
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    return v;
}

template <int N, typename AT, typename ST, typename OT>
__global__ __launch_bounds__(256) void selective_scan_kernel(SelScanArgs a, int Dc, int G) {
    constexpr int LPC = N / 4;          // lanes per channel (4 states each)
    constexpr int CH = 256 / LPC;       // channels per workgroup
    constexpr int TT = 16 * LPC;        // tokens per chunk (LDS stays below 80 KB for every N: two workgroups per CU)
    constexpr int CS = CH + 4;          // row stride of the per-token channel arrays (floats)
    constexpr float LOG2E = 1.4426950408889634f;
    static_assert(N % 4 == 0 && LPC >= 1 && LPC <= 16, "dstate must be a multiple of 4, at most 64");

    constexpr int TS = TT + 4;          // row stride of the per-channel token arrays (floats)
    // delta and delta * u per channel, tokens contiguous (one 16-byte read gives a lane
    // 4 tokens of its channel); the recurrence overwrites delta * u with the C.h sums
    __shared__ __attribute__((aligned(16))) float sDl[CH][TS];
    __shared__ __attribute__((aligned(16))) float sDu[CH][TS];
    __shared__ __attribute__((aligned(16))) float sSk[TT][CS];   // D * u
    __shared__ __attribute__((aligned(16))) float sGt[TT][CS];   // SiLU(z) or 1
    __shared__ __attribute__((aligned(16))) float sB[TT][N];
    __shared__ __attribute__((aligned(16))) float sC[TT][N];

    const int tid = threadIdx.x;
    __shared__ int sSeq;
    const int cblk = blockIdx.x, seq = seq_longest_first(a.cu, a.nseq, blockIdx.y, tid, 256, &sSeq);
    const int c0 = cblk * CH;                 // first channel of the workgroup
    const int g = c0 / (Dc / G);              // its group (CH divides Dc / G)
    const int64_t start = a.cu[seq], end = a.cu[seq + 1];
    const int slot = pool_slot(a.idx[seq], a.num_slots, a.err, cblk == 0 && tid == 0);
    OT *y = static_cast<OT *>(a.y);

    if (slot < 0) {
        for (int64_t i = tid; i < (end - start) * CH; i += 256) {
            const int64_t t = start + i / CH;
            Io<OT>::put(y, t * Dc + c0 + (int)(i % CH), 0.0f);
        }
        return;
    }

    // recurrence role: channel cl of the workgroup, states [n0, n0 + 4)
    const int cl = tid / LPC, sg = tid % LPC, n0 = 4 * sg;
    const int ch = c0 + cl;
    float A2[4], h[4];
    load_k<float, 4>(a.A + (int64_t)ch * N + n0, A2);
#pragma unroll
    for (int j = 0; j < 4; ++j) A2[j] *= LOG2E;
    ST *hp = static_cast<ST *>(a.pool) + ((int64_t)slot * Dc + ch) * N + n0;
    const bool init = a.has_init && a.has_init[seq];
    if (init) load_k<ST, 4>(hp, h);
    else
#pragma unroll
        for (int j = 0; j < 4; ++j) h[j] = 0.0f;

    // staging role: token row sr, channels [4 * sc, 4 * sc + 4) of the workgroup
    constexpr int SC = CH / 4;             // 4-channel pieces per token row
    constexpr int SR = 256 / SC;           // token rows per staging pass
    const int sc = tid % SC, sr0 = tid / SC;
    float bias[4], Dv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        bias[j] = a.delta_bias ? a.delta_bias[c0 + 4 * sc + j] : 0.0f;
        Dv[j] = a.D ? a.D[c0 + 4 * sc + j] : 0.0f;
    }
    const AT *uin = static_cast<const AT *>(a.u);
    const AT *din = static_cast<const AT *>(a.delta);
    const AT *zin = static_cast<const AT *>(a.z);
    const AT *bin = static_cast<const AT *>(a.B);
    const AT *cin = static_cast<const AT *>(a.C);

    // The next chunk's rows are loaded into registers while the current chunk
    // runs its recurrence (rows clamped into the sequence: every load is
    // unconditional; rows past the chunk are zeroed when staged).
    constexpr int RPT = TT / SR;                 // staged token rows per thread
    constexpr int KBC = TT * (N / 4) * 2;        // 4-element pieces of the chunk's B | C
    constexpr int BCP = (KBC + 255) / 256;
    Raw<AT, 4> ur[RPT], dr[RPT], zr[RPT], bcr[BCP];
    auto prefetch = [&](int64_t t0) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int64_t row = t0 + sr0 + i * SR < end ? t0 + sr0 + i * SR : end - 1;
            const int64_t off = row * Dc + c0 + 4 * sc;
            ur[i].load(uin + off);
            dr[i].load(din + off);
        }
        if (zin)
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int64_t row = t0 + sr0 + i * SR < end ? t0 + sr0 + i * SR : end - 1;
                zr[i].load(zin + row * Dc + c0 + 4 * sc);
            }
#pragma unroll
        for (int i = 0; i < BCP; ++i) {
            const int k = min(tid + i * 256, KBC - 1);
            const int which = k / (TT * (N / 4)), rem = k % (TT * (N / 4)), r = rem / (N / 4), q4 = rem % (N / 4);
            const int64_t row = t0 + r < end ? t0 + r : end - 1;
            bcr[i].load((which ? cin : bin) + (row * G + g) * N + 4 * q4);
        }
    };
    if (start < end) prefetch(start);

    for (int64_t t0 = start; t0 < end; t0 += TT) {
        const int cl_n = (int)((end - t0) < TT ? (end - t0) : TT);
        // ---------------- stage the chunk (from the prefetched rows)
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = sr0 + i * SR;
            float dl[4], du[4], sk[4], gt[4];
            const bool ok = r < cl_n;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float uu = ur[i][j];
                float v = dr[i][j] + bias[j];
                if (a.delta_softplus) v = softplus_fast(v);
                dl[j] = ok ? v : 0.0f;
                du[j] = ok ? v * uu : 0.0f;
                sk[j] = ok ? Dv[j] * uu : 0.0f;
                gt[j] = ok ? (zin ? silu_fast(zr[i][j]) : 1.0f) : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sDl[4 * sc + j][r] = dl[j];
                sDu[4 * sc + j][r] = du[j];
            }
            *reinterpret_cast<f32x4 *>(&sSk[r][4 * sc]) = f32x4{sk[0], sk[1], sk[2], sk[3]};
            *reinterpret_cast<f32x4 *>(&sGt[r][4 * sc]) = f32x4{gt[0], gt[1], gt[2], gt[3]};
        }
#pragma unroll
        for (int i = 0; i < BCP; ++i) {
            const int k = tid + i * 256;
            if (k < KBC) {
                const int which = k / (TT * (N / 4)), rem = k % (TT * (N / 4)), r = rem / (N / 4), q4 = rem % (N / 4);
                const bool ok = r < cl_n;
                const f32x4 v = {ok ? bcr[i][0] : 0.0f, ok ? bcr[i][1] : 0.0f, ok ? bcr[i][2] : 0.0f, ok ? bcr[i][3] : 0.0f};
                *reinterpret_cast<f32x4 *>(which ? &sC[r][4 * q4] : &sB[r][4 * q4]) = v;
            }
        }
        __syncthreads();
        prefetch(t0 + TT < end ? t0 + TT : t0);  // the last chunk reloads itself (unused)

        // ---------------- recurrence over the chunk, 4 tokens per step (tokens past the
        // chunk's end were staged with delta = delta * u = 0: they leave h unchanged)
        for (int t = 0; t < cl_n; t += 4) {
            const f32x4 dl4 = *reinterpret_cast<const f32x4 *>(&sDl[cl][t]);
            const f32x4 du4 = *reinterpret_cast<const f32x4 *>(&sDu[cl][t]);
            float ys[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&sB[t + u][n0]);
                const f32x4 c4 = *reinterpret_cast<const f32x4 *>(&sC[t + u][n0]);
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // explicit FMAs (the one-token kernel below rounds exactly alike); the
                    // decayed state is formed first, measured faster than fusing the decay
                    h[j] = fmaf(du4[u], b4[j], __builtin_amdgcn_exp2f(dl4[u] * A2[j]) * h[j]);
                    acc = fmaf(c4[j], h[j], acc);
                }
                ys[u] = lane_group_sum<LPC>(acc);  // every lane of the channel holds the sum
            }
            // C.h of the 4 tokens over delta * u (already read); the channel's lanes write equal values
            *reinterpret_cast<f32x4 *>(&sDu[cl][t]) = f32x4{ys[0], ys[1], ys[2], ys[3]};
        }
        __syncthreads();

        // ---------------- store the y tile (rows of CH channels): (C.h + D u) * gate
        for (int r = sr0; r < cl_n; r += SR) {
            const f32x4 sk = *reinterpret_cast<const f32x4 *>(&sSk[r][4 * sc]);
            const f32x4 gt = *reinterpret_cast<const f32x4 *>(&sGt[r][4 * sc]);
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = (sDu[4 * sc + j][r] + sk[j]) * gt[j];
            store_k<OT, 4>(y + (t0 + r) * Dc + c0 + 4 * sc, o);
        }
        __syncthreads();
    }
    Io<ST>::put(hp, 0, h[0]);
    Io<ST>::put(hp, 1, h[1]);
    Io<ST>::put(hp, 2, h[2]);
    Io<ST>::put(hp, 3, h[3]);
}

// One token per row, the state read and written in place at the row's slot
// (the decode form of the same recurrence). Each thread owns 4 states of one
// channel; the per-(token, channel) quantities and each state update use the
// same arithmetic as the scan kernel above, so T single steps reproduce a
// T-token scan bit for bit on an fp32 pool.
template <int N, typename AT, typename ST, typename OT>
__global__ __launch_bounds__(256) void selective_update_kernel(SelUpdateArgs a, int Dc, int G) {
    constexpr int LPC = N / 4;
    constexpr int CH = 256 / LPC;
    constexpr float LOG2E = 1.4426950408889634f;
    const int tid = threadIdx.x;
    const int row = blockIdx.y;
    const int cl = tid / LPC, sg = tid % LPC, n0 = 4 * sg;
    const int ch = blockIdx.x * CH + cl;
    const int g = (blockIdx.x * CH) / (Dc / G);
    const int slot = pool_slot(a.idx[row], a.num_slots, a.err, blockIdx.x == 0 && tid == 0);
    OT *y = static_cast<OT *>(a.y);
    if (slot < 0) {
        if (sg == 0) Io<OT>::put(y, (int64_t)row * Dc + ch, 0.0f);
        return;
    }
    const int64_t ro = (int64_t)row * Dc + ch;
    ST *hp = static_cast<ST *>(a.pool) + ((int64_t)slot * Dc + ch) * N + n0;
    float h[4], A2[4], b4[4], c4[4];
    load_k<ST, 4>(hp, h);
    load_k<float, 4>(a.A + (int64_t)ch * N + n0, A2);
    load_k<AT, 4>(static_cast<const AT *>(a.B) + ((int64_t)row * G + g) * N + n0, b4);
    load_k<AT, 4>(static_cast<const AT *>(a.C) + ((int64_t)row * G + g) * N + n0, c4);
    const float uu = (float)static_cast<const AT *>(a.u)[ro];
    // D and z are read here with the other loads, unconditionally (from u when absent, the
    // value then unused): read after the state update they cost two more round trips
    const float Dv = (a.D ? a.D : a.A)[a.D ? ch : 0];
    const float zv = (float)static_cast<const AT *>(a.z ? a.z : a.u)[ro];
    float dl = (float)static_cast<const AT *>(a.delta)[ro] + (a.delta_bias ? a.delta_bias[ch] : 0.0f);
    if (a.delta_softplus) dl = softplus_fast(dl);
    const float du = dl * uu;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = fmaf(du, b4[j], __builtin_amdgcn_exp2f(dl * (A2[j] * LOG2E)) * h[j]);
        acc = fmaf(c4[j], h[j], acc);
    }
    acc = lane_group_sum<LPC>(acc);
    store_k<ST, 4>(hp, h);
    if (sg == 0) {
        const float sk = a.D ? Dv * uu : 0.0f;
        const float gt = a.z ? silu_fast(zv) : 1.0f;
        Io<OT>::put(y, ro, (acc + sk) * gt);
    }
}

template <int N, typename AT, typename ST, typename OT>
static hipError_t launch_seu_t(const SelShape &s, const SelUpdateArgs &a, hipStream_t stream) {
    constexpr int CH = 256 / (N / 4);
    dim3 grid(s.Dc / CH, a.batch);
    hipLaunchKernelGGL((selective_update_kernel<N, AT, ST, OT>), grid, dim3(256), 0, stream, a, s.Dc, s.G);
    return hipGetLastError();
}

template <int N, typename AT, typename ST>
static hipError_t launch_seu_o(const SelShape &s, const SelUpdateArgs &a, hipStream_t stream) {
    return s.out_dt == DT_BF16 ? launch_seu_t<N, AT, ST, bf16>(s, a, stream)
                               : launch_seu_t<N, AT, ST, float>(s, a, stream);
}

template <int N, typename AT>
static hipError_t launch_seu_s(const SelShape &s, const SelUpdateArgs &a, hipStream_t stream) {
    return s.state_dt == DT_BF16 ? launch_seu_o<N, AT, bf16>(s, a, stream) : launch_seu_o<N, AT, float>(s, a, stream);
}

template <int N>
static hipError_t launch_seu_a(const SelShape &s, const SelUpdateArgs &a, hipStream_t stream) {
    return s.act_dt == DT_BF16 ? launch_seu_s<N, bf16>(s, a, stream) : launch_seu_s<N, float>(s, a, stream);
}

hipError_t launch_selective_update(const SelShape &s, const SelUpdateArgs &a, hipStream_t stream) {
    if (a.batch == 0) return hipSuccess;
    switch (s.N) {
        case 4: return launch_seu_a<4>(s, a, stream);
        case 8: return launch_seu_a<8>(s, a, stream);
        case 16: return launch_seu_a<16>(s, a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int N, typename AT, typename ST, typename OT>
static hipError_t launch_sel_t(const SelShape &s, const SelScanArgs &a, hipStream_t stream) {
    constexpr int CH = 256 / (N / 4);
    dim3 grid(s.Dc / CH, a.nseq);
    hipLaunchKernelGGL((selective_scan_kernel<N, AT, ST, OT>), grid, dim3(256), 0, stream, a, s.Dc, s.G);
    return hipGetLastError();
}

template <int N, typename AT, typename ST>
static hipError_t launch_sel_o(const SelShape &s, const SelScanArgs &a, hipStream_t stream) {
    return s.out_dt == DT_BF16 ? launch_sel_t<N, AT, ST, bf16>(s, a, stream)
                               : launch_sel_t<N, AT, ST, float>(s, a, stream);
}

template <int N, typename AT>
static hipError_t launch_sel_s(const SelShape &s, const SelScanArgs &a, hipStream_t stream) {
    return s.state_dt == DT_BF16 ? launch_sel_o<N, AT, bf16>(s, a, stream) : launch_sel_o<N, AT, float>(s, a, stream);
}

template <int N>
static hipError_t launch_sel_a(const SelShape &s, const SelScanArgs &a, hipStream_t stream) {
    return s.act_dt == DT_BF16 ? launch_sel_s<N, bf16>(s, a, stream) : launch_sel_s<N, float>(s, a, stream);
}

bool selective_scan_supported(const SelShape &s) {
    if (!(s.N == 4 || s.N == 8 || s.N == 16)) return false;
    const int ch = 256 / (s.N / 4);
    return s.G > 0 && s.Dc % s.G == 0 && (s.Dc / s.G) % ch == 0;
}

hipError_t launch_selective_scan(const SelShape &s, const SelScanArgs &a, hipStream_t stream) {
    if (a.nseq == 0) return hipSuccess;
    switch (s.N) {
        case 4: return launch_sel_a<4>(s, a, stream);
        case 8: return launch_sel_a<8>(s, a, stream);
        case 16: return launch_sel_a<16>(s, a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace m2
