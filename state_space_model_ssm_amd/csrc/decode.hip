// One-token decode kernels for gfx950: the selective state update, which reads
// and writes the SSM pool in place at each row's slot, and the conv1d update,
// which shifts the slot's cached raw inputs in place.
//
// The in-place, index-addressed form is the one the vllm.cpp issue "NemotronH
// runs the PREFILL mamba kernels at decode" asks for (section "The
// divergence"); its cost table ("Cost, at T=1, chunk_size=128, nchunks=1")
// gives the target: one launch, no allocation, no memset, no scratch.
//
// State update, per (row, head): the [P][N] state tile (N fastest) is streamed
// once from HBM and written back once. It is HBM bound (about 5 flops per
// state element), so the layout work is all about the stream:
//   * each lane owns 16 contiguous bytes of one p-row (8 bf16 or 4 fp32
//     values of n); kLpr = N / kVec lanes cover a row, 256 / kLpr rows are in
//     flight per pass, and ITERS passes are issued before any use so that a
//     workgroup keeps ITERS x 4 KiB of loads outstanding (two passes measured
//     best on MI355X: more, smaller workgroups keep the memory pipes busier);
//   * the state is read and written with nontemporal 16-byte accesses: each
//     tile is touched once per step, so it should not evict reusable lines
//     (measured: 5.0 -> 6.0 TB/s on the 256-row bf16 workload);
//   * y[p] = sum_n C[n] h[p][n] is a DPP window sum over the kLpr lanes of a row,
//     left in the row's last lane;
//   * B and C of the row's group and the per-head scalars are read once per
//     lane (they hit L2: the 16 heads of a group share them);
//   * a head's tile is split across `psplit` workgroups when rows x heads alone
//     would not fill the 256 CUs.
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace m2 {

template <typename ST, typename XT, typename AT, int N, int ITERS>
__global__ __launch_bounds__(256) void state_update_kernel(StateUpdateArgs a, int H, int P, int G, int out_dt,
                                                           int psplit) {
    constexpr int kVec = Io<ST>::kVec;
    constexpr int kLpr = N / kVec;   // lanes per p-row
    constexpr int kRpi = 256 / kLpr; // p-rows per pass
    static_assert(kLpr >= 1 && kLpr <= 64 && (kLpr & (kLpr - 1)) == 0, "row must fit a wavefront");

    const int tid = threadIdx.x;
    const int head = blockIdx.x / psplit;
    const int pblk = blockIdx.x - head * psplit;
    const int row = blockIdx.y;
    const int lr = tid & (kLpr - 1);
    const int r = tid / kLpr;
    const int n0 = lr * kVec;
    const int64_t HP = (int64_t)H * P;
    const int64_t cdim = HP + 2LL * G * N;
    const int p_first = pblk * kRpi * ITERS + r;
    const int64_t yrow = (int64_t)row * HP + (int64_t)head * P;

    const int slot = pool_slot(a.idx[row], a.num_slots, a.err, blockIdx.x == 0 && tid == 0);
    if (slot < 0) {  // padding row: y = 0, no state access
        if (lr == 0) {
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const int p = p_first + it * kRpi;
                if (p < P) st(a.y, out_dt, yrow + p, 0.0f);
            }
        }
        return;
    }

    // All loads are unconditional (rows past P are clamped to a valid row and
    // their results dropped) so the compiler issues them back to back instead
    // of waiting on each one behind a branch; only the stores are guarded.
    ST *tile = static_cast<ST *>(a.pool) + ((int64_t)slot * H + head) * (int64_t)P * N;
    const XT *xrow = static_cast<const XT *>(a.xbc) + (int64_t)row * cdim;
    const int g = head / (H / G);
    float Bv[kVec], Cv[kVec];
    load_k<XT, kVec>(xrow + HP + (int64_t)g * N + n0, Bv);
    load_k<XT, kVec>(xrow + HP + (int64_t)G * N + (int64_t)g * N + n0, Cv);
    const float dt_raw = (float)static_cast<const AT *>(a.dt_raw)[(int64_t)row * H + head];
    // without z, read the (valid) dt_raw array instead and ignore the value
    const AT *zsrc = a.z ? static_cast<const AT *>(a.z) : static_cast<const AT *>(a.dt_raw);
    const int64_t zoff = a.z ? yrow : 0;
    float h[ITERS][kVec], xv[ITERS], zg[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int p = min(p_first + it * kRpi, P - 1);
        nt_load16<ST>(tile + (int64_t)p * N + n0, h[it]);
        xv[it] = (float)xrow[(int64_t)head * P + p];
        zg[it] = (float)zsrc[zoff + (a.z ? p : 0)];
    }
    const float dt = softplus_f(dt_raw + a.dt_bias[head]);
    const float decay = expf(dt * -expf(a.A_log[head]));
    const float Dh = a.D[head];

#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int p = p_first + it * kRpi;
        const float dx = dt * xv[it];
        float acc = 0.0f;
        float out[kVec];
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const float s = fmaf(decay, h[it][j], dx * Bv[j]);  // explicit: the multi-token kernel rounds alike
            out[j] = s;
            acc = fmaf(Cv[j], s, acc);
        }
        if (p < P) nt_store16<ST>(tile + (int64_t)p * N + n0, out);
        acc = group_sum_last<kLpr>(acc);
        if (lr == kLpr - 1 && p < P) {
            float yv = fmaf(Dh, xv[it], acc);
            if (a.z) yv *= silu_f(zg[it]);
            st(a.y, out_dt, yrow + p, yv);
        }
    }
}

template <typename ST, typename XT, int N, int ITERS>
static hipError_t launch_su(const LayerShape &s, const StateUpdateArgs &a, hipStream_t stream, int rows_needed) {
    const int psplit = (rows_needed + ITERS - 1) / ITERS;
    dim3 grid(s.H * psplit, a.batch);
    if (s.act_dt == DT_BF16)
        hipLaunchKernelGGL((state_update_kernel<ST, XT, bf16, N, ITERS>), grid, dim3(256), 0, stream, a, s.H, s.P, s.G,
                           s.out_dt, psplit);
    else
        hipLaunchKernelGGL((state_update_kernel<ST, XT, float, N, ITERS>), grid, dim3(256), 0, stream, a, s.H, s.P,
                           s.G, s.out_dt, psplit);
    return hipGetLastError();
}

template <typename ST, typename XT, int N>
static hipError_t dispatch_su_iters(const LayerShape &s, const StateUpdateArgs &a, hipStream_t stream) {
    constexpr int kRpi = 256 / (N / Io<ST>::kVec);
    const int rows_needed = (s.P + kRpi - 1) / kRpi;  // passes that cover one head tile
    // Two passes per workgroup (8 KiB of state in flight) when that still leaves
    // >= 2048 workgroups (8 per CU); one pass otherwise. Small batches (under 8192
    // workgroups of two passes, e.g. 16 rows at 8B dims) take four passes while that
    // still leaves 2048: 0.804 -> 0.781 ms per step of the 48-layer stack at 16 rows.
    int iters = 1;
    if (rows_needed >= 2 && (int64_t)a.batch * s.H * ((rows_needed + 1) / 2) >= 2048) iters = 2;
    if (rows_needed >= 4 && (int64_t)a.batch * s.H * ((rows_needed + 3) / 4) >= 2048 &&
        (int64_t)a.batch * s.H * ((rows_needed + 1) / 2) < 8192) iters = 4;
    return iters == 4 ? launch_su<ST, XT, N, 4>(s, a, stream, rows_needed)
         : iters == 2 ? launch_su<ST, XT, N, 2>(s, a, stream, rows_needed)
                      : launch_su<ST, XT, N, 1>(s, a, stream, rows_needed);
}

template <typename ST, typename XT>
static hipError_t dispatch_su_n(const LayerShape &s, const StateUpdateArgs &a, hipStream_t stream) {
    switch (s.N) {
        case 16: return dispatch_su_iters<ST, XT, 16>(s, a, stream);
        case 64: return dispatch_su_iters<ST, XT, 64>(s, a, stream);
        case 128: return dispatch_su_iters<ST, XT, 128>(s, a, stream);
        default: return hipErrorInvalidValue;
    }
}

bool state_update_supported(const LayerShape &s) { return s.N == 16 || s.N == 64 || s.N == 128; }

hipError_t launch_state_update(const LayerShape &s, const StateUpdateArgs &a, hipStream_t stream) {
    if (a.batch == 0) return hipSuccess;
    if (s.state_dt == DT_BF16) {
        return s.xbc_dt == DT_BF16 ? dispatch_su_n<bf16, bf16>(s, a, stream) : dispatch_su_n<bf16, float>(s, a, stream);
    }
    return s.xbc_dt == DT_BF16 ? dispatch_su_n<float, bf16>(s, a, stream) : dispatch_su_n<float, float>(s, a, stream);
}

// ------------------------------------------------------- multi-token state update
// T tokens per row (drafted tokens being verified, or any short run of decode
// tokens): the row's state is read once from its source slot, kept in registers
// through the T steps (so it is rounded to the pool dtype only where written),
// and after step t written to dst[row][t] when that slot is >= 0 (a per-step
// snapshot the caller can roll back to); with no dst table only the final state
// is written, in place. Per step and lane the inputs are the same handful of
// values as the one-token update.
// K consecutive elements of T kept as their raw bits after one load of 2, 4, 8 or
// 16 bytes (widened where used, so the load is not waited for at once).
template <typename T, int K> struct RawRow {
    static constexpr int kB = K * (int)sizeof(T);
    static_assert(kB == 2 || kB == 4 || kB == 8 || kB == 16, "RawRow: 2, 4, 8 or 16 bytes");
    uint32_t w[(kB + 3) / 4];
    __device__ __forceinline__ void load(const T *p) {
        if constexpr (kB == 16) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else if constexpr (kB == 8) {
            const uint2 v = *reinterpret_cast<const uint2 *>(p);
            w[0] = v.x; w[1] = v.y;
        } else if constexpr (kB == 4) {
            w[0] = *reinterpret_cast<const uint32_t *>(p);
        } else {
            w[0] = *reinterpret_cast<const unsigned short *>(p);
        }
    }
    __device__ __forceinline__ float operator[](int i) const {
        if constexpr (sizeof(T) == 4) return __uint_as_float(w[i]);
        else return __uint_as_float((i & 1) ? (w[i >> 1] & 0xffff0000u) : (w[i >> 1] << 16));
    }
};

// K consecutive outputs in one store (y of a thread's K rows)
// (i: a wave-uniform element index, l: the lane's element offset from it, kept 32-bit so
// that the store takes the scalar-base form)
template <int K> __device__ __forceinline__ void store_row(void *p, int dt, int64_t i, uint32_t l, const float *v) {
    if (dt == DT_BF16) {
        bf16 *q = reinterpret_cast<bf16 *>(static_cast<char *>(p) + i * 2 + 2u * l);
        if constexpr (K == 4) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            *reinterpret_cast<bf16x4 *>(q) = bf16x4{f32_to_bf16(v[0]), f32_to_bf16(v[1]), f32_to_bf16(v[2]), f32_to_bf16(v[3])};
        } else if constexpr (K == 2) {
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            *reinterpret_cast<bf16x2 *>(q) = bf16x2{f32_to_bf16(v[0]), f32_to_bf16(v[1])};
        } else {
            *q = f32_to_bf16(v[0]);
        }
    } else {
        float *q = reinterpret_cast<float *>(static_cast<char *>(p) + i * 4 + 4u * l);
        if constexpr (K == 4) *reinterpret_cast<f32x4 *>(q) = f32x4{v[0], v[1], v[2], v[3]};
        else if constexpr (K == 2) *reinterpret_cast<float2 *>(q) = float2{v[0], v[1]};
        else *q = v[0];
    }
}

// T tokens per row with the state in registers. kLpr lanes cover one p-row's N
// values (kVec each) and each group of kLpr lanes holds ITERS p-rows:
//   CONSEC (final state only): rows p0 .. p0 + ITERS - 1, so x of a token is one
//     vector load and its y leaves the group in one store;
//   otherwise (a snapshot after every token): rows base + g + it * kGrp, so one
//     store instruction of a wave writes consecutive rows (1 KiB contiguous at
//     N = 128 bf16); measured faster for the snapshot stream, slower without it.
// z is a template parameter (its registers only where it is used). The final-state
// form without z on bf16 state and post-conv input asks for four waves per SIMD: six
// spilled registers, measured 3 % faster than three waves without; the other forms
// would spill more.
template <typename ST, typename XT, typename AT, int N, int ITERS, bool CONSEC, bool HasZ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(
    CONSEC && !HasZ && sizeof(ST) == 2 && sizeof(XT) == 2 ? 4 : 1))) void
state_update_multi_kernel(MultiStepArgs a, int H, int P, int G, int out_dt, int psplit) {
    constexpr int kVec = Io<ST>::kVec;
    constexpr int kLpr = N / kVec;
    constexpr int kGrp = 256 / kLpr;  // row groups per workgroup
    constexpr int XK = CONSEC ? ITERS : 1, XI = CONSEC ? 1 : ITERS;  // x / z: XI loads of XK rows
    const int tid = threadIdx.x;
    const int head = blockIdx.x / psplit;
    const int pblk = blockIdx.x - head * psplit;
    const int row = blockIdx.y;
    const int lr = tid & (kLpr - 1);
    const int grp = tid / kLpr;
    const int n0 = lr * kVec;
    // (P % 4 == 0 and ITERS | 4: a consecutive group is wholly inside P or outside it)
    auto prow = [&](int it) { return CONSEC ? (pblk * kGrp + grp) * ITERS + it : pblk * kGrp * ITERS + grp + it * kGrp; };
    int pr[ITERS];  // rows for loads, clamped into the tile; stores are guarded by prow(it) < P
#pragma unroll
    for (int it = 0; it < ITERS; ++it) pr[it] = min(prow(it), P - 1);
    if constexpr (CONSEC) {
        if (prow(0) >= P)
#pragma unroll
            for (int it = 0; it < ITERS; ++it) pr[it] = P - ITERS + it;
    }
    const bool ylane = lr == kLpr - 1;
    // Final-state form with four rows per 16-lane group: y sums reduce-scattered over the group
    // (row16_sum4_scatter) instead of four window sums; the lanes 4k (qlead) store row k's y.
    constexpr bool kScatter = CONSEC && kLpr == 16 && ITERS == 4;
    const bool bit3 = lr & 8, bit2 = lr & 4, qlead = (lr & 3) == 0;
    const int64_t HP = (int64_t)H * P;
    const int64_t cdim = HP + 2LL * G * N;
    const int T = a.T;
    const int64_t ybase = (int64_t)row * T * HP + (int64_t)head * P;
    // y of a token: CONSEC, one store of the group's ITERS rows; otherwise one per row
    auto store_y = [&](int t, const float *yv) {
        if (!ylane) return;
        if constexpr (CONSEC) {
            if (prow(0) < P) store_row<ITERS>(a.y, out_dt, ybase, (uint32_t)t * (uint32_t)HP + prow(0), yv);
        } else {
#pragma unroll
            for (int it = 0; it < ITERS; ++it)
                if (prow(it) < P) store_row<1>(a.y, out_dt, ybase, (uint32_t)t * (uint32_t)HP + prow(it), &yv[it]);
        }
    };
    const int src = pool_slot(a.src[row], a.num_slots, a.err, blockIdx.x == 0 && tid == 0);
    if (src < 0) {  // padding row: y = 0, no state access
        if (ylane)
            for (int it = 0; it < ITERS; ++it)
                if (prow(it) < P)
                    for (int t = 0; t < T; ++t) st(a.y, out_dt, ybase + (int64_t)t * HP + prow(it), 0.0f);
        return;
    }
    const int g = head / (H / G);
    const float A = -expf(a.A_log[head]);
    const float dtb = a.dt_bias[head];
    const float Dh = a.D[head];

    // Per block of TB tokens: B and C are loaded once per workgroup into LDS (every
    // p-row of the head uses the same vectors: re-reading them per row would move
    // TB * 2 * N values per row through L1/L2 against N state values); lane u of
    // wave 0 forms dt and the decay of token t0 + u (library softplus and exp, as the
    // one-token kernel: once per workgroup, not once per wave), read by every wave
    // from LDS. The first block's loads are issued before the state's, so its
    // staging and dt overlap the state's latency.
    constexpr int TB = 4;
    constexpr int NT4 = TB * 2 * N / 4;  // 4-element pieces of the block's B|C
    static_assert(NT4 <= 256, "one B|C piece per thread");
    __shared__ __attribute__((aligned(16))) float sBC[TB][2][N];
    __shared__ float sDt[2][TB];  // dt and decay of the block's tokens, formed by wave 0 alone
    Raw<XT, 4> bcr;
    RawRow<XT, XK> xr[TB][XI];
    RawRow<AT, XK> zr[HasZ ? TB : 1][HasZ ? XI : 1];
    float dr = 0.0f;
    // Addresses: the row's (or the slot's) base, wave-uniform in scalar registers, plus a
    // 32-bit byte offset per lane that includes the token (the scalar-base load and store
    // form; the boundary keeps T x Cdim and P x N small enough for the offsets). With 64-bit
    // address arithmetic per lane and access, which the compiler also makes of a 64-bit
    // token term added to a loop-invariant lane offset, addresses cost a sixth of the
    // kernel's VALU instructions.
    constexpr uint32_t XS = sizeof(XT), AS = sizeof(AT), SS = sizeof(ST);
    uint32_t xoff[XI], soff[ITERS];
#pragma unroll
    for (int i = 0; i < XI; ++i) xoff[i] = (uint32_t)pr[i] * XS;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) soff[it] = ((uint32_t)pr[it] * N + n0) * SS;
    auto tk = [&](int t) { return (uint32_t)min(t, T - 1); };  // token t of the row, clamped to its last
    const char *xrow_b = static_cast<const char *>(a.xbc) + ((int64_t)row * T * cdim + (int64_t)head * P) * XS;
    const char *pool_b = static_cast<const char *>(a.pool) + (int64_t)head * P * N * SS;
    auto xval = [&](int u, int it) {
        if constexpr (CONSEC) return xr[u][0][it];
        else return xr[u][it][0];
    };
    auto zval = [&](int u, int it) {
        if constexpr (!HasZ) return 1.0f;
        else if constexpr (CONSEC) return zr[u][0][it];
        else return zr[u][it][0];
    };
    auto load_block = [&](int t0) {
        if (tid < NT4) {
            const int u = tid / (N / 2), rem = tid % (N / 2), which = rem / (N / 4), n4 = rem % (N / 4);
            const char *bc_b = static_cast<const char *>(a.xbc) + ((int64_t)row * T * cdim + HP + (int64_t)g * N) * XS;
            bcr.load(reinterpret_cast<const XT *>(bc_b + (tk(t0 + u) * (uint32_t)cdim + which * G * N + 4 * n4) * XS));
        }
#pragma unroll
        for (int u = 0; u < TB; ++u)
#pragma unroll
            for (int i = 0; i < XI; ++i)
                xr[u][i].load(reinterpret_cast<const XT *>(xrow_b + (tk(t0 + u) * (uint32_t)cdim * XS + xoff[i])));
        if constexpr (HasZ)
#pragma unroll
            for (int u = 0; u < TB; ++u)
#pragma unroll
                for (int i = 0; i < XI; ++i)
                    zr[u][i].load(reinterpret_cast<const AT *>(static_cast<const char *>(a.z) + ybase * AS +
                                                                (tk(t0 + u) * (uint32_t)HP + pr[i]) * AS));
        const int u = (tid & 63) & (TB - 1);
        dr = (float)*reinterpret_cast<const AT *>(static_cast<const char *>(a.dt_raw) + ((int64_t)row * T * H + head) * AS +
                                                  tk(t0 + u) * (uint32_t)H * AS);
    };
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int t_stage = 0;  // first token of the block being staged
    auto stage_block = [&]() {
        if (tid < NT4) {
            const int u = tid / (N / 2), rem = tid % (N / 2), which = rem / (N / 4), n4 = rem % (N / 4);
            *reinterpret_cast<f32x4 *>(&sBC[u][which][4 * n4]) = f32x4{bcr[0], bcr[1], bcr[2], bcr[3]};
        }
        if (wave == 0) {  // the scalars of the block's tokens once per workgroup, not once per wave
            const float dt_l = softplus_f(dr + dtb);
            const float dec_l = expf(dt_l * A);
            // tokens past T (a last block shorter than TB) take dt = 0 and decay = 1: the state
            // update then gives the state back unchanged, and their y is not stored
            const bool live = t_stage + (tid & 63) < T;
            if ((tid & 63) < TB) {
                sDt[0][tid & 63] = live ? dt_l : 0.0f;
                sDt[1][tid & 63] = live ? dec_l : 1.0f;
            }
        }
    };

    // Issue order: the first block's loads, then the state's (kept as raw bits), then the
    // block's staging, then the state's conversion. Left to itself the compiler issued the
    // block's x and dt loads only after converting the state, two round trips in a row.
    load_block(0);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 hraw[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it)
        hraw[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(pool_b + (int64_t)src * H * P * N * SS + soff[it]));
    __builtin_amdgcn_sched_barrier(0);
    t_stage = 0;
    stage_block();
    __builtin_amdgcn_sched_barrier(0);
    float h[ITERS][kVec];
#pragma unroll
    for (int it = 0; it < ITERS; ++it)
        unpack16<ST>(hraw[it], h[it]);

    for (int t0 = 0; t0 < T; t0 += TB) {
        if (t0 > 0) {
            __syncthreads();  // previous block's B/C fully read
            load_block(t0);
            t_stage = t0;
            stage_block();
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const int t = t0 + u;
            // every token of the block runs (no branch around it, which would make the compiler
            // keep copies of the state registers): past T the decay is 1 and the input 0
            const bool live = t < T;
            float Bv[kVec], Cv[kVec];
#pragma unroll
            for (int j = 0; j < kVec; j += 4) {
                const f32x4 bq = *reinterpret_cast<const f32x4 *>(&sBC[u][0][n0 + j]);
                const f32x4 cq = *reinterpret_cast<const f32x4 *>(&sBC[u][1][n0 + j]);
#pragma unroll
                for (int e = 0; e < 4; ++e) { Bv[j + e] = bq[e]; Cv[j + e] = cq[e]; }
            }
            const float dt = sDt[0][u];
            const float decay = sDt[1][u];
            // (the final-state form, CONSEC, is the one launched without a destination table)
            const int d = (!CONSEC && live && a.dst)
                              ? pool_slot(a.dst[(int64_t)row * T + t], a.num_slots, a.err, blockIdx.x == 0 && tid == 0)
                              : -1;
            float yv[ITERS];
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                const float x = xval(u, it);
                const float dx = dt * x;
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < kVec; ++j) {
                    h[it][j] = fmaf(decay, h[it][j], dx * Bv[j]);  // as the one-token kernel
                    acc = fmaf(Cv[j], h[it][j], acc);
                }
                if (d >= 0 && prow(it) < P)
                    nt_store16<ST>(reinterpret_cast<ST *>(const_cast<char *>(pool_b) + (int64_t)d * H * P * N * SS + soff[it]), h[it]);
                if constexpr (kScatter) {
                    yv[it] = acc;  // partial over the lane's kVec values, summed below
                } else {
                    acc = group_sum_last<kLpr>(acc);
                    yv[it] = fmaf(Dh, x, acc);
                    if constexpr (HasZ) yv[it] *= silu_f(zval(u, it));
                    if constexpr (!CONSEC)  // (stored at once: holding them costs registers here)
                        if (live && ylane && prow(it) < P)
                            store_row<1>(a.y, out_dt, ybase, (uint32_t)t * (uint32_t)HP + prow(it), &yv[it]);
                }
            }
            if constexpr (kScatter) {
                // the four rows' sums reduce-scattered over the group: quad k of it finishes row k
                const float tot = row16_sum4_scatter(yv, bit3, bit2);
                const float xk = bit3 ? (bit2 ? xval(u, 3) : xval(u, 2)) : (bit2 ? xval(u, 1) : xval(u, 0));
                float yk = fmaf(Dh, xk, tot);
                if constexpr (HasZ)
                    yk *= silu_f(bit3 ? (bit2 ? zval(u, 3) : zval(u, 2)) : (bit2 ? zval(u, 1) : zval(u, 0)));
                if (live && qlead && prow(0) < P)
                    store_row<1>(a.y, out_dt, ybase, (uint32_t)t * (uint32_t)HP + prow(0) + (lr >> 2), &yk);
            } else if constexpr (CONSEC) {
                if (live) store_y(t, yv);
            }
        }
    }
    if (CONSEC || !a.dst)
#pragma unroll
        for (int it = 0; it < ITERS; ++it)
            if (prow(it) < P)
                nt_store16<ST>(reinterpret_cast<ST *>(const_cast<char *>(pool_b) + (int64_t)src * H * P * N * SS + soff[it]), h[it]);
}

template <typename ST, typename XT, typename AT, int N, int ITERS, bool CONSEC>
static void launch_sum_k(const LayerShape &s, const MultiStepArgs &a, hipStream_t stream, dim3 grid, int psplit) {
    // The snapshot form runs two workgroups per CU (56 KiB of otherwise unused LDS each): with
    // snapshot slots scattered over the pool, a third workgroup's write stream measured 15 %
    // slower (546 against 475 us at 256 rows x 4 tokens).
    const size_t lds = CONSEC ? 0 : 56 * 1024;
    if (a.z)
        hipLaunchKernelGGL((state_update_multi_kernel<ST, XT, AT, N, ITERS, CONSEC, true>), grid, dim3(256), lds, stream,
                           a, s.H, s.P, s.G, s.out_dt, psplit);
    else
        hipLaunchKernelGGL((state_update_multi_kernel<ST, XT, AT, N, ITERS, CONSEC, false>), grid, dim3(256), lds, stream,
                           a, s.H, s.P, s.G, s.out_dt, psplit);
}

template <typename ST, typename XT, int N, int ITERS>
static hipError_t launch_sum(const LayerShape &s, const MultiStepArgs &a, hipStream_t stream, int rows_needed) {
    const int psplit = (rows_needed + ITERS - 1) / ITERS;
    dim3 grid(s.H * psplit, a.batch);
    if (s.act_dt == DT_BF16) {
        if (a.dst) launch_sum_k<ST, XT, bf16, N, ITERS, false>(s, a, stream, grid, psplit);
        else launch_sum_k<ST, XT, bf16, N, ITERS, true>(s, a, stream, grid, psplit);
    } else {
        if (a.dst) launch_sum_k<ST, XT, float, N, ITERS, false>(s, a, stream, grid, psplit);
        else launch_sum_k<ST, XT, float, N, ITERS, true>(s, a, stream, grid, psplit);
    }
    return hipGetLastError();
}

template <typename ST, typename XT, int N>
static hipError_t launch_sum_i(const LayerShape &s, const MultiStepArgs &a, hipStream_t stream) {
    constexpr int kRpi = 256 / (N / Io<ST>::kVec);
    const int rows_needed = (s.P + kRpi - 1) / kRpi;  // passes that cover one head tile
    // as many state rows per thread as keeps >= 2048 workgroups (8 per CU)
    const int64_t wg1 = (int64_t)a.batch * s.H * rows_needed;
    if (rows_needed >= 4 && wg1 / 4 >= 2048) return launch_sum<ST, XT, N, 4>(s, a, stream, rows_needed);
    if (rows_needed >= 2 && wg1 / 2 >= 2048) return launch_sum<ST, XT, N, 2>(s, a, stream, rows_needed);
    return launch_sum<ST, XT, N, 1>(s, a, stream, rows_needed);
}

template <typename ST, typename XT>
static hipError_t launch_sum_n(const LayerShape &s, const MultiStepArgs &a, hipStream_t stream) {
    switch (s.N) {
        case 16: return launch_sum_i<ST, XT, 16>(s, a, stream);
        case 64: return launch_sum_i<ST, XT, 64>(s, a, stream);
        case 128: return launch_sum_i<ST, XT, 128>(s, a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_state_update_multi(const LayerShape &s, const MultiStepArgs &a, hipStream_t stream) {
    if (a.batch == 0 || a.T == 0) return hipSuccess;
    if (s.state_dt == DT_BF16)
        return s.xbc_dt == DT_BF16 ? launch_sum_n<bf16, bf16>(s, a, stream) : launch_sum_n<bf16, float>(s, a, stream);
    return s.xbc_dt == DT_BF16 ? launch_sum_n<float, bf16>(s, a, stream) : launch_sum_n<float, float>(s, a, stream);
}

// ----------------------------------------------------------------- conv update
// One thread per CPT (8 or 4) channels of one row: window = [cached W-1 inputs || u],
// out = SiLU(bias + sum_k w[k] * window[k]); the cache shifts by one.
template <typename AT, typename ST, typename XT, int W, int CPT>
__global__ __launch_bounds__(256) void conv_update_kernel(ConvUpdateArgs a, int64_t cdim) {
    const int row = blockIdx.y;
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * CPT;
    if (c0 >= cdim) return;
    XT *out = static_cast<XT *>(a.out) + (int64_t)row * cdim + c0;
    const int slot = pool_slot(a.idx[row], a.num_slots, a.err, c0 == 0);
    float o[CPT];
    if (slot < 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) o[j] = 0.0f;
        store_k<XT, CPT>(out, o);
        return;
    }
    float u[CPT], win[W - 1][CPT], w[CPT * W];
    load_k<AT, CPT>(static_cast<const AT *>(a.xbc) + (int64_t)row * cdim + c0, u);
    ST *cache = static_cast<ST *>(a.pool) + (int64_t)slot * (W - 1) * cdim + c0;
#pragma unroll
    for (int k = 0; k < W - 1; ++k) load_k<ST, CPT>(cache + k * cdim, win[k]);
    load_k<float, CPT * W>(a.w + c0 * W, w);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        float v = a.b ? a.b[c0 + j] : 0.0f;
#pragma unroll
        for (int k = 0; k < W - 1; ++k) v += w[j * W + k] * win[k][j];
        v += w[j * W + W - 1] * u[j];
        o[j] = silu_f(v);
    }
    store_k<XT, CPT>(out, o);
#pragma unroll
    for (int k = 0; k < W - 2; ++k) store_k<ST, CPT>(cache + k * cdim, win[k + 1]);
    store_k<ST, CPT>(cache + (W - 2) * cdim, u);
}

template <typename AT, typename ST, typename XT, int CPT>
static hipError_t launch_cu_c(const LayerShape &s, const ConvUpdateArgs &a, hipStream_t stream) {
    const int64_t cdim = s.cdim();
    dim3 grid((unsigned)((cdim / CPT + 255) / 256), a.batch);
    switch (s.W) {
        case 2: hipLaunchKernelGGL((conv_update_kernel<AT, ST, XT, 2, CPT>), grid, dim3(256), 0, stream, a, cdim); break;
        case 3: hipLaunchKernelGGL((conv_update_kernel<AT, ST, XT, 3, CPT>), grid, dim3(256), 0, stream, a, cdim); break;
        case 4: hipLaunchKernelGGL((conv_update_kernel<AT, ST, XT, 4, CPT>), grid, dim3(256), 0, stream, a, cdim); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// 8 channels per thread, or 4 when that grid would have under 4,096 workgroups (up to about
// 800 rows at 8B dims: the kernel is one round trip, so more, shorter threads finish sooner;
// measured on the 48-layer decode stack as one graph: concurrency 1, 0.333 -> 0.294 ms per
// step; 16, 0.847 -> 0.803; 64, 2.45 -> 2.40; and on the 256-row decode step, 192.0 -> 190.1 us)
template <typename AT, typename ST, typename XT>
static hipError_t launch_cu_w(const LayerShape &s, const ConvUpdateArgs &a, hipStream_t stream) {
    const int64_t wg8 = (s.cdim() / 8 + 255) / 256 * (int64_t)a.batch;
    return wg8 < 4096 ? launch_cu_c<AT, ST, XT, 4>(s, a, stream) : launch_cu_c<AT, ST, XT, 8>(s, a, stream);
}

template <typename AT, typename ST>
static hipError_t launch_cu_x(const LayerShape &s, const ConvUpdateArgs &a, hipStream_t stream) {
    return s.xbc_dt == DT_BF16 ? launch_cu_w<AT, ST, bf16>(s, a, stream) : launch_cu_w<AT, ST, float>(s, a, stream);
}

template <typename AT>
static hipError_t launch_cu_s(const LayerShape &s, const ConvUpdateArgs &a, hipStream_t stream) {
    return s.state_dt == DT_BF16 ? launch_cu_x<AT, bf16>(s, a, stream) : launch_cu_x<AT, float>(s, a, stream);
}

hipError_t launch_conv_update(const LayerShape &s, const ConvUpdateArgs &a, hipStream_t stream) {
    if (a.batch == 0) return hipSuccess;
    return s.act_dt == DT_BF16 ? launch_cu_s<bf16>(s, a, stream) : launch_cu_s<float>(s, a, stream);
}

// T tokens per row: window = [cached W-1 inputs || token], shifted per token;
// after token t the window goes to dst[row][t] when that slot is >= 0 (no dst
// table: the final window to the source slot).
template <typename AT, typename ST, typename XT, int W, int CPT>
__global__ __launch_bounds__(256) void conv_update_multi_kernel(ConvMultiArgs a, int64_t cdim) {
    const int row = blockIdx.y;
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * CPT;
    if (c0 >= cdim) return;
    const int T = a.T;
    const int src = pool_slot(a.src[row], a.num_slots, a.err, c0 == 0);
    XT *out = static_cast<XT *>(a.out) + (int64_t)row * T * cdim + c0;
    float o[CPT];
    if (src < 0) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) o[j] = 0.0f;
        for (int t = 0; t < T; ++t) store_k<XT, CPT>(out + (int64_t)t * cdim, o);
        return;
    }
    // The tokens go in blocks of TB whose raw inputs are all loaded before the first is used
    // (rows past T clamped to the last), next to the window and the weights: one round trip
    // per block instead of one per token.
    constexpr int TB = 4;
    const AT *xin = static_cast<const AT *>(a.xbc) + (int64_t)row * T * cdim + c0;
    ST *pool = static_cast<ST *>(a.pool);
    Raw<AT, CPT> ur[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) ur[i].load(xin + (int64_t)min(i, T - 1) * cdim);
    float win[W - 1][CPT], w[CPT * W], bias[CPT];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) load_k<ST, CPT>(pool + ((int64_t)src * (W - 1) + k) * cdim + c0, win[k]);
    load_k<float, CPT * W>(a.w + c0 * W, w);
#pragma unroll
    for (int j = 0; j < CPT; ++j) bias[j] = a.b ? a.b[c0 + j] : 0.0f;
    for (int t0 = 0; t0 < T; t0 += TB) {
        if (t0 > 0)
#pragma unroll
            for (int i = 0; i < TB; ++i) ur[i].load(xin + (int64_t)min(t0 + i, T - 1) * cdim);
#pragma unroll
        for (int i = 0; i < TB; ++i) {
            const int t = t0 + i;
            if (t < T) {
                float u[CPT];
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    u[j] = ur[i][j];
                    float v = bias[j];  // the order of the one-token update: bias, cached taps, new input
#pragma unroll
                    for (int k = 0; k < W - 1; ++k) v += w[j * W + k] * win[k][j];
                    v += w[j * W + W - 1] * u[j];
                    o[j] = silu_f(v);
                }
                store_k<XT, CPT>(out + (int64_t)t * cdim, o);
#pragma unroll
                for (int k = 0; k < W - 2; ++k)
#pragma unroll
                    for (int j = 0; j < CPT; ++j) win[k][j] = win[k + 1][j];
#pragma unroll
                for (int j = 0; j < CPT; ++j) win[W - 2][j] = u[j];
                if (a.dst) {
                    const int d = pool_slot(a.dst[(int64_t)row * T + t], a.num_slots, a.err, c0 == 0);
                    if (d >= 0)
#pragma unroll
                        for (int k = 0; k < W - 1; ++k) store_k<ST, CPT>(pool + ((int64_t)d * (W - 1) + k) * cdim + c0, win[k]);
                }
            }
        }
    }
    if (!a.dst)
#pragma unroll
        for (int k = 0; k < W - 1; ++k) store_k<ST, CPT>(pool + ((int64_t)src * (W - 1) + k) * cdim + c0, win[k]);
}

// 4 channels per thread where 8 would give under 2,048 workgroups (256 rows at 8B dims give
// 1,280: the kernel is a few round trips, so more, shorter threads finish sooner)
template <typename AT, typename ST, typename XT, int CPT>
static hipError_t launch_cum_c(const LayerShape &s, const ConvMultiArgs &a, hipStream_t stream) {
    const int64_t cdim = s.cdim();
    dim3 grid((unsigned)((cdim / CPT + 255) / 256), a.batch);
    switch (s.W) {
        case 2: hipLaunchKernelGGL((conv_update_multi_kernel<AT, ST, XT, 2, CPT>), grid, dim3(256), 0, stream, a, cdim); break;
        case 3: hipLaunchKernelGGL((conv_update_multi_kernel<AT, ST, XT, 3, CPT>), grid, dim3(256), 0, stream, a, cdim); break;
        case 4: hipLaunchKernelGGL((conv_update_multi_kernel<AT, ST, XT, 4, CPT>), grid, dim3(256), 0, stream, a, cdim); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename AT, typename ST, typename XT>
static hipError_t launch_cum_w(const LayerShape &s, const ConvMultiArgs &a, hipStream_t stream) {
    const int64_t wg8 = (s.cdim() / 8 + 255) / 256 * (int64_t)a.batch;
    return wg8 < 2048 ? launch_cum_c<AT, ST, XT, 4>(s, a, stream) : launch_cum_c<AT, ST, XT, 8>(s, a, stream);
}

template <typename AT, typename ST>
static hipError_t launch_cum_x(const LayerShape &s, const ConvMultiArgs &a, hipStream_t stream) {
    return s.xbc_dt == DT_BF16 ? launch_cum_w<AT, ST, bf16>(s, a, stream) : launch_cum_w<AT, ST, float>(s, a, stream);
}

template <typename AT>
static hipError_t launch_cum_s(const LayerShape &s, const ConvMultiArgs &a, hipStream_t stream) {
    return s.state_dt == DT_BF16 ? launch_cum_x<AT, bf16>(s, a, stream) : launch_cum_x<AT, float>(s, a, stream);
}

hipError_t launch_conv_update_multi(const LayerShape &s, const ConvMultiArgs &a, hipStream_t stream) {
    if (a.batch == 0 || a.T == 0) return hipSuccess;
    return s.act_dt == DT_BF16 ? launch_cum_s<bf16>(s, a, stream) : launch_cum_s<float>(s, a, stream);
}

}  // namespace m2

// ----------------------------------------------------------------- slot index checks
namespace m2 {

// Count of pool indices >= the caller's slot count that kernels skipped, on this device:
// a file-scope device word, one copy per device for the life of the process. Host code
// never passes the name itself to a kernel; it passes the address that slot_error_word
// looks up (once per device) with hipGetSymbolAddress.
static __device__ __align__(16) unsigned g_slot_errors[4];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<unsigned *> g_err_addr[kMaxDevices];
std::mutex g_err_mu;
}  // namespace

hipError_t slot_error_word(unsigned **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    unsigned *p = g_err_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_err_mu);
        p = g_err_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void *sym = nullptr;
            e = hipGetSymbolAddress(&sym, HIP_SYMBOL(g_slot_errors));
            if (e != hipSuccess) return e;
            p = static_cast<unsigned *>(sym);
            g_err_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

// One workgroup: indices >= num_slots, and indices in [0, num_slots) that repeat an earlier
// entry of the list (O(n^2) compares: a debug check).
__global__ __launch_bounds__(1024) void check_slots_kernel(const int32_t *idx, int n, int num_slots,
                                                          unsigned *result) {
    __shared__ unsigned s_bad, s_dup;
    if (threadIdx.x == 0) {
        s_bad = 0;
        s_dup = 0;
    }
    __syncthreads();
    unsigned bad = 0, dup = 0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int v = idx[i];
        if (v >= num_slots) {
            ++bad;
        } else if (v >= 0) {
            for (int j = 0; j < i; ++j)
                if (idx[j] == v) {
                    ++dup;
                    break;
                }
        }
    }
    atomicAdd(&s_bad, bad);
    atomicAdd(&s_dup, dup);
    __syncthreads();
    if (threadIdx.x == 0) {
        result[0] = s_bad;
        result[1] = s_dup;
    }
}

// Copies the count into the caller's memory and, if asked, clears it (one thread).
__global__ void read_slot_errors_kernel(unsigned *word, unsigned *dst, int reset) {
    dst[0] = word[0];
    if (reset) word[0] = 0;
}

hipError_t launch_read_slot_errors(unsigned *dst, int reset, hipStream_t stream) {
    unsigned *word = nullptr;
    hipError_t e = slot_error_word(&word);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(read_slot_errors_kernel, dim3(1), dim3(1), 0, stream, word, dst, reset);
    return hipGetLastError();
}

hipError_t launch_check_slots(const int32_t *idx, int n, int num_slots, unsigned *result, hipStream_t stream) {
    hipLaunchKernelGGL(check_slots_kernel, dim3(1), dim3(1024), 0, stream, idx, n, num_slots, result);
    return hipGetLastError();
}

}  // namespace m2
