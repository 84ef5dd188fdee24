// Fused prefill for the Nemotron-H head shape (P = 64, N = 128, y in bf16):
// conv1d + SiLU and the chunked SSD scan in two kernels, with the x channels
// going from raw input to y without a post-conv round trip through HBM.
//
// The record page ("Nemotron-H-8B-Base-8K", mixer tensors conv1d, A_log, D,
// dt_bias, norm; section "REQUIRED KERNEL CLASS") fixes the layer's pieces;
// the conv reading is the one the conv kernels use (last tap on the current
// token, left context from the slot's cached raw inputs or zeros). The chunk
// algebra is that of the chunked scan (scan.hip). Chunks here are blocks of L
// tokens aligned to absolute token positions (block b = tokens [bL, bL + L)),
// cut at sequence boundaries; any partition of a sequence into chunks gives
// the same result in exact arithmetic.
//
// 1. prep kernel, one workgroup per (block, group): conv + SiLU of the group's
//    B and C channels (once per group instead of once per head), written as
//      Cp  [T][G][N] bf16, token-major, n permuted inside each 32-block so
//          that one 16-byte read gives the k-slots of the carried-state
//          product below,
//      BT  [block][G][hi|lo][N][L] bf16, the B^T operand of the state update
//          (hi = RNE(B), lo = RNE(B - hi)),
//      CB  [block][G][L/16][L/32][64 lanes][8] fp32: C_t . B_s for the block,
//          already in the per-lane layout of the intra-chunk MFMA operand.
//    Rows of other sequences inside a block are harmless: the scan multiplies
//    them by x = 0 and never stores their outputs.
//
// 2. scan kernel, one workgroup of four wavefronts per (sequence, head); wave
//    w owns channels [16w, 16w + 16) of the head for the whole sequence:
//      * the carried state H^T (N x 16 per wave) lives in MFMA accumulators;
//        converted to bf16 in place, those registers are the A operand of
//        the carried-state output (k-slots = the permuted n order of Cp), so
//        H never goes through LDS;
//      * each lane computes the conv + SiLU of its own channel for eight
//        consecutive tokens per 32-token block: exactly the k-slots of the
//        x operands (x dt for the output, x dt exp(lam_end - lam) as hi/lo
//        for the state), so post-conv x is never shared or stored; its raw
//        rows reach the lanes through a small wave-private LDS tile;
//      * D x is one more MFMA per t-tile, against a selector operand that
//        holds D (in bf16) on the diagonal;
//      * the shared LDS tiles are B^T hi/lo, C and the decayed C.B^T operands
//        (each wave forms half of one t-tile's), double-buffered: about 80 KB
//        per workgroup with the wave-private tiles, so two workgroups share a
//        CU and overlap each other's phases;
//      * block b computes from tiles staged one iteration earlier while block
//        b + 1 is staged into the other buffer; block b + 3's tiles, raw x,
//        dt and C.B^T are loaded into one of two register sets as soon as
//        the registers they fill are free, two iterations ahead of use.
//
// With conv width W = 1 both kernels take post-conv xBC as it is (no conv, no
// SiLU, no context rows): that instantiation is mamba2_chunk_scan_fwd's form
// when the caller passes a workspace.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace m2 {

namespace {

template <typename T> __device__ __forceinline__ float bits_f(uint32_t v) {
    if constexpr (sizeof(T) == 4) return __uint_as_float(v);
    else return __uint_as_float(v << 16);
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// segment flags (segment mode): the sequence's first segment; its only one
constexpr int kSegFirst = 1, kSegOnly = 2;
constexpr int kMinSeg = 1024;  // tokens per segment at least

// Segment mode's plan, seg[v] for v = r * smax + k: segment k of sequence r (empty
// past its last one) as {start, end, sequence, first/only flags}; written by the
// first workgroup of the prep kernel, read by the scan and the passes after it.
__device__ __forceinline__ void seg_plan(const int32_t *cu, int smax, int v, int32_t *seg) {
    const int r = v / smax, k = v % smax;
    const int s0 = cu[r], s1 = cu[r + 1], len = s1 - s0;
    const int S = max(1, min(smax, len / kMinSeg));
    const int step = (len + S - 1) / S;
    auto bound = [&](int i) {  // segment boundaries at multiples of 32 of the packed position
        if (i <= 0) return s0;
        if (i >= S) return s1;
        return min((s0 + i * step + 31) / 32 * 32, s1);
    };
    int32_t *o = seg + 4 * v;
    o[0] = k < S ? bound(k) : s1;
    o[1] = k < S ? bound(k + 1) : s1;
    o[2] = r;
    o[3] = k < S ? ((k == 0 ? kSegFirst : 0) | (S == 1 ? kSegOnly : 0)) : 0;
}

}  // namespace

// ---------------------------------------------------------------- prep
// XT: xbc element type. W == 1: xbc is already conv + SiLU output and its B/C
// rows are taken as they are.
template <typename XT, typename ST, int W, int L>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(XT) == 2 ? 4 : 1))) void fused_prep_kernel(FusedArgs a, int H, int G, int smax) {
    constexpr bool CONV = W > 1;
    constexpr int P = 64, N = 128;
    constexpr int RL = L / 8;   // tokens per thread
    constexpr int NS = N + 16;  // bf16 row stride of the token-major tiles (288 bytes: conflict-free operand reads)
    constexpr int CBS = L + 4;  // float row stride of the C.B^T tile
    constexpr int TL = L / 16, KL = L / 32, KN = N / 32;
    __shared__ __attribute__((aligned(16))) bf16 sB[2][L * NS];
    __shared__ __attribute__((aligned(16))) bf16 sC[L * NS];
    __shared__ __attribute__((aligned(16))) float sCB[L * CBS];
    constexpr int kCu = 256;  // cu_seqlens entries staged in LDS for the sequence search
    __shared__ int32_t sCu[kCu + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int blk = blockIdx.x, g = blockIdx.y;
    const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N, cdim = HP + 2 * GN;
    // waves 0 and 2 take the B channels, waves 1 and 3 the C channels (16 groups of 8 channels x
    // 4 runs of RL tokens each): the per-token output path is one branch per wave, not both
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const bool isC = wv & 1;
    const int cg = (tid & 15) + (isC ? 16 : 0), run = ((tid >> 4) & 3) + 4 * (wv >> 1);
    const int n0 = 8 * (cg & 15);
    const int64_t c0 = HP + (isC ? GN : 0) + (int64_t)g * N + n0;  // first of this thread's 8 channels
    const int64_t t0 = (int64_t)blk * L + run * RL;
    const XT *in = static_cast<const XT *>(a.xbc) + c0;

    float w[8 * W], bias[8];
    if constexpr (CONV) {
        load_k<float, 8 * W>(a.conv_w + c0 * W, w);
#pragma unroll
        for (int j = 0; j < 8; ++j) bias[j] = a.conv_b ? a.conv_b[c0 + j] : 0.0f;
    }
    // The run's raw rows (the conv window of its RL tokens) as raw bits at 32-bit offsets from
    // the window's first row, clamped only to the packed rows [0, T): issued before the
    // sequence lookup below, whose cu_seqlens load would otherwise come first. Rows outside
    // the run's sequence are replaced by its context or never used.
    constexpr int NR = RL + W - 1;
    const int64_t r0 = t0 - (W - 1);
    Raw<XT, 8> rw[CONV ? NR : 1];
    if (CONV && t0 < a.T) {
        const char *wbase = reinterpret_cast<const char *>(in + r0 * cdim);
        const uint32_t rowb = (uint32_t)(cdim * (int64_t)sizeof(XT));
#pragma unroll
        for (int i = 0; i < (CONV ? NR : 1); ++i) {
            int64_t r = r0 + i;
            r = r < 0 ? 0 : (r > a.T - 1 ? a.T - 1 : r);
            rw[i].load(reinterpret_cast<const XT *>(wbase + (uint32_t)(r - r0) * rowb));
        }
    }

    // one coalesced load of cu_seqlens per workgroup, then searches in LDS (global
    // binary search, one dependent load per step, past kCu sequences)
    if (smax && blockIdx.x == 0 && blockIdx.y == 0)  // segment mode: the plan (the scan runs after this kernel)
        for (int v = threadIdx.x; v < a.nseq * smax; v += 256) seg_plan(a.cu, smax, v, const_cast<int32_t *>(a.seg));
    const bool cu_lds = CONV && a.nseq <= kCu;
    if (cu_lds)
        for (int i = tid; i <= a.nseq; i += 256) sCu[i] = a.cu[i];
    __syncthreads();
    const int32_t *cus = cu_lds ? sCu : a.cu;

    // Token i of the thread's run leaves as soon as it is computed: B as hi / lo rows of
    // the token-major tiles (C.B^T below, and the transposed planes); C in natural order
    // in LDS and as a permuted token-major row of the workspace. Rows past T or of
    // padding sequences are zeros.
    const int tl0 = run * RL;  // first token of the thread inside the block
    bf16 *cp = static_cast<bf16 *>(a.cp) + (int64_t)g * N + (n0 & ~31);
    const int u0 = n0 & 31;
    auto emit = [&](int i, const float *o) {
        if (!isC) {
            bf16x8 h, l;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                h[j] = f32_to_bf16(o[j]);
                l[j] = f32_to_bf16(o[j] - (float)h[j]);
            }
            *reinterpret_cast<bf16x8 *>(&sB[0][(tl0 + i) * NS + n0]) = h;
            *reinterpret_cast<bf16x8 *>(&sB[1][(tl0 + i) * NS + n0]) = l;
        } else {
            bf16x8 c;
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = f32_to_bf16(o[j]);
            *reinterpret_cast<bf16x8 *>(&sC[(tl0 + i) * NS + n0]) = c;
            if (t0 + i < a.T) {
                bf16 *row = cp + (t0 + i) * GN;
                *reinterpret_cast<bf16x4 *>(row + perm32(u0)) = bf16x4{c[0], c[1], c[2], c[3]};
                *reinterpret_cast<bf16x4 *>(row + perm32(u0 + 4)) = bf16x4{c[4], c[5], c[6], c[7]};
            }
        }
    };
    const float zero8[8] = {};
    int done = 0;  // tokens of the run emitted so far (the rest are emitted as zeros below)

    // conv + SiLU of 8 channels x RL tokens
    if constexpr (!CONV) {
        // post-conv rows as they are
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            float o[8];
            if (t0 + i < a.T) load_k<XT, 8>(in + (t0 + i) * cdim, o);
            else
#pragma unroll
                for (int j = 0; j < 8; ++j) o[j] = 0.0f;
            emit(i, o);
        }
        done = RL;
    } else if (t0 < a.T) {
        const int64_t tl = (t0 + RL < a.T ? t0 + RL : a.T) - 1;  // last token of the run
        const int sa = find_seq(cus, a.nseq, t0), sb = find_seq(cus, a.nseq, tl);
        if (sa == sb) {
            // one sequence holds the whole run: its rows were loaded up front (rw)
            const int64_t ss = cus[sa];
            const int slot = pool_slot(a.idx[sa], a.num_slots, a.err, false);
            // rows before the sequence (only among the first W - 1): its cached raw inputs or zeros
            const bool head = r0 < ss;
            float ctx[W - 1][8];
            if (head) {
                const bool init = slot >= 0 && a.has_init && a.has_init[sa];
                const ST *cache = static_cast<const ST *>(a.conv_pool) + (int64_t)(slot < 0 ? 0 : slot) * (W - 1) * cdim + c0;
#pragma unroll
                for (int k = 0; k < W - 1; ++k) {
                    const int64_t d = ss - (r0 + k);
                    if (d <= 0) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) ctx[k][j] = rw[k][j];
                    } else if (init) {
                        load_k<ST, 8>(cache + (int64_t)((W - 1) - d) * cdim, ctx[k]);
                    } else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) ctx[k][j] = 0.0f;
                    }
                }
            }
            if (slot >= 0) {
#pragma unroll
                for (int i = 0; i < RL; ++i) {
                    if (t0 + i > tl) break;
                    float o[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        float v = bias[j];
#pragma unroll
                        for (int k = 0; k < W; ++k) {
                            const int rr = i + k;
                            v += w[j * W + k] * ((rr < W - 1 && head) ? ctx[rr][j] : rw[rr][j]);
                        }
                        o[j] = silu_fast(v);
                    }
                    emit(i, o);
                    done = i + 1;
                }
            }
        } else {
            // a sequence boundary inside the run: token by token, restarting the window
            int seq = sa;
            int64_t seq_start = cus[seq], seq_end = cus[seq + 1];
            int slot = pool_slot(a.idx[seq], a.num_slots, a.err, false);
            float win[W - 1][8];
            auto fill_window = [&](int64_t t) {
                const bool init = slot >= 0 && a.has_init && a.has_init[seq];
                const ST *cache = static_cast<const ST *>(a.conv_pool) + (int64_t)(slot < 0 ? 0 : slot) * (W - 1) * cdim + c0;
#pragma unroll
                for (int k = 0; k < W - 1; ++k) {
                    const int64_t src = t - (W - 1) + k;
                    if (src >= seq_start) load_k<XT, 8>(in + src * cdim, win[k]);
                    else if (init) load_k<ST, 8>(cache + (int64_t)((W - 1) - (seq_start - src)) * cdim, win[k]);
                    else
#pragma unroll
                        for (int j = 0; j < 8; ++j) win[k][j] = 0.0f;
                }
            };
            fill_window(t0);
            for (int i = 0; i < RL && t0 + i <= tl; ++i) {
                const int64_t t = t0 + i;
                if (t >= seq_end) {  // the next non-empty sequence starts exactly at t
                    while (seq + 1 < a.nseq && cus[seq + 1] <= t) ++seq;
                    seq_start = cus[seq];
                    seq_end = cus[seq + 1];
                    slot = pool_slot(a.idx[seq], a.num_slots, a.err, false);
                    fill_window(t);
                }
                float u[8], o[8];
                load_k<XT, 8>(in + t * cdim, u);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float v = bias[j];
#pragma unroll
                    for (int k = 0; k < W - 1; ++k) v += w[j * W + k] * win[k][j];
                    v += w[j * W + W - 1] * u[j];
                    o[j] = slot >= 0 ? silu_fast(v) : 0.0f;
                }
                emit(i, o);
                done = i + 1;
#pragma unroll
                for (int k = 0; k < W - 2; ++k)
#pragma unroll
                    for (int j = 0; j < 8; ++j) win[k][j] = win[k + 1][j];
#pragma unroll
                for (int j = 0; j < 8; ++j) win[W - 2][j] = u[j];
            }
        }
    }

    for (int i = done; i < RL; ++i) emit(i, zero8);
    __syncthreads();

    // B^T hi / lo planes [hl][n][L] from the token-major tiles: 16-byte pieces of 8 tokens,
    // consecutive threads on consecutive pieces
    {
        constexpr int PCS = 2 * N * L / 8 / 256;
        bf16 *bt = static_cast<bf16 *>(a.bt) + ((int64_t)blk * G + g) * (2 * N * L);
#pragma unroll
        for (int i = 0; i < PCS; ++i) {
            const int id = tid + i * 256;
            const int k = id % (L / 8), n = (id / (L / 8)) % N, hl = id / (N * L / 8);
            bf16x8 v;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = sB[hl][(8 * k + j) * NS + n];
            *reinterpret_cast<bf16x8 *>(bt + 8 * id) = v;
        }
    }

    // C.B^T (B as hi + lo), rows t, columns s; every (t-tile, s-tile) pair so
    // that the scan may load whole operand rows unconditionally.
    float *cbg = static_cast<float *>(a.cb) + ((int64_t)blk * G + g) * (TL * KL) * 512;
    if constexpr (TL == 2) {
        // one 16x16 tile per wave: t-tile wave >> 1, s-tile wave & 1
        const int tt = wave >> 1, si = wave & 1;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kn = 0; kn < KN; ++kn) {
            const bf16x8 ca = *reinterpret_cast<const bf16x8 *>(&sC[(16 * tt + col) * NS + 32 * kn + 8 * q]);
            const int off = (16 * si + col) * NS + 32 * kn + 8 * q;
            acc = mma(ca, *reinterpret_cast<const bf16x8 *>(&sB[0][off]), acc);
            acc = mma(ca, *reinterpret_cast<const bf16x8 *>(&sB[1][off]), acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sCB[(16 * tt + 4 * q + r) * CBS + 16 * si + col] = acc[r];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // this wave's columns are k-slots 8 qo + [0, 8) for qo in {2 si, 2 si + 1}: 16 bytes per lane
        const int co = lane & 15, qo = 2 * si + ((lane >> 4) & 1), half = lane >> 5;
        const f32x4 v = *reinterpret_cast<const f32x4 *>(&sCB[(16 * tt + co) * CBS + 8 * qo + 4 * half]);
        *reinterpret_cast<f32x4 *>(cbg + (tt * KL) * 512 + (qo * 16 + co) * 8 + 4 * half) = v;
    } else {
        for (int tt = wave; tt < TL; tt += 4) {
            bf16x8 ca[KN];
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) ca[kn] = *reinterpret_cast<const bf16x8 *>(&sC[(16 * tt + col) * NS + 32 * kn + 8 * q]);
#pragma unroll
            for (int si = 0; si < TL; ++si) {
                f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kn = 0; kn < KN; ++kn) {
                    const int off = (16 * si + col) * NS + 32 * kn + 8 * q;
                    acc = mma(ca[kn], *reinterpret_cast<const bf16x8 *>(&sB[0][off]), acc);
                    acc = mma(ca[kn], *reinterpret_cast<const bf16x8 *>(&sB[1][off]), acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) sCB[(16 * tt + 4 * q + r) * CBS + 16 * si + col] = acc[r];
            }
            // the rows just written belong to this wave: a wave-level fence suffices
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            float *cb = cbg + (tt * KL) * 512 + lane * 8;
#pragma unroll
            for (int m = 0; m < KL; ++m) {
                const float *src = &sCB[(16 * tt + col) * CBS + 32 * m + 8 * q];
                *reinterpret_cast<f32x4 *>(cb + m * 512) = *reinterpret_cast<const f32x4 *>(src);
                *reinterpret_cast<f32x4 *>(cb + m * 512 + 4) = *reinterpret_cast<const f32x4 *>(src + 4);
            }
        }
    }
}

// ---------------------------------------------------------------- scan
// Per block b the loop body computes block b (carried-state output, intra-block
// output, D x, the state update: MFMA work on LDS tiles staged one iteration
// earlier) and stages block b + 1 (tiles into the other LDS buffer, token
// arrays, conv + SiLU of x, decayed C.B^T: VALU work), in one instruction
// stream so the two overlap. The loads of block b + 3 go out as the registers
// they fill come free, and the waves meet at the one barrier of the iteration.
template <int L, int W, typename ST, typename AT, typename XT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void fused_scan_kernel(FusedArgs a, int H, int G) {
    constexpr int P = 64, N = 128, NT = 256;
    constexpr int TL = L / 16, KL = L / 32, KN = N / 32, NTL = N / 16;
    // Row strides of the LDS tiles read as MFMA operands (16 bytes per lane, rows by lane & 15,
    // pieces by lane >> 4): a stride of 32 mod 64 bytes keeps those reads free of bank
    // conflicts on gfx950 (measured: 80 or 272 bytes cost two passes, 96 or 288 one). With
    // fp32 x rows the wider B^T stride would leave room for one workgroup per CU, not two.
    constexpr int BTS = sizeof(XT) == 2 ? L + 16 : L + 8;  // bf16 row stride of the B^T tiles [n][s]
    constexpr int CS = N + 16;                               // bf16 row stride of the C tile [t][n]
    constexpr bool CONV = W > 1;               // W == 1: xbc is already conv + SiLU output (taken as is)
    constexpr int XR = 8 + W - 1;              // raw x rows behind one lane's 8 tokens
    constexpr int XRW = L + W - 1;             // raw x rows of a block
    constexpr uint32_t AS = sizeof(AT);        // dt_raw and z elements
    constexpr uint32_t XS = sizeof(XT);        // xbc elements
    constexpr int XRB = 16 * XS + 8;           // bytes per row of a wave's raw x tile (its 16 channels + pad)
    constexpr int CPR = XS;                    // 16-byte pieces per raw row of 16 channels
    constexpr int XP = (CPR * XRW + 63) / 64;  // raw x pieces per lane
    constexpr int BTP = (2 * N * L / 8) / NT;  // 16-byte B^T pieces per thread
    constexpr int CPC = (L * N / 8) / NT;      // 16-byte C pieces per thread
    constexpr float LOG2E = 1.4426950408889634f;
    // The decayed C.B^T operands are split over the waves: with two t-tiles,
    // wave w forms k-slots [4 (w & 1), 4 (w & 1) + 4) of t-tile w >> 1; with
    // more, wave w forms all k-slots of t-tile w.
    constexpr bool MSPLIT = TL == 2;
    constexpr int MJ = MSPLIT ? 4 : 8;
    static_assert(L == 32 || L == 64, "block of 32 or 64 tokens");
    static_assert(BTP * NT * 8 == 2 * N * L && CPC * NT * 8 == L * N, "tile pieces divide over threads");

    __shared__ __attribute__((aligned(16))) bf16 sBT[2][2 * N * BTS];
    __shared__ __attribute__((aligned(16))) bf16 sC[2][L * CS];
    __shared__ __attribute__((aligned(16))) bf16x8 sM[2][TL * KL * 64];
    __shared__ __attribute__((aligned(16))) float sTok[4][3][64];  // per wave: dt, lam (log2 units), state weight
    __shared__ __attribute__((aligned(16))) char sXr[4][XRW * XRB];  // per wave: raw x rows of its channels

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in a scalar register
    const int col = lane & 15, q = lane >> 4;
    __shared__ int sSeq;
    const int head = xcd_head(blockIdx.x, H);
    // the workgroup's tokens: a whole sequence, or in segment mode one segment of one
    int seq, sflags;
    int64_t start, end;
    if (a.seg) {
        const int32_t *sg = a.seg + 4 * blockIdx.y;
        start = sg[0];
        end = sg[1];
        seq = sg[2];
        sflags = sg[3];
    } else {
        seq = seq_longest_first(a.cu, a.nseq, blockIdx.y, tid, NT, &sSeq);
        start = a.cu[seq];
        end = a.cu[seq + 1];
        sflags = kSegFirst | kSegOnly;
    }
    // a later segment starts from zero state and reads its conv context from the tokens before it
    const bool first = sflags & kSegFirst, only = sflags & kSegOnly;
    const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N, cdim = HP + 2 * GN;
    const int g = head / (H / G);
    const int slot = pool_slot(a.idx[seq], a.num_slots, a.err, head == 0 && tid == 0 && first);
    bf16 *y = static_cast<bf16 *>(a.y);

    if (slot < 0) {
        for (int64_t i = tid; i < (end - start) * P; i += NT) y[(start + i / P) * HP + (int64_t)head * P + (i % P)] = f32_to_bf16(0.0f);
        return;
    }

    const float A2 = -expf(a.A_log[head]) * LOG2E;  // log2 decay per unit dt
    const float dtb = a.dt_bias[head];
    const float Dh = a.D[head];
    const int p = 16 * wv + col;  // this lane's channel inside the head (x operands, state column)
    const int64_t chx = (int64_t)head * P + p;
    const bool init = first && a.has_init && a.has_init[seq];

    float cw[W], ctx[CONV ? W - 1 : 1];
    float cbias = 0.0f;
    if constexpr (CONV) {
#pragma unroll
        for (int k = 0; k < W; ++k) cw[k] = a.conv_w[chx * W + k];
        cbias = a.conv_b ? a.conv_b[chx] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < W - 1; ++k)
        ctx[k] = init ? (float)static_cast<const ST *>(a.conv_pool)[((int64_t)slot * (W - 1) + k) * cdim + chx] : 0.0f;

    // carried state: lane holds H[p][16 nt + 4q + r]
    ST *pool_h = static_cast<ST *>(a.pool) + ((int64_t)slot * H + head) * (int64_t)P * N + (int64_t)p * N;
    f32x4 Hacc[NTL];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (init) load_k<ST, 4>(pool_h + 16 * nt + 4 * q, v);
        Hacc[nt] = f32x4{v[0], v[1], v[2], v[3]};
    }

    // D x as an MFMA: column t of a 32-token block picks k-slot t with weight D (in bf16: x is
    // a bf16 operand already, and y is stored in bf16, whose rounding is of the same size)
    bf16x8 Dsel[2];  // [t-tile parity]
    {
        const bf16 dh = f32_to_bf16(Dh), zero = f32_to_bf16(0.0f);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 8; ++j) Dsel[h][j] = 8 * q + j == 16 * h + col ? dh : zero;
    }

    // ---- loads of a block into registers (raw bits, converted where used)
    const int ttw = MSPLIT ? (wv >> 1) : (wv < TL ? wv : TL - 1);
    const int mj0 = MSPLIT ? 4 * (wv & 1) : 0;
    struct Pre {  // one block's loads in registers: B^T, C, raw x, C.B^T and dt
        u32x4 btr[BTP], cr[CPC], xq[XP];
        f32x4 cbr[KL][MJ / 4];
        AT dtr;  // (as its own type: held as zero-extended bits it cost a copy, and a wait, per block pair)
    };
    Pre P0, P1;  // two sets in turn, so each block's loads have two iterations to arrive
    // Loads take a wave-uniform base plus a 32-bit unsigned byte offset per lane
    // (the global_load scalar-base form). Rows are clamped in offset space
    // (offsets grow with the row), so a block at a sequence edge costs one
    // v_med3 per load and every load stays unconditional; values that do not
    // belong to the sequence are replaced when staged.
    const uint32_t xrow = (uint32_t)cdim * XS;                  // bytes per xbc row
    uint32_t xq_off[XP], xq_part[XP];                           // raw x piece k of this lane: row, 16-byte part
#pragma unroll
    for (int k = 0; k < XP; ++k) {
        const int id = lane + 64 * k, rho = min(id / CPR, XRW - 1);
        xq_off[k] = (uint32_t)rho * xrow;
        xq_part[k] = 16u * (id % CPR);
    }
    const uint32_t dtlane = (uint32_t)(lane < L ? lane : L - 1) * H * AS;
    const uint32_t crow = (uint32_t)GN * 2;                                // bytes per Cp row
    const uint32_t clane = (uint32_t)(tid / (N / 8)) * crow + 16 * (tid % (N / 8));
    const uint32_t zrow = (uint32_t)HP * AS;                               // bytes per z row
    const uint32_t ylane = col * (uint32_t)HP * 2 + 8 * q;                 // y: row col of a t-tile, channels 4q..
    // The workgroup's blocks, and the sequence (or segment) bounds and the packed end relative to
    // the first one's start: per block, edges are then 32-bit differences (a sequence has fewer
    // than 2^31 tokens), not 64-bit compares and selects.
    const int64_t b0 = start / L, b1 = end > start ? (end - 1) / L : b0 - 1;
    const int32_t s_rel = (int32_t)(start - b0 * L), e_rel = (int32_t)(end - b0 * L);
    const int32_t t_rel = (int32_t)(a.T - b0 * L);  // (T fits: the boundary refuses totals past int32)
    auto rel = [&](int64_t b) { return (int32_t)(b - b0) * L; };  // block b's first token, relative to block b0
    // Loads of a block in two parts, each issued as soon as the registers it fills are free
    // (the tiles' once they are staged into LDS, the token and C.B^T values' once the operands
    // are formed), into the set that block b + 1 has just left: two iterations to arrive.
    auto prefetch_tiles = [&](int64_t b, Pre &R) __attribute__((always_inline)) {
        const int64_t bL = b * L;
        const char *btb = static_cast<const char *>(a.bt) + (b * G + g) * (int64_t)(2 * N * L * 2);
#pragma unroll
        for (int i = 0; i < BTP; ++i) R.btr[i] = *reinterpret_cast<const u32x4 *>(btb + 16u * (tid + i * NT));
        const int tr = t_rel - 1 - rel(b);
        const int tmax = tr < L - 1 ? tr : L - 1;  // C rows end at T
        const char *cpb = static_cast<const char *>(a.cp) + (bL * GN + (int64_t)g * N) * 2;
        const uint32_t cmax = (uint32_t)tmax * crow + 16 * (tid % (N / 8));
#pragma unroll
        for (int i = 0; i < CPC; ++i)
            R.cr[i] = *reinterpret_cast<const u32x4 *>(cpb + min(clane + (uint32_t)(i * (NT / (N / 8))) * crow, cmax));
        const int sr = s_rel - rel(b), er = e_rel - 1 - rel(b);
        const int lo = sr > -W ? sr : -W;          // first valid row, block-relative
        const int hi = er < L + 8 ? er : L + 8;    // last valid row
        // first x row that holds data: a later segment's context rows are tokens of its sequence
        const int xl = first ? lo : (sr - (W - 1) > -W ? sr - (W - 1) : -W);
        // raw x rows bL - (W-1) + rho, rho in [0, L + W - 1), of this wave's 16 channels
        const char *xc = static_cast<const char *>(a.xbc) + ((bL - (W - 1)) * cdim + (int64_t)head * P + 16 * wv) * XS;
        const uint32_t xlo = (uint32_t)(xl + (W - 1) > 0 ? xl + (W - 1) : 0) * xrow, xhi = (uint32_t)(hi + (W - 1)) * xrow;
#pragma unroll
        for (int k = 0; k < XP; ++k)
            R.xq[k] = *reinterpret_cast<const u32x4 *>(xc + (min(max(xq_off[k], xlo), xhi) + xq_part[k]));
    };
    auto prefetch_ops = [&](int64_t b, Pre &R) __attribute__((always_inline)) {
        const int64_t bL = b * L;
        const int sr = s_rel - rel(b), er = e_rel - 1 - rel(b);
        const int lo = sr > -W ? sr : -W;          // first valid row, block-relative
        const int hi = er < L + 8 ? er : L + 8;    // last valid row
        const char *dtc = static_cast<const char *>(a.dt_raw) + (bL * H + head) * AS;
        R.dtr = *(reinterpret_cast<const AT *>(dtc + min(max(dtlane, (uint32_t)max(lo, 0) * H * AS), (uint32_t)hi * H * AS)));
        const char *cbb = static_cast<const char *>(a.cb) + ((b * G + g) * (int64_t)(TL * KL) + ttw * KL) * 512 * 4;
#pragma unroll
        for (int m = 0; m < KL; ++m)
#pragma unroll
            for (int h = 0; h < MJ / 4; ++h)
                R.cbr[m][h] = *reinterpret_cast<const f32x4 *>(cbb + (lane * 32u + (uint32_t)(m * 2048 + 4 * mj0 + 16 * h)));
    };

    // ---- staging of a block (from the prefetch registers) for the next iteration
    bf16x8 X[KL], XD[KL], XSh[KL], XSl[KL];  // x, x dt, (x w) hi / lo: k-slots 32m + 8q + j of channel p
    float el[TL], dec = 1.0f, l2e = 0.0f;    // exp(lam_t) for t = 16 tt + col; exp(lam_end); lam_end (log2)
    float lsum = 0.0f;                       // log2 of the decay over the blocks computed so far
    // tiles of block b into LDS buffer buf: B^T and C (shared), raw x rows (this wave's)
    auto stage_tiles = [&](int64_t b, int buf, Pre &R) __attribute__((always_inline)) {
        const int64_t bL = b * L;
        // shared tiles
        bf16 *sbt = sBT[buf];
        bf16 *sc = sC[buf];
#pragma unroll
        for (int i = 0; i < BTP; ++i) {
            const int id = tid + i * NT, n = (id / (L / 8)) % N, hl = id / (N * L / 8);
            *reinterpret_cast<u32x4 *>(&sbt[hl * N * BTS + n * BTS + 8 * (id % (L / 8))]) = R.btr[i];
        }
#pragma unroll
        for (int i = 0; i < CPC; ++i) {
            const int id = tid + i * NT;
            *reinterpret_cast<u32x4 *>(&sc[(id / (N / 8)) * CS + 8 * (id % (N / 8))]) = R.cr[i];
        }
        // raw x rows into this wave's tile (lanes past the last piece repeat it)
        char *xt = sXr[wv];
#pragma unroll
        for (int k = 0; k < XP; ++k) {
            const int id = min(lane + 64 * k, CPR * XRW - 1);
            char *d = xt + (id / CPR) * XRB + 16 * (id % CPR);
            *reinterpret_cast<uint2 *>(d) = uint2{R.xq[k][0], R.xq[k][1]};
            *reinterpret_cast<uint2 *>(d + 8) = uint2{R.xq[k][2], R.xq[k][3]};
        }
    };
    // operands of block b (token arrays, conv + SiLU of x, decayed C.B^T into sM[buf])
    auto stage_ops = [&](int64_t b, int buf, Pre &R) __attribute__((always_inline)) {
        const int64_t bL = b * L;
        const int sr = s_rel - rel(b), er = e_rel - rel(b);
        const int lo = sr > 0 ? sr : 0;
        const int hi = er < L ? er : L;
        // sequence start, block-relative (a later segment has none: its context rows are real tokens)
        const int ctxlo = first ? (sr > -W ? sr : -W) : -W;
        // token arrays, every wave its own copy: dt, inclusive lam, dt exp(lam_end - lam)
        {
            // (softplus for every lane, then a multiply by 0 / 1: no branch around it)
            const float dt = softplus_fast((float)R.dtr + dtb) * (lane < L && lane >= lo && lane < hi ? 1.0f : 0.0f);
            const float v = wave_prefix_sum(dt * A2);
            const float l2end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), L - 1));
            sTok[wv][0][lane] = dt;  // lanes >= L fill padding
            sTok[wv][1][lane] = v;
            sTok[wv][2][lane] = dt * __builtin_amdgcn_exp2f(l2end - v);
            dec = __builtin_amdgcn_exp2f(l2end);
            l2e = l2end;
        }
        const char *xt = sXr[wv];  // (rows written by this wave in the tile pass)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int tt = 0; tt < TL; ++tt) el[tt] = __builtin_amdgcn_exp2f(sTok[wv][1][16 * tt + col]);
        // conv + SiLU of this lane's channel, tokens 32m + 8q + j
#pragma unroll
        for (int m = 0; m < KL; ++m) {
            float u[XR];
            const char *xr0 = xt + (32 * m + 8 * q) * XRB + XS * col;
#pragma unroll
            for (int i = 0; i < XR; ++i) {
                if constexpr (XS == 4) u[i] = *reinterpret_cast<const float *>(xr0 + i * XRB);
                else u[i] = bits_f<XT>(*reinterpret_cast<const unsigned short *>(xr0 + i * XRB));
            }
            // rows before the sequence: its cached raw inputs (or zeros), at full precision
            // (post-conv input has no context: those rows only reach their own unstored outputs)
            if (CONV && ctxlo > 1 - W) {
#pragma unroll
                for (int i = 0; i < XR; ++i) {
                    const int d = ctxlo - (32 * m + 8 * q - (W - 1) + i);  // rows before the start
                    if (d > 0) {
                        float c = 0.0f;
#pragma unroll
                        for (int k = 0; k < W - 1; ++k) c = (d == W - 1 - k) ? ctx[k] : c;
                        u[i] = c;
                    }
                }
            }
            const int s0 = 32 * m + 8 * q;
            const f32x4 d0 = *reinterpret_cast<const f32x4 *>(&sTok[wv][0][s0]);
            const f32x4 d1 = *reinterpret_cast<const f32x4 *>(&sTok[wv][0][s0 + 4]);
            const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&sTok[wv][2][s0]);
            const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&sTok[wv][2][s0 + 4]);
            // Tokens outside the sequence need no mask: their dt and state weight are 0,
            // and their x reaches only their own (unstored) output through D x.
            float xv[8], xd[8], xs[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float x = u[j];
                if constexpr (CONV) {
                    float v = cbias;
#pragma unroll
                    for (int k = 0; k < W; ++k) v += cw[k] * u[j + k];
                    x = silu_fast(v);
                }
                xv[j] = x;
                xd[j] = x * (j < 4 ? d0[j] : d1[j - 4]);
                xs[j] = x * (j < 4 ? w0[j] : w1[j - 4]);
            }
            X[m] = cvt8(xv);
            XD[m] = cvt8(xd);
            split8(xs, XSh[m], XSl[m]);
        }
        // decayed C.B^T of t-tile ttw, k-slots [mj0, mj0 + MJ): M[t][s] = CB[t][s] exp(lam_t - lam_s), s <= t
        if (MSPLIT || wv < TL) {
            const int t = 16 * ttw + col;
            const float l2t = sTok[wv][1][t];
#pragma unroll
            for (int m = 0; m < KL; ++m) {
                if (KL > 1 && 2 * m > ttw) break;  // (one 32-token block: always m = 0 <= ttw)
                const int s0 = 32 * m + 8 * q + mj0;
                float mv[MJ];
#pragma unroll
                for (int h = 0; h < MJ / 4; ++h) {
                    const f32x4 ls = *reinterpret_cast<const f32x4 *>(&sTok[wv][1][s0 + 4 * h]);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        mv[4 * h + j] = s0 + 4 * h + j <= t ? R.cbr[m][h][j] * __builtin_amdgcn_exp2f(l2t - ls[j]) : 0.0f;
                }
                bf16 *dst = reinterpret_cast<bf16 *>(&sM[buf][(ttw * KL + m) * 64 + lane]) + mj0;
                if constexpr (MJ == 8) *reinterpret_cast<bf16x8 *>(dst) = cvt8(mv);
                else *reinterpret_cast<bf16x4 *>(dst) = bf16x4{f32_to_bf16(mv[0]), f32_to_bf16(mv[1]), f32_to_bf16(mv[2]), f32_to_bf16(mv[3])};
            }
        }
    };

    if (b0 <= b1) {
        prefetch_tiles(b0, P0);
        prefetch_ops(b0, P0);
        stage_tiles(b0, 0, P0);
        stage_ops(b0, 0, P0);
        prefetch_tiles(b0 + 1 <= b1 ? b0 + 1 : b1, P1);
        prefetch_ops(b0 + 1 <= b1 ? b0 + 1 : b1, P1);
        prefetch_tiles(b0 + 2 <= b1 ? b0 + 2 : b1, P0);
        prefetch_ops(b0 + 2 <= b1 ? b0 + 2 : b1, P0);
        __syncthreads();
    }

    // block b: computes b, stages b + 1 from R (the set that holds it) and loads b + 3 into R
    auto block = [&](int64_t b, Pre &R) __attribute__((always_inline)) {
        const int buf = (int)((b - b0) & 1);
        const int64_t bL = b * L;
        const int sr = s_rel - rel(b), er = e_rel - rel(b);
        const int lo = sr > 0 ? sr : 0;
        const int hi = er < L ? er : L;
        // this block's staged operands (the next stage overwrites the variables)
        bf16x8 Xc[KL], XDc[KL], XShc[KL], XSlc[KL];
        float elc[TL];
        const float decc = dec;
        lsum += l2e;
        if (a.seg && tid == 0 && rel(b) >= s_rel && rel(b) + L <= e_rel) a.seg_lam[b * H + head] = lsum;
#pragma unroll
        for (int m = 0; m < KL; ++m) { Xc[m] = X[m]; XDc[m] = XD[m]; XShc[m] = XSh[m]; XSlc[m] = XSl[m]; }
#pragma unroll
        for (int tt = 0; tt < TL; ++tt) elc[tt] = el[tt];
        const bf16 *sbt = sBT[buf];
        const bf16 *sc = sC[buf];

        Raw<AT, 4> zr[TL];
        if (a.z) {  // gate rows of this block, clamped into the sequence at its edges
            const char *zc = static_cast<const char *>(a.z) + (bL * HP + (int64_t)head * P + 16 * wv) * AS;
            const uint32_t zlo = (uint32_t)lo * zrow, zhi = (uint32_t)(hi - 1) * zrow;
#pragma unroll
            for (int tt = 0; tt < TL; ++tt)
                zr[tt].load(reinterpret_cast<const AT *>(
                    zc + (min(max(col * zrow + (uint32_t)(16 * tt) * zrow, zlo), zhi) + 4 * q * AS)));
        }

        // tiles of the next block into the other buffer, then the tile loads of block b + 3
        // (the last blocks reload themselves, keeping the loads unconditional)
        const int64_t b3 = b + 3 <= b1 ? b + 3 : b1;
        stage_tiles(b < b1 ? b + 1 : b, buf ^ 1, R);
        prefetch_tiles(b3, R);

        // carried-state output: y[t][p] = exp(lam_t) sum_n C_t[n] H[p][n]
        f32x4 acc[TL];
        {
            bf16x8 Hb[KN];
#pragma unroll
            for (int kn = 0; kn < KN; ++kn)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Hb[kn][r] = f32_to_bf16(Hacc[2 * kn][r]);
                    Hb[kn][4 + r] = f32_to_bf16(Hacc[2 * kn + 1][r]);
                }
#pragma unroll
            for (int tt = 0; tt < TL; ++tt) {
                acc[tt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kn = 0; kn < KN; ++kn)
                    acc[tt] = mma(Hb[kn], *reinterpret_cast<const bf16x8 *>(&sc[(16 * tt + col) * CS + 32 * kn + 8 * q]),
                                  acc[tt]);
            }
        }

        // carried state: H^T <- exp(lam_end) H^T + sum_s B^T[n][s] (x w)[s][p]   (3-term split).
        // Issued before the staging below, so the matrix cores work through these while the
        // VALU stages the next block.
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) Hacc[nt] *= decc;
#pragma unroll
        for (int m = 0; m < KL; ++m) {
#pragma unroll
            for (int nt = 0; nt < NTL; ++nt) {
                const int off = (16 * nt + col) * BTS + 32 * m + 8 * q;
                const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(&sbt[off]);
                const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(&sbt[N * BTS + off]);
                Hacc[nt] = mma(bh, XShc[m], Hacc[nt]);
                Hacc[nt] = mma(bl, XShc[m], Hacc[nt]);
                Hacc[nt] = mma(bh, XSlc[m], Hacc[nt]);
            }
        }
        // intra-block output and D x
#pragma unroll
        for (int tt = 0; tt < TL; ++tt) {
            acc[tt] *= elc[tt];
#pragma unroll
            for (int m = 0; m < KL; ++m)
                if (2 * m <= tt) acc[tt] = mma(XDc[m], sM[buf][(tt * KL + m) * 64 + lane], acc[tt]);
            acc[tt] = mma(Xc[tt / 2], Dsel[tt & 1], acc[tt]);
        }
        // operands of the next block (VALU work beside the MFMAs above; the last block restages
        // itself into the unused buffer), then the token and C.B^T loads of block b + 3
        stage_ops(b < b1 ? b + 1 : b, buf ^ 1, R);
        prefetch_ops(b3, R);

        // epilogue
        {
            char *yc = reinterpret_cast<char *>(y + bL * HP + (int64_t)head * P + 16 * wv);
#pragma unroll
            for (int tt = 0; tt < TL; ++tt) {
                const int t = 16 * tt + col;
                float o[4];
                if (a.z) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = acc[tt][r] * silu_fast(zr[tt][r]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = acc[tt][r];
                }
                if (t >= lo && t < hi)
                    *reinterpret_cast<bf16x4 *>(yc + (ylane + (uint32_t)(tt * 16) * (uint32_t)HP * 2)) =
                        bf16x4{f32_to_bf16(o[0]), f32_to_bf16(o[1]), f32_to_bf16(o[2]), f32_to_bf16(o[3])};
            }
        }

        __syncthreads();
    };
    for (int64_t b = b0; b <= b1; b += 2) {
        block(b, P1);
        if (b + 1 <= b1) block(b + 1, P0);
    }

    if (!only) {
        // a segment of a longer sequence: its local final state and total decay, for the fix-up pass
        float *gs = a.seg_state + (((int64_t)blockIdx.y * H + head) * P + p) * N;
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) *reinterpret_cast<f32x4 *>(gs + 16 * nt + 4 * q) = Hacc[nt];
        if (tid == 0) a.seg_dec[(int64_t)blockIdx.y * H + head] = lsum;
        return;
    }
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) {
        const float v[4] = {Hacc[nt][0], Hacc[nt][1], Hacc[nt][2], Hacc[nt][3]};
        store_k<ST, 4>(pool_h + 16 * nt + 4 * q, v);
    }
}

// ---------------------------------------------------------------- segment mode
// With few sequences (nseq * H well under the two workgroups per CU the scan fits),
// a long sequence is cut into up to smax segments of whole 32-token blocks, each at
// least kMinSeg tokens, scanned in parallel: the first from the sequence's initial
// state, the others from zero. The exact result follows from the linearity of the
// recurrence in the state: the true state entering segment v is
//   H_in(v) = sum_{u < v} exp2(lam_u) ... H_u,  built as H <- exp2(lam_u) H + H_u over u,
// (H_u: segment u's local final state, lam_u: its total log2 decay), and the tokens
// of segment v miss exactly exp2(lam_t) C_t . H_in(v) in y (lam_t: log2 decay from
// the segment's start through t), the carried-state output term of the scan.

// True initial state of each later segment (one workgroup of four waves per (head,
// segment), the scan's lane layout: wave w, lane (col, q) holds H[16 w + col][16 nt +
// 4 q + r]), kept as the bf16 A operand of the fix-up MFMAs; for the sequence's last
// segment, the true final state into the pool.
template <typename ST>
__global__ __launch_bounds__(256) void fused_seg_combine_kernel(FusedArgs a, int H, int smax) {
    constexpr int P = 64, N = 128, KN = 4, NTL = 8;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, q = lane >> 4;
    const int head = blockIdx.x, v = blockIdx.y, k = v % smax;
    const int32_t *sg = a.seg + 4 * v;
    if (k == 0 || sg[0] >= sg[1]) return;  // first segments are exact; empty ones hold no tokens
    const int slot = pool_slot(a.idx[sg[2]], a.num_slots, a.err, false);
    if (slot < 0) return;
    const bool last = k + 1 == smax || a.seg[4 * (v + 1)] >= a.seg[4 * (v + 1) + 1];
    const int p = 16 * wv + col;
    // H <- exp2(lam_u) H + H_u over the earlier segments u of the sequence
    f32x4 Hin[NTL];
#pragma unroll
    for (int nt = 0; nt < NTL; ++nt) Hin[nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int u = v - k; u < v; ++u) {
        const float d = __builtin_amdgcn_exp2f(a.seg_dec[(int64_t)u * H + head]);
        const float *gs = a.seg_state + (((int64_t)u * H + head) * P + p) * N;
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) Hin[nt] = Hin[nt] * d + *reinterpret_cast<const f32x4 *>(gs + 16 * nt + 4 * q);
    }
    // the A operand of the carried-state output (k-slots in the permuted n order of the C plane)
    bf16x8 *hb = static_cast<bf16x8 *>(a.seg_hin) + (((int64_t)v * H + head) * 4 + wv) * 64 * KN + lane * KN;
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) {
        bf16x8 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            o[r] = f32_to_bf16(Hin[2 * kn][r]);
            o[4 + r] = f32_to_bf16(Hin[2 * kn + 1][r]);
        }
        hb[kn] = o;
    }
    if (last) {
        const float d = __builtin_amdgcn_exp2f(a.seg_dec[(int64_t)v * H + head]);
        const float *gs = a.seg_state + (((int64_t)v * H + head) * P + p) * N;
        ST *pool_h = static_cast<ST *>(a.pool) + ((int64_t)slot * H + head) * (int64_t)P * N + (int64_t)p * N;
#pragma unroll
        for (int nt = 0; nt < NTL; ++nt) {
            const f32x4 hf = Hin[nt] * d + *reinterpret_cast<const f32x4 *>(gs + 16 * nt + 4 * q);
            const float o[4] = {hf[0], hf[1], hf[2], hf[3]};
            store_k<ST, 4>(pool_h + 16 * nt + 4 * q, o);
        }
    }
}

// y += exp2(lam_t) C_t . H_in (times SiLU(z)) for the tokens of later segments; one
// workgroup per (head, kFixBlocks consecutive 32-token blocks). A block holds tokens of
// at most one later segment: those start at block boundaries and span many blocks.
// Every block's loads are issued the same way (addresses clamped, stores masked, every
// loaded value used on every path), kFixNB - 1 blocks ahead of the block being applied,
// and values are widened only where used, so the compiler's waits count just the loads
// of the block being applied. The block's C rows are read from HBM/L2 once per workgroup
// and shared by its 4 waves through LDS (two buffers, one barrier per block; every wave
// passes every barrier). lam_t only falls along a segment, so once exp2 of it is exactly
// 0 in fp32 every later token of the segment would add exactly 0, and the workgroup
// stops there.
constexpr int kFixBlocks = 16;
constexpr int kFixNB = 3;  // register buffers of the fix-up pass
template <typename AT, bool HasZ>
__global__ __launch_bounds__(256) void fused_seg_fix_kernel(FusedArgs a, int H, int G, int nseg, int smax) {
    constexpr int P = 64, N = 128, L = 32, TL = 2, KN = 4;
    constexpr int CS = N + 16;  // LDS row stride (bf16): 288 bytes, 32 mod 64, keeps the 16-byte operand reads conflict-free
    __shared__ __align__(16) bf16 sC[2][L * CS];
    constexpr float LOG2E = 1.4426950408889634f;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, q = lane >> 4;
    const int head = xcd_head(blockIdx.x, H);
    const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N;
    const int g = head / (H / G);
    const int64_t nblk = (a.T + L - 1) / L;
    const int64_t b0 = (int64_t)blockIdx.y * kFixBlocks, b1 = b0 + kFixBlocks < nblk ? b0 + kFixBlocks : nblk;
    const AT *dtr = static_cast<const AT *>(a.dt_raw);
    const AT *zr = static_cast<const AT *>(a.z);
    const bf16 *cp = static_cast<const bf16 *>(a.cp);
    bf16 *y = static_cast<bf16 *>(a.y);

    // The later segment holding position pos, [sstart, send), with sv its record (-1 if
    // there is none or it is a padding row's); where there is none, send is the start
    // of the next later segment. A scalar search of the few records, run again only
    // once the blocks reach send.
    int sv = -1;
    int64_t sstart = 0, send = -1;
    auto locate = [&](int64_t pos) {
        if (pos < send) return;
        bool found = false;
        int64_t next = INT64_MAX;
        sv = -1;
        for (int u = 0; u < nseg; ++u) {
            const int32_t *sg = a.seg + 4 * u;
            const int64_t s0 = sg[0], s1 = sg[1];
            if (u % smax == 0 || s0 >= s1) continue;  // first segments need no fix; empty records
            if (s0 <= pos && pos < s1) {
                found = true;
                sstart = s0;
                send = s1;
                sv = pool_slot(a.idx[sg[2]], a.num_slots, a.err, false) < 0 ? -1 : u;
            } else if (s0 > pos && s0 < next) {
                next = s0;
            }
        }
        if (!found) {
            sstart = pos;
            send = next;
        }
    };
    if (b0 >= b1) return;
    locate(b0 * L);
    if (sv < 0 && send >= b1 * L) return;  // nothing to fix in these blocks

    struct Blk {
        int64_t bL, send;
        int v, hi;
        bool first;
        float carry;
        AT dtraw;
        u32x4 c[2];  // this thread's 32 bytes of the block's C rows
        bf16x4 yo[TL];
        Raw<AT, 4> zv[TL];
    };
    auto fetch = [&](Blk &k, int64_t b) {
        const int64_t bc = b < b1 ? b : b1 - 1;
        k.bL = bc * L;
        locate(k.bL);
        k.v = b < b1 ? sv : -1;
        const int64_t lim = sv >= 0 ? send : a.T;
        k.hi = (int)(lim - k.bL < L ? lim - k.bL : L);  // >= 1: the block starts inside
        k.first = k.bL == sstart;
        k.send = send;
        k.carry = a.seg_lam[(bc > 0 ? bc - 1 : 0) * H + head];
        k.dtraw = dtr[(k.bL + (lane < k.hi ? lane : k.hi - 1)) * H + head];
        {
            const int row = tid >> 3, rc = row < k.hi ? row : k.hi - 1;  // rows past the segment repeat its last one
            const u32x4 *src = reinterpret_cast<const u32x4 *>(cp + (k.bL + rc) * GN + (int64_t)g * N + (tid & 7) * 16);
            k.c[0] = src[0];
            k.c[1] = src[1];
        }
#pragma unroll
        for (int tt = 0; tt < TL; ++tt) {
            const int t = 16 * tt + col, tc = t < k.hi ? t : k.hi - 1;
            const int64_t off = (k.bL + tc) * HP + (int64_t)head * P + 16 * wv + 4 * q;
            k.yo[tt] = *reinterpret_cast<const bf16x4 *>(y + off);
            if constexpr (HasZ) k.zv[tt].load(zr + off);
        }
    };
    const float A2 = -expf(a.A_log[head]) * LOG2E;
    const float dtb = a.dt_bias[head];
    bf16x8 Hb[KN];
    int hv = -1;
    constexpr float kDead = -160.0f;  // exp2 of anything below is 0 in fp32
    // true: this block and the rest of the workgroup's blocks add nothing (one segment)
    auto done = [&](const Blk &k) {
        const float c = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(k.carry)));
        return k.v >= 0 && !k.first && c < kDead && k.send >= b1 * L;
    };
    auto apply = [&](const Blk &k, bf16 *sc) {
        u32x4 *dst = reinterpret_cast<u32x4 *>(sc + (tid >> 3) * CS + (tid & 7) * 16);
        dst[0] = k.c[0];
        dst[1] = k.c[1];
        __syncthreads();
        // a block with nothing to fix (v < 0) still runs the arithmetic on its loaded values
        // (every load is then used on every path) and only its stores are masked
        if (k.v >= 0 && k.v != hv) {  // a new segment: its H_in (rare, so waiting for it here is fine)
            hv = k.v;
            const bf16x8 *hb = static_cast<const bf16x8 *>(a.seg_hin) + (((int64_t)hv * H + head) * 4 + wv) * 64 * KN + lane * KN;
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) Hb[kn] = hb[kn];
            // used here, so the wait for these loads stays on this path
            asm volatile("" ::"v"(Hb[0]), "v"(Hb[1]), "v"(Hb[2]), "v"(Hb[3]));
        }
        // lam_t: log2 decay from the segment's start through token t
        const float dt = lane < k.hi ? softplus_fast((float)k.dtraw + dtb) : 0.0f;
        const float lam = wave_prefix_sum(dt * A2) + (k.first ? 0.0f : k.carry);
#pragma unroll
        for (int tt = 0; tt < TL; ++tt) {
            const int t = 16 * tt + col;
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kn = 0; kn < KN; ++kn)
                acc = mma(Hb[kn], *reinterpret_cast<const bf16x8 *>(sc + (16 * tt + col) * CS + 32 * kn + 8 * q), acc);
            const float el = __builtin_amdgcn_exp2f(__shfl(lam, t));
            if (k.v >= 0 && t < k.hi) {
                bf16x4 o = k.yo[tt];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float gate = 1.0f;
                    if constexpr (HasZ) gate = silu_fast(k.zv[tt][r]);
                    o[r] = f32_to_bf16((float)o[r] + acc[r] * el * gate);
                }
                *reinterpret_cast<bf16x4 *>(y + (k.bL + t) * HP + (int64_t)head * P + 16 * wv + 4 * q) = o;
            }
        }
    };
    // kFixNB register buffers in turn (a copy of one into another would wait for its loads):
    // block b + kFixNB - 1 is fetched into the buffer block b - 1 has just left, so kFixNB - 1
    // blocks' loads are in flight while one is applied; LDS buffers alternate by block.
    Blk kb[kFixNB];
#pragma unroll
    for (int i = 0; i < kFixNB - 1; ++i) fetch(kb[i], b0 + i);
    // straight-line over the workgroup's blocks (blocks past b1 are clamped and masked), so
    // the compiler's wait counts follow the buffers exactly
#pragma unroll
    for (int j = 0; j < kFixBlocks; ++j) {
        fetch(kb[(j + kFixNB - 1) % kFixNB], b0 + j + kFixNB - 1);
        if (done(kb[j % kFixNB])) return;  // the rest of the blocks add exactly 0 (uniform: every wave returns)
        apply(kb[j % kFixNB], sC[j & 1]);
    }
}

// ---------------------------------------------------------------- launch
namespace {

constexpr int kFusedL = 32;

int64_t up256(int64_t v) { return (v + 255) / 256 * 256; }

struct FusedLayout {
    int64_t nblk, cp, bt, cb, seg, segdec, segstate, seglam, seghin, bytes;  // block count and byte offsets / total
};

// Segments the segment mode may use: nseq * smax <= 512 / H (see seg_max), and only
// from 2 * kMinSeg tokens; their states take at most 512 * P * N * 4 bytes (16 MiB at
// P = 64, N = 128).
int64_t max_segments(const LayerShape &s, int64_t T) { return T >= 2 * kMinSeg ? 512 / s.H : 0; }

FusedLayout fused_layout(const LayerShape &s, int64_t T) {
    FusedLayout f;
    const int64_t L = kFusedL;
    const int64_t nv = max_segments(s, T);
    f.nblk = (T + L - 1) / L;
    f.cp = 0;
    f.bt = up256(T * s.G * s.N * 2);
    f.cb = f.bt + up256(f.nblk * s.G * 2 * s.N * L * 2);
    f.seg = f.cb + up256(f.nblk * s.G * L * L * 4);
    f.segdec = f.seg + up256(nv * 4 * 4);
    f.segstate = f.segdec + up256(nv * s.H * 4);
    f.seglam = f.segstate + up256(nv * s.H * s.P * s.N * 4);
    f.seghin = f.seglam + up256(nv ? f.nblk * s.H * 4 : 0);
    f.bytes = f.seghin + up256(nv * s.H * s.P * s.N * 2);
    return f;
}

// Segments per sequence for a batch of few sequences (0: one workgroup per sequence): while
// nseq * H streams leave at least half the 512 workgroup slots (two per CU) empty.
int seg_max(const LayerShape &s, const FusedArgs &a) {
    if (a.T < 2 * kMinSeg || (int64_t)a.nseq * s.H > 256) return 0;
    const int smax = (int)std::min<int64_t>(8, 512 / ((int64_t)a.nseq * s.H));
    return smax >= 2 ? smax : 0;
}

// W == 1: post-conv xbc of type XT (chunk scan alone); W >= 2: raw xbc of type AT
template <int W, typename ST, typename AT, typename XT>
hipError_t launch_fw(const LayerShape &s, const FusedArgs &a, int64_t nblk, int smax, hipStream_t stream) {
    hipError_t e;
    // (segment mode needs tokens, so the prep kernel, which writes its plan, always runs then)
    if (nblk > 0) {  // no tokens (only empty sequences): the scan alone writes their states
        hipLaunchKernelGGL((fused_prep_kernel<XT, ST, W, kFusedL>), dim3((unsigned)nblk, s.G), dim3(256), 0, stream, a,
                           s.H, s.G, smax);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((fused_scan_kernel<kFusedL, W, ST, AT, XT>), dim3(s.H, smax ? a.nseq * smax : a.nseq), dim3(256),
                       0, stream, a, s.H, s.G);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (smax && nblk > 0) {
        const int nv = a.nseq * smax;
        hipLaunchKernelGGL((fused_seg_combine_kernel<ST>), dim3(s.H, nv), dim3(256), 0, stream, a, s.H, smax);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const dim3 fg(s.H, (unsigned)((nblk + kFixBlocks - 1) / kFixBlocks));
        if (a.z)
            hipLaunchKernelGGL((fused_seg_fix_kernel<AT, true>), fg, dim3(256), 0, stream, a, s.H, s.G, nv, smax);
        else
            hipLaunchKernelGGL((fused_seg_fix_kernel<AT, false>), fg, dim3(256), 0, stream, a, s.H, s.G, nv, smax);
        e = hipGetLastError();
    }
    return e;
}

template <typename ST, typename AT>
hipError_t launch_fa(const LayerShape &s, const FusedArgs &a, int64_t nblk, int smax, hipStream_t stream) {
    switch (s.W) {
        case 2: return launch_fw<2, ST, AT, AT>(s, a, nblk, smax, stream);
        case 3: return launch_fw<3, ST, AT, AT>(s, a, nblk, smax, stream);
        case 4: return launch_fw<4, ST, AT, AT>(s, a, nblk, smax, stream);
        default: return hipErrorInvalidValue;
    }
}

// Workspace planes, and the segment arrays when the batch runs in segment mode
// (*smax > 0; a.seg stays null otherwise).
void set_workspace(const LayerShape &s, FusedArgs &a, void *workspace, int64_t *nblk, int *smax) {
    const FusedLayout f = fused_layout(s, a.T);
    char *ws = static_cast<char *>(workspace);
    a.cp = ws ? ws + f.cp : nullptr;
    a.bt = ws ? ws + f.bt : nullptr;
    a.cb = ws ? ws + f.cb : nullptr;
    *nblk = f.nblk;
    *smax = ws ? seg_max(s, a) : 0;
    a.seg = *smax ? reinterpret_cast<const int32_t *>(ws + f.seg) : nullptr;
    a.seg_dec = *smax ? reinterpret_cast<float *>(ws + f.segdec) : nullptr;
    a.seg_state = *smax ? reinterpret_cast<float *>(ws + f.segstate) : nullptr;
    a.seg_lam = *smax ? reinterpret_cast<float *>(ws + f.seglam) : nullptr;
    a.seg_hin = *smax ? static_cast<void *>(ws + f.seghin) : nullptr;
}

}  // namespace

bool prefill_fused_supported(const LayerShape &s) {
    return s.P == 64 && s.N == 128 && s.W >= 2 && s.W <= 4 && s.out_dt == DT_BF16 && s.H % s.G == 0;
}

bool chunk_scan_blocks_supported(const LayerShape &s) {
    return s.P == 64 && s.N == 128 && s.out_dt == DT_BF16 && s.act_dt == DT_BF16 && s.H % s.G == 0;
}

int64_t fused_workspace_bytes(const LayerShape &s, int64_t T) { return fused_layout(s, T).bytes; }

hipError_t launch_fused_prefill(const LayerShape &s, FusedArgs a, void *workspace, hipStream_t stream) {
    if (a.nseq == 0) return hipSuccess;
    int64_t nblk = 0;
    int smax = 0;
    set_workspace(s, a, workspace, &nblk, &smax);
    if (s.state_dt == DT_BF16)
        return s.act_dt == DT_BF16 ? launch_fa<bf16, bf16>(s, a, nblk, smax, stream)
                                   : launch_fa<bf16, float>(s, a, nblk, smax, stream);
    return s.act_dt == DT_BF16 ? launch_fa<float, bf16>(s, a, nblk, smax, stream)
                               : launch_fa<float, float>(s, a, nblk, smax, stream);
}

hipError_t launch_block_scan(const LayerShape &s, FusedArgs a, void *workspace, hipStream_t stream) {
    if (a.nseq == 0) return hipSuccess;
    int64_t nblk = 0;
    int smax = 0;
    set_workspace(s, a, workspace, &nblk, &smax);
    if (s.state_dt == DT_BF16)
        return s.xbc_dt == DT_BF16 ? launch_fw<1, bf16, bf16, bf16>(s, a, nblk, smax, stream)
                                   : launch_fw<1, bf16, bf16, float>(s, a, nblk, smax, stream);
    return s.xbc_dt == DT_BF16 ? launch_fw<1, float, bf16, bf16>(s, a, nblk, smax, stream)
                               : launch_fw<1, float, bf16, float>(s, a, nblk, smax, stream);
}

}  // namespace m2
