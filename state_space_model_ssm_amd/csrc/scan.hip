// Chunked SSD scan for prefill on gfx950 (MFMA), varlen over cu_seqlens.
//
// The "Nemotron-H-8B-Base-8K" record (section "REQUIRED KERNEL CLASS") asks
// for a chunked scan kernel for the SSM layers; the recurrence itself is a
// multiplicative chain, so only the chunk-local pieces are dense
// contractions. Per chunk of L tokens of one (sequence, head), with
// lam_t = sum_{r <= t in chunk} dt_r * A (inclusive):
//
//   CB^T[s][t] = sum_n B_s[n] C_t[n]                                   (MFMA)
//   Md^T[s][t] = CB^T[s][t] * exp(lam_t - lam_s), s <= t               (registers)
//   Yd^T[p][t] = sum_s (dt_s x_s[p]) Md^T[s][t]                        (MFMA, intra-chunk)
//   Yo^T[p][t] = exp(lam_t) sum_n H[p][n] C_t[n]                       (MFMA, carried state)
//   y_t[p]     = Yd + Yo + D x_t[p]   (x SiLU(z) when z is given)
//   H         <- exp(lam_end) H + sum_s (dt_s exp(lam_end - lam_s) x_s[p]) B_s[n]   (MFMA)
//
// which equals the token-by-token recurrence in exact arithmetic (unrolling
// h_t = a_t h_{t-1} + dt_t x_t B_t^T over the chunk).
//
// Design (one workgroup of NW wavefronts per (sequence, head), looping over
// the sequence's chunks in order):
//   * The carried state H [P][N] fp32 lives in MFMA accumulator registers for
//     the whole sequence (the inter-chunk pass is the loop itself), so chunk
//     states never touch HBM; the only traffic is x/B/C/dt in, y out, and the
//     initial/final state.
//   * C.B^T is computed transposed: two stacked 16x16 accumulator tiles are
//     exactly the B operand of the next v_mfma_f32_16x16x32_bf16 in a
//     permuted k order, so the decay-masked matrix never goes through LDS.
//     x is staged in LDS transposed in that same permuted token order; the
//     per-token weights (dt for the output, dt * exp(lam_end - lam) for the
//     state) are applied as the fragments are fetched.
//   * Software pipeline: the next chunk's x, B, C fragments and dt are loaded
//     into registers while the current chunk computes, so global latency is
//     hidden behind MFMA work; with 8 wavefronts (two per SIMD) at chunk 128
//     LDS and MFMA latencies of one wave hide behind the other. t-tiles are
//     assigned so each SIMD gets the same causal work.
//   * Precision: MFMA operands are bf16. The chunk-state contraction (the only
//     path into the carried state) always uses a 3-term hi/lo split
//     (hi*hi + hi*lo + lo*hi), which keeps fp32-level accuracy; the output
//     contractions use the split only when y is stored in fp32 (PRECISE),
//     single bf16 operands otherwise.
//   * Ragged tails are zero padded (dt = 0 keeps lam flat, x = B = C = 0 adds
//     nothing); only valid rows are stored.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace m2 {

template <int P, int N, int L, int NW, typename ST, typename XT, bool PRECISE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void chunk_scan_kernel(ScanArgs a, int H, int G, int act_dt, int out_dt) {
    constexpr int NT = NW * 64;
    constexpr int TP = P / 16, TN = N / 16, TL = L / 16;
    constexpr int KN = (N + 31) / 32, KL = (L + 31) / 32;
    constexpr int LP = KL * 32, NP = KN * 32;
    constexpr int XS = LP + 4;  // sXT row stride (floats)
    constexpr int BS = NP + 4;  // sB row stride (floats)
    constexpr int HS = NP + 8;  // sH row stride (bf16)
    constexpr int NJ = (TN + NW - 1) / NW;  // n-tiles of H per wave
    constexpr int TW = (TL + NW - 1) / NW;  // t-tiles of y per wave
    constexpr int XV = P / 4, BV = N / 4;   // 4-element groups per token row of x / B
    constexpr int XI = (LP * XV + NT - 1) / NT;
    constexpr int BI = (LP * BV + NT - 1) / NT;
    constexpr int LB = (LP + 63) / 64;      // 64-token blocks of the lam scan
    static_assert(P % 16 == 0 && N % 16 == 0 && L % 16 == 0, "tile multiples");

    __shared__ __attribute__((aligned(16))) float sXT[P * XS];  // x (unscaled), [p][pos(s)]
    __shared__ __attribute__((aligned(16))) float sB[LP * BS];  // B natural [s][n]
    __shared__ __attribute__((aligned(16))) bf16 sHhi[P * HS];
    __shared__ __attribute__((aligned(16))) bf16 sHlo[PRECISE ? P * HS : 8];
    __shared__ float sLam[LP];                                  // lam, natural order
    __shared__ __attribute__((aligned(16))) float sDtP[LP];     // dt, permuted order
    __shared__ __attribute__((aligned(16))) float sWsP[LP];     // dt * exp(lam_end - lam), permuted

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    __shared__ int sSeq;
    const int head = xcd_head(blockIdx.x, H), seq = seq_longest_first(a.cu, a.nseq, blockIdx.y, tid, NT, &sSeq);
    const int64_t HP = (int64_t)H * P;
    const int64_t cdim = HP + 2LL * G * N;
    const int g = head / (H / G);
    const int64_t start = a.cu[seq], end = a.cu[seq + 1];
    const int slot = pool_slot(a.idx[seq], a.num_slots, a.err, head == 0 && tid == 0);
    const int64_t offX = (int64_t)head * P;
    const int64_t offB = HP + (int64_t)g * N;
    const int64_t offC = HP + (int64_t)G * N + (int64_t)g * N;

    if (slot < 0) {  // padding sequence: y rows are zero, no state access
        for (int64_t i = tid; i < (end - start) * P; i += NT)
            st(a.y, out_dt, (start + i / P) * HP + offX + (i % P), 0.0f);
        return;
    }

    const float A = -expf(a.A_log[head]);
    const float dtb = a.dt_bias[head];
    const float Dh = a.D[head];
    const XT *xbc = static_cast<const XT *>(a.xbc);
    ST *pool_tile = static_cast<ST *>(a.pool) + ((int64_t)slot * H + head) * (int64_t)P * N;
    const bool init = a.has_init && a.has_init[seq];

    // Carried state, D layout: Hacc[pt][j] holds H[16pt + 4q + r][16nt + col], nt = wave + j*NW.
    f32x4 Hacc[TP][NJ];
#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int nt = wave + j * NW;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = 0.0f;
                if (init && nt < TN) v = (float)pool_tile[(int64_t)(16 * pt + 4 * q + r) * N + 16 * nt + col];
                Hacc[pt][j][r] = v;
            }
        }

    // Zero the padding columns n in [N, NP) of sB and sH once; they are never rewritten.
    if constexpr (NP > N) {
        for (int i = tid; i < LP * (NP - N); i += NT) sB[(i / (NP - N)) * BS + N + i % (NP - N)] = 0.0f;
        for (int i = tid; i < P * (NP - N); i += NT) {
            sHhi[(i / (NP - N)) * HS + N + i % (NP - N)] = f32_to_bf16(0.0f);
            if constexpr (PRECISE) sHlo[(i / (NP - N)) * HS + N + i % (NP - N)] = f32_to_bf16(0.0f);
        }
        __syncthreads();
    }

    auto write_sH = [&]() {
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int nt = wave + j * NW;
                if (nt < TN) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int idx = (16 * pt + 4 * q + r) * HS + 16 * nt + col;
                        const float v = Hacc[pt][j][r];
                        const bf16 hi = f32_to_bf16(v);
                        sHhi[idx] = hi;
                        if constexpr (PRECISE) sHlo[idx] = f32_to_bf16(v - (float)hi);
                    }
                }
            }
    };
    write_sH();

    // ---------------- prefetch registers (next chunk)
    float xr[XI][4], br[BI][4], cr[TW][KN][8], dtr[LB];
    auto prefetch = [&](int64_t c0, int cl) {
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int id = tid + i * NT, s = id / XV, g4 = id - (id / XV) * XV;
            if (id < LP * XV && s < cl) load_k<XT, 4>(xbc + (c0 + s) * cdim + offX + 4 * g4, xr[i]);
            else xr[i][0] = xr[i][1] = xr[i][2] = xr[i][3] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const int id = tid + i * NT, s = id / BV, g4 = id - (id / BV) * BV;
            if (id < LP * BV && s < cl) load_k<XT, 4>(xbc + (c0 + s) * cdim + offB + 4 * g4, br[i]);
            else br[i][0] = br[i][1] = br[i][2] = br[i][3] = 0.0f;
        }
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const int tt = ttile_of<TL, NW>(wave, w);
            const int t = 16 * tt + col;
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) {
                const int k0 = kn * 32 + q * 8;
                if (tt < TL && t < cl && k0 < N) load_k<XT, 8>(xbc + (c0 + t) * cdim + offC + k0, cr[w][kn]);
                else
#pragma unroll
                    for (int j = 0; j < 8; ++j) cr[w][kn][j] = 0.0f;
            }
        }
        if (wave == 0) {
#pragma unroll
            for (int b = 0; b < LB; ++b) {
                const int t = b * 64 + lane;
                dtr[b] = (t < cl) ? ld(a.dt_raw, act_dt, (c0 + t) * H + head) : 0.0f;
            }
        }
    };

    if (start < end) prefetch(start, (int)((end - start) < L ? (end - start) : L));

    for (int64_t c0 = start; c0 < end; c0 += L) {
        const int cl = (int)((end - c0) < L ? (end - c0) : L);

        // ---------------- stage this chunk (registers -> LDS)
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int id = tid + i * NT, s = id / XV, g4 = id - (id / XV) * XV;
            if (id < LP * XV) {
                const int pos = pos_of(s);
#pragma unroll
                for (int j = 0; j < 4; ++j) sXT[(4 * g4 + j) * XS + pos] = xr[i][j];
            }
        }
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const int id = tid + i * NT, s = id / BV, g4 = id - (id / BV) * BV;
            if (id < LP * BV) Io<float>::store(&sB[s * BS + 4 * g4], br[i]);
        }
        if (wave == 0) {
            // lam = inclusive cumsum of dt*A; weights for the output and the state
            float carry = 0.0f, lamv[LB], dtv[LB];
#pragma unroll
            for (int b = 0; b < LB; ++b) {
                const int t = b * 64 + lane;
                const float dtt = (t < cl) ? softplus_f(dtr[b] + dtb) : 0.0f;
                float v = dtt * A;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_up(v, off, 64);
                    if (lane >= off) v += o;
                }
                v += carry;
                lamv[b] = v;
                dtv[b] = dtt;
                carry = __shfl(v, 63, 64);
            }
            const float lam_end = __shfl(lamv[(LP - 1) / 64], (LP - 1) % 64, 64);
#pragma unroll
            for (int b = 0; b < LB; ++b) {
                const int t = b * 64 + lane;
                if (t < LP) {
                    sLam[t] = lamv[b];
                    sDtP[pos_of(t)] = dtv[b];
                    sWsP[pos_of(t)] = dtv[b] * expf(lam_end - lamv[b]);
                }
            }
        }
        bf16x8 Chi[TW][KN];
        bf16x8 Clo[PRECISE ? TW : 1][PRECISE ? KN : 1];
#pragma unroll
        for (int w = 0; w < TW; ++w)
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) {
                if constexpr (PRECISE) split8(cr[w][kn], Chi[w][kn], Clo[w][kn]);
                else Chi[w][kn] = cvt8(cr[w][kn]);
            }
        __syncthreads();

        // next chunk's loads fly while this one computes
        if (c0 + L < end) prefetch(c0 + L, (int)((end - c0 - L) < L ? (end - c0 - L) : L));

        // ---------------- outputs of this wave's t-tiles
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const int tt = ttile_of<TL, NW>(wave, w);
            if (tt >= TL) break;
            const int t = 16 * tt + col;
            const float lam_t = sLam[t];

            // acc = exp(lam_t) * Yo^T first (carried state: sum_n H[p][n] C_t[n]) ...
            f32x4 acc[TP];
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) acc[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) {
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const int idx = (16 * pt + col) * HS + kn * 32 + q * 8;
                    const bf16x8 hh = *reinterpret_cast<const bf16x8 *>(&sHhi[idx]);
                    acc[pt] = mma(hh, Chi[w][kn], acc[pt]);
                    if constexpr (PRECISE) {
                        const bf16x8 hl = *reinterpret_cast<const bf16x8 *>(&sHlo[idx]);
                        acc[pt] = mma(hh, Clo[w][kn], acc[pt]);
                        acc[pt] = mma(hl, Chi[w][kn], acc[pt]);
                    }
                }
            }
            const float elam = expf(lam_t);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) acc[pt] *= elam;

            // ... then the intra-chunk part, one 32-token block of s at a time:
            // CB^T tiles (2m, 2m+1) -> decay mask -> B operand of Yd^T[p][t] += (dt x)^T Md^T
#pragma unroll
            for (int m = 0; m < KL; ++m) {
                if (2 * m > tt) break;
                f32x4 cb[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int si = 2 * m + h2;
                    cb[h2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    if (si < TL && si <= tt) {
#pragma unroll
                        for (int kn = 0; kn < KN; ++kn) {
                            float v[8];
                            ld8f(&sB[(16 * si + col) * BS + kn * 32 + q * 8], v);
                            if constexpr (PRECISE) {
                                bf16x8 bh, bl;
                                split8(v, bh, bl);
                                cb[h2] = mma(bh, Chi[w][kn], cb[h2]);
                                cb[h2] = mma(bh, Clo[w][kn], cb[h2]);
                                cb[h2] = mma(bl, Chi[w][kn], cb[h2]);
                            } else {
                                cb[h2] = mma(cvt8(v), Chi[w][kn], cb[h2]);
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int s = 16 * si + 4 * q + r;
                            cb[h2][r] = (s <= t) ? cb[h2][r] * expf(lam_t - sLam[s]) : 0.0f;
                        }
                    }
                }
                float mv[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    mv[r] = cb[0][r];
                    mv[4 + r] = cb[1][r];
                }
                bf16x8 mh, ml;
                if constexpr (PRECISE) split8(mv, mh, ml);
                else mh = cvt8(mv);
                float dtw[8];
                ld8f(&sDtP[32 * m + q * 8], dtw);
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    float xv[8];
                    ld8f(&sXT[(16 * pt + col) * XS + 32 * m + q * 8], xv);
#pragma unroll
                    for (int j = 0; j < 8; ++j) xv[j] *= dtw[j];
                    if constexpr (PRECISE) {
                        bf16x8 xh, xl;
                        split8(xv, xh, xl);
                        acc[pt] = mma(xh, mh, acc[pt]);
                        acc[pt] = mma(xh, ml, acc[pt]);
                        acc[pt] = mma(xl, mh, acc[pt]);
                    } else {
                        acc[pt] = mma(cvt8(xv), mh, acc[pt]);
                    }
                }
            }
            // epilogue: x comes back from LDS (unscaled, permuted column of token t)
            if (t < cl) {
                const int64_t tok = c0 + t;
                const int pt_col = pos_of(t);
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    float o[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int p = 16 * pt + 4 * q + r;
                        float v = acc[pt][r] + Dh * sXT[p * XS + pt_col];
                        if (a.z) v *= silu_f(ld(a.z, act_dt, tok * HP + offX + p));
                        o[r] = v;
                    }
                    const int64_t yo_idx = tok * HP + offX + 16 * pt + 4 * q;
                    if (out_dt == DT_BF16) store_k<bf16, 4>(static_cast<bf16 *>(a.y) + yo_idx, o);
                    else store_k<float, 4>(static_cast<float *>(a.y) + yo_idx, o);
                }
            }
        }

        // ---------------- carried state: H <- exp(lam_end) H + sum_s (dt w x)^T B
        {
            const float dec = expf(sLam[LP - 1]);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Hacc[pt][j] *= dec;
#pragma unroll
            for (int m = 0; m < KL; ++m) {
                bf16x8 bh[NJ], bl[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int n = 16 * (wave + j * NW) + col;
                    float v[8];
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const int s = 32 * m + tok_of_slot(q, jj);
                        v[jj] = (n < NP) ? sB[s * BS + (n < NP ? n : 0)] : 0.0f;
                    }
                    split8(v, bh[j], bl[j]);
                }
                float ws[8];
                ld8f(&sWsP[32 * m + q * 8], ws);
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    float xv[8];
                    ld8f(&sXT[(16 * pt + col) * XS + 32 * m + q * 8], xv);
#pragma unroll
                    for (int j = 0; j < 8; ++j) xv[j] *= ws[j];
                    bf16x8 xh, xl;
                    split8(xv, xh, xl);
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        if (wave + j * NW < TN) {
                            Hacc[pt][j] = mma(xh, bh[j], Hacc[pt][j]);
                            Hacc[pt][j] = mma(xh, bl[j], Hacc[pt][j]);
                            Hacc[pt][j] = mma(xl, bh[j], Hacc[pt][j]);
                        }
                    }
                }
            }
        }
        __syncthreads();
        write_sH();
    }

    // final state -> pool slot
#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int nt = wave + j * NW;
            if (nt < TN) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Io<ST>::put(pool_tile, (int64_t)(16 * pt + 4 * q + r) * N + 16 * nt + col, Hacc[pt][j][r]);
            }
        }
}

// ---------------------------------------------------------------------------
// Fast path for the Nemotron-H head shape (P = 64, N = 128) when y is stored in
// bf16. Same algorithm as chunk_scan_kernel, restructured so the bf16 operand
// planes are produced once per chunk instead of once per fragment fetch:
//   * staging writes x*dt (hi), x*dt*w (hi, lo) and B (hi, lo) as bf16 planes,
//     so every MFMA operand is a single 16-byte LDS read with no conversion;
//   * the per-token arrays (lam in log2 units, dt, w = dt*exp(lam_end - lam))
//     are double-buffered: wave 0 builds the next chunk's while the current
//     chunk computes, so staging can apply the weights right away;
//   * decays are exp2 of log2-domain differences (one v_exp_f32 each);
//   * x for the D*x term is re-read from global (L2) at the start of each
//     t-tile, overlapping the carried-state MFMAs.
// The state contraction keeps its 3-term split; the output contractions use
// single bf16 operands (y is bf16).
template <int L, int NW, typename ST, typename XT, typename AT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void chunk_scan_fast_kernel(ScanArgs a, int H, int G) {
    constexpr int P = 64, N = 128;
    constexpr int NT = NW * 64;
    constexpr int TP = P / 16, TN = N / 16, TL = L / 16;
    constexpr int KN = N / 32, KL = L / 32;
    constexpr int XSb = L + 8;  // bf16 row stride of the x planes [p][pos(s)]
    constexpr int NSb = N + 8;  // bf16 row stride of the B planes [s][n] and of H [p][n]
    constexpr int NJ = TN / NW;
    constexpr int TW = (TL + NW - 1) / NW;
    constexpr int XT2 = (L / 2) * (P / 4);  // x tasks: (token pair, 4 channels)
    constexpr int XI = (XT2 + NT - 1) / NT;
    constexpr int BI = (L * (N / 4) + NT - 1) / NT;
    constexpr int LB = (L + 63) / 64;
    constexpr float LOG2E = 1.4426950408889634f;
    static_assert(L % 32 == 0 && TN % NW == 0, "fast path shape");
    static_assert(XT2 % NT == 0 && (L * (N / 4)) % NT == 0 && TL % NW == 0, "loads divide evenly over threads");

    __shared__ __attribute__((aligned(16))) bf16 sXD[P * XSb];
    __shared__ __attribute__((aligned(16))) bf16 sXSh[P * XSb];
    __shared__ __attribute__((aligned(16))) bf16 sXSl[P * XSb];
    __shared__ __attribute__((aligned(16))) bf16 sBh[L * NSb];
    __shared__ __attribute__((aligned(16))) bf16 sBl[L * NSb];
    __shared__ __attribute__((aligned(16))) bf16 sHh[P * NSb];
    __shared__ __attribute__((aligned(16))) float sL2[2][L];
    __shared__ __attribute__((aligned(16))) float sDt[2][L];
    __shared__ __attribute__((aligned(16))) float sW[2][L];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    __shared__ int sSeq;
    const int head = xcd_head(blockIdx.x, H), seq = seq_longest_first(a.cu, a.nseq, blockIdx.y, tid, NT, &sSeq);
    const int64_t HP = (int64_t)H * P;
    const int64_t cdim = HP + 2LL * G * N;
    const int g = head / (H / G);
    const int64_t start = a.cu[seq], end = a.cu[seq + 1];
    const int slot = pool_slot(a.idx[seq], a.num_slots, a.err, head == 0 && tid == 0);
    const int64_t offX = (int64_t)head * P;
    const int64_t offB = HP + (int64_t)g * N;
    const int64_t offC = HP + (int64_t)G * N + (int64_t)g * N;
    bf16 *y = static_cast<bf16 *>(a.y);

    if (slot < 0) {
        for (int64_t i = tid; i < (end - start) * P; i += NT) y[(start + i / P) * HP + offX + (i % P)] = f32_to_bf16(0.0f);
        return;
    }

    const float A = -expf(a.A_log[head]);
    const float dtb = a.dt_bias[head];
    const float Dh = a.D[head];
    const XT *xbc = static_cast<const XT *>(a.xbc);
    ST *pool_tile = static_cast<ST *>(a.pool) + ((int64_t)slot * H + head) * (int64_t)P * N;
    const bool init = a.has_init && a.has_init[seq];

    f32x4 Hacc[TP][NJ];
#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Hacc[pt][j][r] = init ? (float)pool_tile[(int64_t)(16 * pt + 4 * q + r) * N + 16 * (wave + j * NW) + col]
                                      : 0.0f;

    auto write_sH = [&]() {
#pragma unroll
        for (int pt = 0; pt < TP; ++pt)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sHh[(16 * pt + 4 * q + r) * NSb + 16 * (wave + j * NW) + col] = f32_to_bf16(Hacc[pt][j][r]);
    };

    // Prefetch of a chunk into registers. Every load is unconditional: rows past
    // the chunk's valid length are clamped to its last valid row and zeroed when
    // staged, so no load sits behind a branch (a branch join would force a wait
    // on every load in flight).
    float xr[XI][2][4], br[BI][4], cr[TW][KN][8], dtr[LB];
    auto prefetch = [&](int64_t c0, int cl) {
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int id = tid + i * NT, sp = id / (P / 4), g4 = id % (P / 4);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int s = min(2 * sp + u, cl - 1);
                load_k<XT, 4>(xbc + (c0 + s) * cdim + offX + 4 * g4, xr[i][u]);
            }
        }
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const int id = tid + i * NT, s = min(id / (N / 4), cl - 1), g4 = id % (N / 4);
            load_k<XT, 4>(xbc + (c0 + s) * cdim + offB + 4 * g4, br[i]);
        }
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const int t = min(16 * ttile_of<TL, NW>(wave, w) + col, cl - 1);
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) load_k<XT, 8>(xbc + (c0 + t) * cdim + offC + kn * 32 + q * 8, cr[w][kn]);
        }
        if (wave == 0) {
#pragma unroll
            for (int b = 0; b < LB; ++b) {
                const int t = min(b * 64 + lane, cl - 1);
                dtr[b] = (float)static_cast<const AT *>(a.dt_raw)[(c0 + t) * H + head];
            }
        }
    };
    // wave 0: lam (log2 units), dt and state weights of a chunk into buffer `buf`. The other
    // waves meet wave 0 at the barrier after this, so it stays short: hardware exp2 / log2
    // softplus and DPP prefix sums (no LDS round trips).
    const float A2 = A * LOG2E;
    auto token_arrays = [&](int buf, int cl) {
        float carry = 0.0f, l2v[LB], dtv[LB];
#pragma unroll
        for (int b = 0; b < LB; ++b) {
            const int t = b * 64 + lane;
            const float dtt = (t < cl) ? softplus_fast(dtr[b] + dtb) : 0.0f;
            const float v = wave_prefix_sum(dtt * A2) + carry;
            l2v[b] = v;
            dtv[b] = dtt;
            carry = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
        }
        const float l2end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l2v[(L - 1) / 64]), (L - 1) % 64));
#pragma unroll
        for (int b = 0; b < LB; ++b) {
            const int t = b * 64 + lane;
            if (t < L) {
                sL2[buf][t] = l2v[b];
                sDt[buf][t] = dtv[b];
                sW[buf][t] = dtv[b] * __builtin_amdgcn_exp2f(l2end - l2v[b]);
            }
        }
    };

    write_sH();
    if (start < end) {
        const int cl0 = (int)((end - start) < L ? (end - start) : L);
        prefetch(start, cl0);
        if (wave == 0) token_arrays(0, cl0);
    }
    __syncthreads();

    int buf = 0;
    for (int64_t c0 = start; c0 < end; c0 += L, buf ^= 1) {
        const int cl = (int)((end - c0) < L ? (end - c0) : L);
        const float *dtp = sDt[buf], *wp = sW[buf], *l2p = sL2[buf];

        // ---------------- stage: registers -> bf16 planes
#pragma unroll
        for (int i = 0; i < XI; ++i) {
            const int id = tid + i * NT;
            if (id < XT2) {
                const int sp = id / (P / 4), g4 = id % (P / 4), s0 = 2 * sp;
                const float d0 = dtp[s0], d1 = dtp[s0 + 1], w0 = wp[s0], w1 = wp[s0 + 1];
                const int pos = pos_of(s0);  // s0 even: s0 + 1 sits at pos + 1
                const bool ok0 = s0 < cl, ok1 = s0 + 1 < cl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int idx = (4 * g4 + j) * XSb + pos;
                    const float v0 = ok0 ? xr[i][0][j] : 0.0f, v1 = ok1 ? xr[i][1][j] : 0.0f;
                    const float s0v = v0 * w0, s1v = v1 * w1;
                    const bf16 h0 = f32_to_bf16(s0v), h1 = f32_to_bf16(s1v);
                    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                    *reinterpret_cast<bf16x2 *>(&sXD[idx]) = bf16x2{f32_to_bf16(v0 * d0), f32_to_bf16(v1 * d1)};
                    *reinterpret_cast<bf16x2 *>(&sXSh[idx]) = bf16x2{h0, h1};
                    *reinterpret_cast<bf16x2 *>(&sXSl[idx]) =
                        bf16x2{f32_to_bf16(s0v - (float)h0), f32_to_bf16(s1v - (float)h1)};
                }
            }
        }
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const int id = tid + i * NT, s = id / (N / 4), g4 = id % (N / 4);
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 hi, lo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v = s < cl ? br[i][j] : 0.0f;
                hi[j] = f32_to_bf16(v);
                lo[j] = f32_to_bf16(v - (float)hi[j]);
            }
            *reinterpret_cast<bf16x4 *>(&sBh[s * NSb + 4 * g4]) = hi;
            *reinterpret_cast<bf16x4 *>(&sBl[s * NSb + 4 * g4]) = lo;
        }
        bf16x8 Chi[TW][KN];
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const bool okc = 16 * ttile_of<TL, NW>(wave, w) + col < cl;
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) {
                float v[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = okc ? cr[w][kn][j] : 0.0f;
                Chi[w][kn] = cvt8(v);
            }
        }
        __syncthreads();

        const bool more = c0 + L < end;
        const int cl_next = more ? (int)((end - c0 - L) < L ? (end - c0 - L) : L) : 0;
        // With chunks of 128 (eight waves) the next chunk's loads go out after this chunk's outputs:
        // issued before them, the outputs' own x loads (and the stores) queued behind the whole
        // prefetch, and the state loop below waited for all of it (1.32 -> 1.14 ms at 4 x 8192
        // together with the unrolled state loop). With chunks of 64 the registers do not allow it.
        constexpr bool kLatePrefetch = NW == 8;
        if (!kLatePrefetch && more) prefetch(c0 + L, cl_next);

        // ---------------- outputs of this wave's t-tiles
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const int tt = ttile_of<TL, NW>(wave, w);
            if (tt >= TL) break;
            const int t = 16 * tt + col;
            const bool valid = t < cl;
            float xe[TP][4];
            const int64_t tcl = c0 + min(t, cl - 1);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) load_k<XT, 4>(xbc + tcl * cdim + offX + 16 * pt + 4 * q, xe[pt]);
            const float l2t = l2p[t];
            f32x4 acc[TP];
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) acc[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kn = 0; kn < KN; ++kn)
#pragma unroll
                for (int pt = 0; pt < TP; ++pt)
                    acc[pt] = mma(*reinterpret_cast<const bf16x8 *>(&sHh[(16 * pt + col) * NSb + kn * 32 + q * 8]),
                                  Chi[w][kn], acc[pt]);
            const float el = __builtin_amdgcn_exp2f(l2t);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) acc[pt] *= el;
#pragma unroll 1
            for (int m = 0; m < KL; ++m) {
                if (2 * m > tt) break;
                f32x4 cb[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int si = 2 * m + h2;
                    cb[h2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    if (si <= tt) {
#pragma unroll
                        for (int kn = 0; kn < KN; ++kn)
                            cb[h2] = mma(*reinterpret_cast<const bf16x8 *>(&sBh[(16 * si + col) * NSb + kn * 32 + q * 8]),
                                         Chi[w][kn], cb[h2]);
                        const f32x4 l2s = *reinterpret_cast<const f32x4 *>(&l2p[16 * si + 4 * q]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int s = 16 * si + 4 * q + r;
                            cb[h2][r] = (s <= t) ? cb[h2][r] * __builtin_amdgcn_exp2f(l2t - l2s[r]) : 0.0f;
                        }
                    }
                }
                bf16x8 mh;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    mh[r] = f32_to_bf16(cb[0][r]);
                    mh[4 + r] = f32_to_bf16(cb[1][r]);
                }
#pragma unroll
                for (int pt = 0; pt < TP; ++pt)
                    acc[pt] = mma(*reinterpret_cast<const bf16x8 *>(&sXD[(16 * pt + col) * XSb + 32 * m + q * 8]), mh,
                                  acc[pt]);
            }
            if (valid) {
                const int64_t tok = c0 + t;
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    float o[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float v = acc[pt][r] + Dh * xe[pt][r];
                        if (a.z) v *= silu_f((float)static_cast<const AT *>(a.z)[tok * HP + offX + 16 * pt + 4 * q + r]);
                        o[r] = v;
                    }
                    store_k<bf16, 4>(y + tok * HP + offX + 16 * pt + 4 * q, o);
                }
            }
        }

        if (kLatePrefetch && more) prefetch(c0 + L, cl_next);

        // ---------------- carried state: H <- exp(lam_end) H + sum_s (x dt w)^T B   (3-term split)
        {
            const float dec = __builtin_amdgcn_exp2f(l2p[L - 1]);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Hacc[pt][j] *= dec;
            auto state_step = [&](int m) __attribute__((always_inline)) {
                bf16x8 bh[NJ], bl[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int n = 16 * (wave + j * NW) + col;
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const int s = 32 * m + tok_of_slot(q, jj);
                        bh[j][jj] = sBh[s * NSb + n];
                        bl[j][jj] = sBl[s * NSb + n];
                    }
                }
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const int idx = (16 * pt + col) * XSb + 32 * m + q * 8;
                    const bf16x8 xh = *reinterpret_cast<const bf16x8 *>(&sXSh[idx]);
                    const bf16x8 xl = *reinterpret_cast<const bf16x8 *>(&sXSl[idx]);
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        Hacc[pt][j] = mma(xh, bh[j], Hacc[pt][j]);
                        Hacc[pt][j] = mma(xh, bl[j], Hacc[pt][j]);
                        Hacc[pt][j] = mma(xl, bh[j], Hacc[pt][j]);
                    }
                }
            };
            // unrolled with chunks of 128 (a loop made the compiler wait there for every load in
            // flight, the prefetch included); a loop with chunks of 64, whose registers are full
            if constexpr (kLatePrefetch) {
#pragma unroll
                for (int m = 0; m < KL; ++m) state_step(m);
            } else {
#pragma unroll 1
                for (int m = 0; m < KL; ++m) state_step(m);
            }
        }
        if (more && wave == 0) token_arrays(buf ^ 1, cl_next);
        __syncthreads();
        write_sH();
    }
    __syncthreads();

#pragma unroll
    for (int pt = 0; pt < TP; ++pt)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Io<ST>::put(pool_tile, (int64_t)(16 * pt + 4 * q + r) * N + 16 * (wave + j * NW) + col, Hacc[pt][j][r]);
}

template <int P, int N, int L, typename ST, typename XT, bool PRECISE>
static hipError_t launch_scan_t(const LayerShape &s, const ScanArgs &a, hipStream_t stream) {
    constexpr int NW = (L >= 128) ? 8 : 4;
    dim3 grid(s.H, a.nseq);
    if constexpr (!PRECISE && P == 64 && N == 128) {
        if (s.act_dt == DT_BF16)
            hipLaunchKernelGGL((chunk_scan_fast_kernel<L, NW, ST, XT, bf16>), grid, dim3(NW * 64), 0, stream, a, s.H,
                               s.G);
        else
            hipLaunchKernelGGL((chunk_scan_fast_kernel<L, NW, ST, XT, float>), grid, dim3(NW * 64), 0, stream, a, s.H,
                               s.G);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((chunk_scan_kernel<P, N, L, NW, ST, XT, PRECISE>), grid, dim3(NW * 64), 0, stream, a, s.H,
                       s.G, s.act_dt, s.out_dt);
    return hipGetLastError();
}

template <int P, int N, int L, typename ST, typename XT>
static hipError_t launch_scan_p(const LayerShape &s, const ScanArgs &a, hipStream_t stream) {
    return s.out_dt == DT_F32 ? launch_scan_t<P, N, L, ST, XT, true>(s, a, stream)
                              : launch_scan_t<P, N, L, ST, XT, false>(s, a, stream);
}

template <int P, int N, int L, typename ST>
static hipError_t launch_scan_x(const LayerShape &s, const ScanArgs &a, hipStream_t stream) {
    return s.xbc_dt == DT_BF16 ? launch_scan_p<P, N, L, ST, bf16>(s, a, stream)
                               : launch_scan_p<P, N, L, ST, float>(s, a, stream);
}

template <int P, int N, int L>
static hipError_t launch_scan_s(const LayerShape &s, const ScanArgs &a, hipStream_t stream) {
    return s.state_dt == DT_BF16 ? launch_scan_x<P, N, L, bf16>(s, a, stream)
                                 : launch_scan_x<P, N, L, float>(s, a, stream);
}

bool scan_supported(const LayerShape &s) {
    if (s.P == 16 && s.N == 16) return s.Q == 16 || s.Q == 32 || s.Q == 64;
    if (s.P == 64 && s.N == 128) return s.Q == 64 || s.Q == 128;
    return false;
}

hipError_t launch_chunk_scan(const LayerShape &s, const ScanArgs &a, hipStream_t stream) {
    if (a.nseq == 0) return hipSuccess;
    if (s.P == 16 && s.N == 16) {
        if (s.Q == 16) return launch_scan_s<16, 16, 16>(s, a, stream);
        if (s.Q == 32) return launch_scan_s<16, 16, 32>(s, a, stream);
        if (s.Q == 64) return launch_scan_s<16, 16, 64>(s, a, stream);
    }
    if (s.P == 64 && s.N == 128) {
        if (s.Q == 64) return launch_scan_s<64, 128, 64>(s, a, stream);
        if (s.Q == 128) return launch_scan_s<64, 128, 128>(s, a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace m2
