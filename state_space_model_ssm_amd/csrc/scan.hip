// Chunked SSD scan for prefill on gfx950 (MFMA), varlen over cu_seqlens.
//
// The "Nemotron-H-8B-Base-8K" record (section "REQUIRED KERNEL CLASS") asks
// for a chunked scan kernel for the SSM layers; the recurrence itself is a
// multiplicative chain, so only the chunk-local pieces are dense
// contractions. Per chunk of L tokens of one (sequence, head), with
// lam_t = sum_{r <= t in chunk} dt_r * A (inclusive), xh_s = dt_s * x_s:
//
//   CB^T[s][t] = sum_n B_s[n] C_t[n]                       (MFMA)
//   Md^T[s][t] = CB^T[s][t] * exp(lam_t - lam_s), s <= t   (registers)
//   Yd^T[p][t] = sum_s xh^T[p][s] Md^T[s][t]               (MFMA, intra-chunk)
//   Yo^T[p][t] = exp(lam_t) sum_n H[p][n] C_t[n]           (MFMA, carried state)
//   y_t[p]     = Yd + Yo + D x_t[p]   (x SiLU(z) when z is given)
//   H         <- exp(lam_end) H + sum_s xh^T[p][s] B_s[n] exp(lam_end - lam_s)   (MFMA)
//
// which equals the token-by-token recurrence exactly in exact arithmetic
// (unrolling h_t = a_t h_{t-1} + dt_t x_t B_t^T over the chunk).
//
// Design (one workgroup of 4 wavefronts per (sequence, head), looping over the
// sequence's chunks in order):
//   * The carried state H [P][N] fp32 lives in MFMA accumulator registers for
//     the whole sequence (the inter-chunk pass is the loop itself), so chunk
//     states never touch HBM; the only traffic is x/B/C/dt in, y out, and the
//     initial/final state.
//   * C.B^T is computed transposed: its 16x16 accumulator tiles, two stacked,
//     are exactly the B operand of the next v_mfma_f32_16x16x32_bf16 in a
//     permuted k order, so the decay-masked matrix never goes through LDS.
//     xh^T is staged in LDS in that same permuted token order.
//   * Precision: MFMA operands are bf16. The chunk-state contraction (the only
//     path into the carried state) always uses a 3-term hi/lo split
//     (hi*hi + hi*lo + lo*hi), which keeps fp32-level accuracy; the output
//     contractions use the split only when y is stored in fp32 (PRECISE),
//     single bf16 operands otherwise.
//   * Ragged tails are zero padded (dt = 0 keeps lam flat, x = B = C = 0 adds
//     nothing); only valid rows are stored.
#include "common.hpp"
#include "kernels.hpp"

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
__device__ __forceinline__ int tok_of_slot(int q, int j) { return j < 4 ? 4 * q + j : 16 + 4 * q + (j - 4); }

template <int P, int N, int L, typename ST, typename XT, bool PRECISE>
__global__ __launch_bounds__(256) void chunk_scan_kernel(ScanArgs a, int H, int G, int act_dt, int out_dt) {
    constexpr int NW = 4;
    constexpr int TP = P / 16, TN = N / 16, TL = L / 16;
    constexpr int KN = (N + 31) / 32, KL = (L + 31) / 32;
    constexpr int LP = KL * 32, NP = KN * 32;
    constexpr int XS = LP + 4;  // sXT row stride (floats)
    constexpr int BS = NP + 4;  // sB row stride (floats)
    constexpr int HS = NP + 8;  // sH row stride (bf16)
    constexpr int NJ = (TN + NW - 1) / NW;  // n-tiles of H per wave
    constexpr int TW = (TL + NW - 1) / NW;  // t-tiles of y per wave
    static_assert(P % 16 == 0 && N % 16 == 0 && L % 16 == 0, "tile multiples");

    __shared__ __attribute__((aligned(16))) float sXT[P * XS];
    __shared__ __attribute__((aligned(16))) float sB[LP * BS];
    __shared__ __attribute__((aligned(16))) bf16 sHhi[P * HS];
    __shared__ __attribute__((aligned(16))) bf16 sHlo[PRECISE ? P * HS : 8];
    __shared__ float sLam[LP];
    __shared__ float sWt[LP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int head = blockIdx.x, seq = blockIdx.y;
    const int64_t HP = (int64_t)H * P;
    const int64_t cdim = HP + 2LL * G * N;
    const int g = head / (H / G);
    const int64_t start = a.cu[seq], end = a.cu[seq + 1];
    const int slot = a.idx[seq];
    const int64_t offX = (int64_t)head * P;
    const int64_t offB = HP + (int64_t)g * N;
    const int64_t offC = HP + (int64_t)G * N + (int64_t)g * N;

    if (slot < 0) {  // padding sequence: y rows are zero, no state access
        for (int64_t i = tid; i < (end - start) * P; i += 256)
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

    // Zero padding columns once (n in [N, NP) of sB and sH); they are never rewritten.
    if constexpr (NP > N) {
        for (int i = tid; i < LP * (NP - N); i += 256) sB[(i / (NP - N)) * BS + N + i % (NP - N)] = 0.0f;
        for (int i = tid; i < P * (NP - N); i += 256) {
            sHhi[(i / (NP - N)) * HS + N + i % (NP - N)] = f32_to_bf16(0.0f);
            if constexpr (PRECISE) sHlo[(i / (NP - N)) * HS + N + i % (NP - N)] = f32_to_bf16(0.0f);
        }
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

    for (int64_t c0 = start; c0 < end; c0 += L) {
        const int cl = (int)((end - c0) < L ? (end - c0) : L);

        // ---------------- load stage
        // xh^T[p][perm(s)] = dt_s * x_s[p]
        constexpr int XG = P / 4;
        for (int id = tid; id < LP * XG; id += 256) {
            const int s = id / XG, pg = id - (id / XG) * XG;
            float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (s < cl) {
                const float dts = softplus_f(ld(a.dt_raw, act_dt, (c0 + s) * H + head) + dtb);
                load_k<XT, 4>(xbc + (c0 + s) * cdim + offX + 4 * pg, v);
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] *= dts;
            }
            const int pos = (s & ~31) + perm32(s & 31);
#pragma unroll
            for (int i = 0; i < 4; ++i) sXT[(4 * pg + i) * XS + pos] = v[i];
        }
        // B natural [s][n]
        constexpr int BG = N / 4;
        for (int id = tid; id < LP * BG; id += 256) {
            const int s = id / BG, ng = id - (id / BG) * BG;
            float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (s < cl) load_k<XT, 4>(xbc + (c0 + s) * cdim + offB + 4 * ng, v);
            Io<float>::store(&sB[s * BS + 4 * ng], v);
        }
        // lam (inclusive cumsum of dt*A) and the chunk-state weights exp(lam_end - lam_s)
        if (wave == 0) {
            float carry = 0.0f;
            float lamv[KL * 32 / 64 + 1];
#pragma unroll
            for (int b = 0; b * 64 < LP; ++b) {
                const int t = b * 64 + lane;
                float v = 0.0f;
                if (t < cl) v = softplus_f(ld(a.dt_raw, act_dt, (c0 + t) * H + head) + dtb) * A;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_up(v, off, 64);
                    if (lane >= off) v += o;
                }
                v += carry;
                lamv[b] = v;
                carry = __shfl(v, 63, 64);
            }
            // lam_end = lam at the last valid token (flat over the zero padding)
            const float lam_end = __shfl(lamv[(LP - 1) / 64], (LP - 1) % 64, 64);
#pragma unroll
            for (int b = 0; b * 64 < LP; ++b) {
                const int t = b * 64 + lane;
                if (t < LP) {
                    sLam[t] = lamv[b];
                    sWt[t] = expf(lam_end - lamv[b]);
                }
            }
        }
        // C fragments (B operand, k = n) of this wave's t-tiles, straight from global
        bf16x8 Chi[TW][KN];
        bf16x8 Clo[PRECISE ? TW : 1][PRECISE ? KN : 1];
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const int tt = wave + w * NW;
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) {
                float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                const int t = 16 * tt + col, k0 = kn * 32 + q * 8;
                if (tt < TL && t < cl && k0 < N) load_k<XT, 8>(xbc + (c0 + t) * cdim + offC + k0, v);
                if constexpr (PRECISE) split8(v, Chi[w][kn], Clo[w][kn]);
                else Chi[w][kn] = cvt8(v);
            }
        }
        __syncthreads();

        // ---------------- outputs of this wave's t-tiles
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const int tt = wave + w * NW;
            if (tt >= TL) break;
            const int t = 16 * tt + col;
            const float lam_t = sLam[t];

            f32x4 cb[TL];
#pragma unroll
            for (int si = 0; si < TL; ++si) {
                cb[si] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                if (si <= tt) {
#pragma unroll
                    for (int kn = 0; kn < KN; ++kn) {
                        float v[8];
                        const float *src = &sB[(16 * si + col) * BS + kn * 32 + q * 8];
                        Io<float>::load(src, v);
                        Io<float>::load(src + 4, v + 4);
                        if constexpr (PRECISE) {
                            bf16x8 bh, bl;
                            split8(v, bh, bl);
                            cb[si] = mma(bh, Chi[w][kn], cb[si]);
                            cb[si] = mma(bh, Clo[w][kn], cb[si]);
                            cb[si] = mma(bl, Chi[w][kn], cb[si]);
                        } else {
                            cb[si] = mma(cvt8(v), Chi[w][kn], cb[si]);
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int s = 16 * si + 4 * q + r;
                        cb[si][r] = (s <= t) ? cb[si][r] * expf(lam_t - sLam[s]) : 0.0f;
                    }
                }
            }

            f32x4 yd[TP], yo[TP];
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                yd[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                yo[pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
            // intra-chunk: Yd^T[p][t] = sum_s xh^T[p][s] Md^T[s][t]
#pragma unroll
            for (int m = 0; m < KL; ++m) {
                if (2 * m > tt) break;
                float mv[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    mv[r] = cb[2 * m][r];
                    mv[4 + r] = (2 * m + 1 < TL && 2 * m + 1 <= tt) ? cb[(2 * m + 1 < TL) ? 2 * m + 1 : 0][r] : 0.0f;
                }
                bf16x8 mh, ml;
                if constexpr (PRECISE) split8(mv, mh, ml);
                else mh = cvt8(mv);
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    float xv[8];
                    const float *src = &sXT[(16 * pt + col) * XS + 32 * m + q * 8];
                    Io<float>::load(src, xv);
                    Io<float>::load(src + 4, xv + 4);
                    if constexpr (PRECISE) {
                        bf16x8 xh, xl;
                        split8(xv, xh, xl);
                        yd[pt] = mma(xh, mh, yd[pt]);
                        yd[pt] = mma(xh, ml, yd[pt]);
                        yd[pt] = mma(xl, mh, yd[pt]);
                    } else {
                        yd[pt] = mma(cvt8(xv), mh, yd[pt]);
                    }
                }
            }
            // carried state: Yo^T[p][t] = sum_n H[p][n] C_t[n]
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) {
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    const int idx = (16 * pt + col) * HS + kn * 32 + q * 8;
                    const bf16x8 hh = *reinterpret_cast<const bf16x8 *>(&sHhi[idx]);
                    yo[pt] = mma(hh, Chi[w][kn], yo[pt]);
                    if constexpr (PRECISE) {
                        const bf16x8 hl = *reinterpret_cast<const bf16x8 *>(&sHlo[idx]);
                        yo[pt] = mma(hh, Clo[w][kn], yo[pt]);
                        yo[pt] = mma(hl, Chi[w][kn], yo[pt]);
                    }
                }
            }
            // epilogue
            if (t < cl) {
                const float elam = expf(lam_t);
                const int64_t tok = c0 + t;
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    float o[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t p = 16 * pt + 4 * q + r;
                        const float xv = (float)xbc[tok * cdim + offX + p];
                        float v = yd[pt][r] + elam * yo[pt][r] + Dh * xv;
                        if (a.z) v *= silu_f(ld(a.z, act_dt, tok * HP + offX + p));
                        o[r] = v;
                    }
                    const int64_t yo_idx = tok * HP + offX + 16 * pt + 4 * q;
                    if (out_dt == DT_BF16) store_k<bf16, 4>(static_cast<bf16 *>(a.y) + yo_idx, o);
                    else store_k<float, 4>(static_cast<float *>(a.y) + yo_idx, o);
                }
            }
        }

        // ---------------- carried state: H <- exp(lam_end) H + sum_s xh^T B~
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
                        v[jj] = (n < NP) ? sB[s * BS + (n < NP ? n : 0)] * sWt[s] : 0.0f;
                    }
                    split8(v, bh[j], bl[j]);
                }
#pragma unroll
                for (int pt = 0; pt < TP; ++pt) {
                    float xv[8];
                    const float *src = &sXT[(16 * pt + col) * XS + 32 * m + q * 8];
                    Io<float>::load(src, xv);
                    Io<float>::load(src + 4, xv + 4);
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

template <int P, int N, int L, typename ST, typename XT, bool PRECISE>
static hipError_t launch_scan_t(const LayerShape &s, const ScanArgs &a, hipStream_t stream) {
    dim3 grid(s.H, a.nseq);
    hipLaunchKernelGGL((chunk_scan_kernel<P, N, L, ST, XT, PRECISE>), grid, dim3(256), 0, stream, a, s.H, s.G,
                       s.act_dt, s.out_dt);
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
    if (s.P == 16 && s.N == 16) return s.Q == 16 || s.Q == 32;
    if (s.P == 64 && s.N == 128) return s.Q == 64 || s.Q == 128;
    return false;
}

hipError_t launch_chunk_scan(const LayerShape &s, const ScanArgs &a, hipStream_t stream) {
    if (a.nseq == 0) return hipSuccess;
    if (s.P == 16 && s.N == 16) {
        if (s.Q == 16) return launch_scan_s<16, 16, 16>(s, a, stream);
        if (s.Q == 32) return launch_scan_s<16, 16, 32>(s, a, stream);
    }
    if (s.P == 64 && s.N == 128) {
        if (s.Q == 64) return launch_scan_s<64, 128, 64>(s, a, stream);
        if (s.Q == 128) return launch_scan_s<64, 128, 128>(s, a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace m2
