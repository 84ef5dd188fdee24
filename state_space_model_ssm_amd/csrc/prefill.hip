// Fused prefill for the Nemotron-H head shape (P = 64, N = 128, y in bf16):
// the causal conv1d + SiLU of x runs inside the chunked SSD scan, so the x
// channels go from raw input to y without a post-conv round trip through HBM.
//
// The record page ("Nemotron-H-8B-Base-8K", mixer tensors conv1d, A_log, D,
// dt_bias, norm) fixes the layer's pieces; the conv reading is the one the
// conv kernels use (last tap on the current token, left context from the
// slot's cached raw inputs or zeros). The SSD algebra is that of the chunked
// scan kernel (scan.hip); what differs here is where each operand comes from:
//
//   x  raw rows of xBC (bf16 or fp32). Each thread owns a strip of R = 4
//      tokens x 4 channels and loads the W-1 rows before it as well, so the
//      conv needs no exchange between threads; the rows before a sequence's
//      first token come from the conv slot (has_initial_state) or are zero.
//      The post-conv values are written to the operand planes (x*dt for the
//      output, x*dt*exp(lam_end - lam) as hi/lo for the state) and, rounded to
//      bf16, to a token-major plane that the epilogue reads for D*x.
//   B, C  the bf16 operand planes [B hi | B lo | C] that the conv pass wrote
//      for each token (the group's conv runs once, not once per head): the
//      scan copies them into LDS / registers with no conversion.
//
// Per (sequence, head) workgroup and L-token chunk the global reads are the
// x strip (with a (W-1)/R halo that hits in cache), 3 * L * N bf16 of B/C
// planes (shared by the group's heads in L2), dt and z; y is written once.
// The conv cache is rewritten by a separate pass after this kernel, because
// every workgroup of a sequence reads the old cache here.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma.hpp"

namespace m2 {

template <int L, int NW, int W, typename ST, typename AT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void prefill_scan_kernel(PrefillArgs a, int H, int G) {
    constexpr int P = 64, N = 128;
    constexpr int NT = NW * 64;
    constexpr int TP = P / 16, TN = N / 16, TL = L / 16;
    constexpr int KN = N / 32, KL = L / 32;
    constexpr int XSb = L + 8;  // bf16 row stride of the x planes [p][pos(s)]
    constexpr int NSb = N + 8;  // bf16 row stride of the B planes [s][n] and of H [p][n]
    constexpr int XRb = P + 4;  // bf16 row stride of the post-conv x plane [t][p]
    constexpr int NJ = TN / NW;
    constexpr int TW = (TL + NW - 1) / NW;
    constexpr int R = 4;                 // tokens per x strip
    constexpr int XG = P / 4;            // 4-channel groups of x
    constexpr int NR = R + W - 1;        // raw rows per strip (with the conv context)
    constexpr int BPR = 2 * (N / 8);     // 16-byte pieces of the B hi + lo planes per token
    constexpr int BI = L * BPR / NT;
    constexpr int LB = (L + 63) / 64;
    constexpr float LOG2E = 1.4426950408889634f;
    static_assert(L % 32 == 0 && TN % NW == 0 && TL % NW == 0, "fast path shape");
    static_assert((L / R) * XG == NT, "one x strip per thread");
    static_assert((L * BPR) % NT == 0, "B pieces divide evenly over threads");

    __shared__ __attribute__((aligned(16))) bf16 sXD[P * XSb];
    __shared__ __attribute__((aligned(16))) bf16 sXSh[P * XSb];
    __shared__ __attribute__((aligned(16))) bf16 sXSl[P * XSb];
    __shared__ __attribute__((aligned(16))) bf16 sX[L * XRb];
    __shared__ __attribute__((aligned(16))) bf16 sBh[L * NSb];
    __shared__ __attribute__((aligned(16))) bf16 sBl[L * NSb];
    __shared__ __attribute__((aligned(16))) bf16 sHh[P * NSb];
    __shared__ __attribute__((aligned(16))) float sL2[2][L];
    __shared__ __attribute__((aligned(16))) float sDt[2][L];
    __shared__ __attribute__((aligned(16))) float sW[2][L];
    __shared__ __attribute__((aligned(16))) float sCtx[W - 1][P];  // x conv context before the first token

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, q = lane >> 4;
    const int head = xcd_head(blockIdx.x, H), seq = blockIdx.y;
    const int64_t HP = (int64_t)H * P;
    const int64_t cdim = HP + 2LL * G * N;
    const int64_t GN = (int64_t)G * N;
    const int64_t bcs = 3 * GN;  // row stride of the B/C planes
    const int g = head / (H / G);
    const int64_t start = a.cu[seq], end = a.cu[seq + 1];
    const int slot = a.idx[seq];
    const int64_t offX = (int64_t)head * P;
    const int64_t offBh = (int64_t)g * N, offBl = GN + (int64_t)g * N, offC = 2 * GN + (int64_t)g * N;
    bf16 *y = static_cast<bf16 *>(a.y);

    if (slot < 0) {
        for (int64_t i = tid; i < (end - start) * P; i += NT) y[(start + i / P) * HP + offX + (i % P)] = f32_to_bf16(0.0f);
        return;
    }

    const float A = -expf(a.A_log[head]);
    const float dtb = a.dt_bias[head];
    const float Dh = a.D[head];
    const AT *xin = static_cast<const AT *>(a.xbc);
    const bf16 *bc = static_cast<const bf16 *>(a.bc);
    ST *pool_tile = static_cast<ST *>(a.pool) + ((int64_t)slot * H + head) * (int64_t)P * N;
    const bool init = a.has_init && a.has_init[seq];

    // this thread's x strip: channels [4*xg, 4*xg + 4), tokens [R*xs, R*xs + R) of each chunk
    const int xg = tid % XG, xs = tid / XG;
    float cw[4 * W], cb[4];
    load_k<float, 4 * W>(a.conv_w + (offX + 4 * xg) * W, cw);
#pragma unroll
    for (int j = 0; j < 4; ++j) cb[j] = a.conv_b ? a.conv_b[offX + 4 * xg + j] : 0.0f;
    for (int i = tid; i < (W - 1) * P; i += NT) {
        const int k = i / P, c = i % P;
        sCtx[k][c] = init ? (float)static_cast<const ST *>(a.conv_pool)[((int64_t)slot * (W - 1) + k) * cdim + offX + c]
                          : 0.0f;
    }

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

    // Prefetch of a chunk into registers, as raw bits (converted at staging, so
    // no load waits at issue). Every load is unconditional: rows are clamped to
    // [start, last valid row of the chunk] and out-of-range values are replaced
    // or zeroed when staged.
    Raw<AT, 4> xr[NR];
    u32x4 br[BI];
    u32x4 cr[TW][KN];
    float dtr[LB];
    // Addresses are a 64-bit chunk base plus 32-bit row offsets (rows of one
    // chunk span far less than 2^31 elements).
    const int xrow0 = R * xs - (W - 1);  // first raw row of the strip, relative to the chunk
    auto prefetch = [&](int64_t c0, int cl) {
        const AT *xc = xin + c0 * cdim + offX + 4 * xg;
        const bf16 *bcc = bc + c0 * bcs;
        const int lo = (int)(start - c0);
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            int r = xrow0 + i;
            r = r < lo ? lo : (r > cl - 1 ? cl - 1 : r);
            xr[i].load(xc + r * (int)cdim);
        }
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const int id = tid + i * NT, sr = min(id / BPR, cl - 1), pc = id % BPR;
            const int off = (pc < N / 8 ? (int)offBh : (int)offBl - N) + 8 * pc;
            br[i] = *reinterpret_cast<const u32x4 *>(bcc + sr * (int)bcs + off);
        }
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const int t = min(16 * ttile_of<TL, NW>(wave, w) + col, cl - 1);
#pragma unroll
            for (int kn = 0; kn < KN; ++kn)
                cr[w][kn] = *reinterpret_cast<const u32x4 *>(bcc + t * (int)bcs + (int)offC + kn * 32 + q * 8);
        }
        if (wave == 0) {
            const AT *dtc = static_cast<const AT *>(a.dt_raw) + c0 * H + head;
#pragma unroll
            for (int b = 0; b < LB; ++b) {
                const int t = min(b * 64 + lane, cl - 1);
                dtr[b] = (float)dtc[t * H];
            }
        }
    };
    // wave 0: lam (log2 units), dt and state weights of a chunk into buffer `buf`
    auto token_arrays = [&](int buf, int cl) {
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
        const float lam_end = __shfl(lamv[(L - 1) / 64], (L - 1) % 64, 64);
#pragma unroll
        for (int b = 0; b < LB; ++b) {
            const int t = b * 64 + lane;
            if (t < L) {
                sL2[buf][t] = lamv[b] * LOG2E;
                sDt[buf][t] = dtv[b];
                sW[buf][t] = dtv[b] * __builtin_amdgcn_exp2f((lam_end - lamv[b]) * LOG2E);
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

        // ---------------- stage x: conv + SiLU of the strip -> planes
        {
            float u[NR][4];
#pragma unroll
            for (int i = 0; i < NR; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) u[i][j] = xr[i][j];
            if (c0 == start && xs == 0) {  // rows before the sequence: its cached context
#pragma unroll
                for (int i = 0; i < W - 1; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) u[i][j] = sCtx[i][4 * xg + j];
            }
#pragma unroll
            for (int tp = 0; tp < R; tp += 2) {
                const int s0 = R * xs + tp;  // even
                float xv[2][4];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const bool ok = s0 + h2 < cl;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float v = cb[j];
#pragma unroll
                        for (int k = 0; k < W; ++k) v += cw[j * W + k] * u[tp + h2 + k][j];
                        xv[h2][j] = ok ? silu_fast(v) : 0.0f;
                    }
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    bf16x4 xb;
#pragma unroll
                    for (int j = 0; j < 4; ++j) xb[j] = f32_to_bf16(xv[h2][j]);
                    *reinterpret_cast<bf16x4 *>(&sX[(s0 + h2) * XRb + 4 * xg]) = xb;
                }
                const float d0 = dtp[s0], d1 = dtp[s0 + 1], w0 = wp[s0], w1 = wp[s0 + 1];
                const int pos = pos_of(s0);  // s0 even: s0 + 1 sits at pos + 1
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int idx = (4 * xg + j) * XSb + pos;
                    const float s0v = xv[0][j] * w0, s1v = xv[1][j] * w1;
                    const bf16 h0 = f32_to_bf16(s0v), h1 = f32_to_bf16(s1v);
                    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                    *reinterpret_cast<bf16x2 *>(&sXD[idx]) =
                        bf16x2{f32_to_bf16(xv[0][j] * d0), f32_to_bf16(xv[1][j] * d1)};
                    *reinterpret_cast<bf16x2 *>(&sXSh[idx]) = bf16x2{h0, h1};
                    *reinterpret_cast<bf16x2 *>(&sXSl[idx]) =
                        bf16x2{f32_to_bf16(s0v - (float)h0), f32_to_bf16(s1v - (float)h1)};
                }
            }
        }
        // ---------------- stage B (copies of the hi / lo planes) and C
#pragma unroll
        for (int i = 0; i < BI; ++i) {
            const int id = tid + i * NT, s = id / BPR, pc = id % BPR;
            const u32x4 v = s < cl ? br[i] : u32x4{0u, 0u, 0u, 0u};
            bf16 *dst = pc < N / 8 ? &sBh[s * NSb + 8 * pc] : &sBl[s * NSb + 8 * (pc - N / 8)];
            *reinterpret_cast<u32x4 *>(dst) = v;
        }
        bf16x8 Chi[TW][KN];
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const bool okc = 16 * ttile_of<TL, NW>(wave, w) + col < cl;
#pragma unroll
            for (int kn = 0; kn < KN; ++kn) {
                const u32x4 v = okc ? cr[w][kn] : u32x4{0u, 0u, 0u, 0u};
                Chi[w][kn] = *reinterpret_cast<const bf16x8 *>(&v);
            }
        }
        __syncthreads();

        const bool more = c0 + L < end;
        const int cl_next = more ? (int)((end - c0 - L) < L ? (end - c0 - L) : L) : 0;
        if (more) prefetch(c0 + L, cl_next);

        // ---------------- outputs of this wave's t-tiles
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const int tt = ttile_of<TL, NW>(wave, w);
            if (tt >= TL) break;
            const int t = 16 * tt + col;
            const bool valid = t < cl;
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
                f32x4 cbt[2];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int si = 2 * m + h2;
                    cbt[h2] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                    if (si <= tt) {
#pragma unroll
                        for (int kn = 0; kn < KN; ++kn)
                            cbt[h2] = mma(*reinterpret_cast<const bf16x8 *>(&sBh[(16 * si + col) * NSb + kn * 32 + q * 8]),
                                          Chi[w][kn], cbt[h2]);
                        const f32x4 l2s = *reinterpret_cast<const f32x4 *>(&l2p[16 * si + 4 * q]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int s = 16 * si + 4 * q + r;
                            cbt[h2][r] = (s <= t) ? cbt[h2][r] * __builtin_amdgcn_exp2f(l2t - l2s[r]) : 0.0f;
                        }
                    }
                }
                bf16x8 mh;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    mh[r] = f32_to_bf16(cbt[0][r]);
                    mh[4 + r] = f32_to_bf16(cbt[1][r]);
                }
#pragma unroll
                for (int pt = 0; pt < TP; ++pt)
                    acc[pt] = mma(*reinterpret_cast<const bf16x8 *>(&sXD[(16 * pt + col) * XSb + 32 * m + q * 8]), mh,
                                  acc[pt]);
            }
            // Epilogue: y = acc + D x (times SiLU(z)). The tile goes through this
            // wave's own rows of sX (the rows it just read x from), so the global
            // store writes whole 128-byte rows (2 x 8 rows of 64 bf16) instead of
            // 32 bytes into each of 16 rows per instruction.
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const int64_t tokc = c0 + (valid ? t : cl - 1);
            bf16 *yc = y + c0 * HP + offX;
#pragma unroll
            for (int pt = 0; pt < TP; ++pt) {
                bf16x4 *px = reinterpret_cast<bf16x4 *>(&sX[t * XRb + 16 * pt + 4 * q]);
                const bf16x4 xb = *px;
                float o[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = acc[pt][r] + Dh * (float)xb[r];
                if (a.z) {
                    float zf[4];
                    load_k<AT, 4>(static_cast<const AT *>(a.z) + tokc * HP + offX + 16 * pt + 4 * q, zf);
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] *= silu_fast(zf[r]);
                }
                bf16x4 ob;
#pragma unroll
                for (int r = 0; r < 4; ++r) ob[r] = f32_to_bf16(o[r]);
                *px = ob;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int tr = 16 * tt + 8 * it + (lane >> 3), seg = lane & 7;
                if (tr < cl) {
                    const uint2 lo = *reinterpret_cast<const uint2 *>(&sX[tr * XRb + seg * 8]);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(&sX[tr * XRb + seg * 8 + 4]);
                    *reinterpret_cast<uint4 *>(yc + tr * (int)HP + seg * 8) = uint4{lo.x, lo.y, hi.x, hi.y};
                }
            }
        }

        // ---------------- carried state: H <- exp(lam_end) H + sum_s (x dt w)^T B   (3-term split)
        {
            const float dec = __builtin_amdgcn_exp2f(l2p[L - 1]);
#pragma unroll
            for (int pt = 0; pt < TP; ++pt)
#pragma unroll
                for (int j = 0; j < NJ; ++j) Hacc[pt][j] *= dec;
#pragma unroll 1
            for (int m = 0; m < KL; ++m) {
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

template <int L, int W, typename ST, typename AT>
static hipError_t launch_ps(const LayerShape &s, const PrefillArgs &a, hipStream_t stream) {
    constexpr int NW = (L >= 128) ? 8 : 4;
    dim3 grid(s.H, a.nseq);
    hipLaunchKernelGGL((prefill_scan_kernel<L, NW, W, ST, AT>), grid, dim3(NW * 64), 0, stream, a, s.H, s.G);
    return hipGetLastError();
}

template <int L, typename ST, typename AT>
static hipError_t launch_ps_w(const LayerShape &s, const PrefillArgs &a, hipStream_t stream) {
    switch (s.W) {
        case 2: return launch_ps<L, 2, ST, AT>(s, a, stream);
        case 3: return launch_ps<L, 3, ST, AT>(s, a, stream);
        case 4: return launch_ps<L, 4, ST, AT>(s, a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int L, typename ST>
static hipError_t launch_ps_a(const LayerShape &s, const PrefillArgs &a, hipStream_t stream) {
    return s.act_dt == DT_BF16 ? launch_ps_w<L, ST, bf16>(s, a, stream) : launch_ps_w<L, ST, float>(s, a, stream);
}

template <int L>
static hipError_t launch_ps_s(const LayerShape &s, const PrefillArgs &a, hipStream_t stream) {
    return s.state_dt == DT_BF16 ? launch_ps_a<L, bf16>(s, a, stream) : launch_ps_a<L, float>(s, a, stream);
}

bool prefill_fused_supported(const LayerShape &s) {
    return s.P == 64 && s.N == 128 && (s.Q == 64 || s.Q == 128) && s.W >= 2 && s.W <= 4 && s.out_dt == DT_BF16 &&
           s.H % s.G == 0;
}

hipError_t launch_prefill_scan(const LayerShape &s, const PrefillArgs &a, hipStream_t stream) {
    if (a.nseq == 0) return hipSuccess;
    if (s.Q == 64) return launch_ps_s<64>(s, a, stream);
    if (s.Q == 128) return launch_ps_s<128>(s, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace m2
