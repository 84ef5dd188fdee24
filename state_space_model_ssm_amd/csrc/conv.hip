// Prefill causal depthwise conv1d + SiLU over packed (cu_seqlens) sequences.
//
// The conv1d tensor is one of the Mamba-2 mixer tensors of the
// "Nemotron-H-8B-Base-8K" record. Reading where the pages are silent: the
// last tap multiplies the current token, the left context of a sequence is
// its slot's W-1 cached raw inputs (has_initial_state) or zeros, and the
// cache afterwards holds the last W-1 entries of [old cache || tokens].
//
// Memory bound elementwise work (2 reads of nothing but xBC, 1 write). Each
// thread owns 8 channels (one 16-byte bf16 vector) and TT consecutive tokens,
// so halo re-reads cost (W-1)/TT of the input stream. A thread finds its
// sequence by binary search in cu_seqlens. When its tokens lie in one
// sequence it loads all TT + W - 1 rows before computing (TT + W - 1 loads in
// flight per thread: 4.2 -> 5.3 TB/s at prefill-8b); a run that crosses into
// the next sequence carries a sliding window of the previous W-1 raw inputs
// and restarts it at the boundary. No host synchronisation, no per-sequence
// launch.
//
// The cache update runs as a second kernel after the conv (stream order),
// because the conv reads the old cache: doing both in one grid would race.
//
#include "common.hpp"
#include "kernels.hpp"

namespace m2 {

template <typename AT, typename ST, typename XT, int W, int TT>
__global__ __launch_bounds__(256) void conv_fwd_kernel(ConvFwdArgs a, int64_t cdim) {
    const int cv = threadIdx.x & 63;
    const int tg = threadIdx.x >> 6;
    const int64_t c0 = ((int64_t)blockIdx.x * 64 + cv) * 8;
    const int64_t t0 = ((int64_t)blockIdx.y * 4 + tg) * TT;
    if (c0 >= cdim || t0 >= a.T) return;
    const int64_t t1 = t0 + TT < a.T ? t0 + TT : a.T;
    const AT *in = static_cast<const AT *>(a.xbc) + c0;
    XT *out = static_cast<XT *>(a.out) + c0;

    float w[8 * W];
    load_k<float, 8 * W>(a.w + c0 * W, w);
    float bias[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bias[j] = a.b ? a.b[c0 + j] : 0.0f;

    int seq = find_seq(a.cu, a.nseq, t0);
    int64_t seq_start = a.cu[seq], seq_end = a.cu[seq + 1];
    // (conv_state_kernel, run for every sequence after this one, counts bad indices)
    int slot = pool_slot(a.idx[seq], a.num_slots, a.err, false);

    if (t1 <= seq_end) {
        // The run lies in one sequence (all but the runs that cross a boundary): every
        // row is loaded before any is used, so a thread has TT + W - 1 loads in flight
        // instead of one; rows before the sequence come from its cache or are zeros.
        constexpr int NR = TT + W - 1;
        Raw<AT, 8> r[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
            int64_t src = t0 - (W - 1) + i;
            src = src < seq_start ? seq_start : (src >= t1 ? t1 - 1 : src);
            r[i].load(in + src * cdim);
        }
        float ctx[W - 1][8];
        const bool head = t0 - (W - 1) < seq_start;
        if (head) {
            const bool init = slot >= 0 && a.has_init && a.has_init[seq];
            const ST *cache = static_cast<const ST *>(a.pool) + (int64_t)(slot < 0 ? 0 : slot) * (W - 1) * cdim + c0;
#pragma unroll
            for (int k = 0; k < W - 1; ++k) {
                const int64_t src = t0 - (W - 1) + k;
                if (src >= seq_start) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) ctx[k][j] = r[k][j];
                } else if (init) {
                    load_k<ST, 8>(cache + (int64_t)((W - 1) - (seq_start - src)) * cdim, ctx[k]);
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) ctx[k][j] = 0.0f;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < TT; ++i) {
            if (t0 + i >= t1) break;
            float o[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float v = bias[j];
#pragma unroll
                for (int k = 0; k < W; ++k) {
                    const int rr = i + k;  // window row: raw input at t0 + i - (W-1) + k
                    const float uv = (rr < W - 1 && head) ? ctx[rr][j] : r[rr][j];
                    v += w[j * W + k] * uv;
                }
                o[j] = slot < 0 ? 0.0f : silu_fast(v);
            }
            store_k<XT, 8>(out + (t0 + i) * cdim, o);
        }
        return;
    }

    float win[W - 1][8];  // win[k] = raw input at t - (W-1) + k

    auto fill_window = [&](int64_t t) {
        const bool init = slot >= 0 && a.has_init && a.has_init[seq];
        const ST *cache = static_cast<const ST *>(a.pool) + (int64_t)(slot < 0 ? 0 : slot) * (W - 1) * cdim + c0;
#pragma unroll
        for (int k = 0; k < W - 1; ++k) {
            const int64_t src = t - (W - 1) + k;
            if (src >= seq_start) {
                load_k<AT, 8>(in + src * cdim, win[k]);
            } else if (init) {
                load_k<ST, 8>(cache + (int64_t)((W - 1) - (seq_start - src)) * cdim, win[k]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) win[k][j] = 0.0f;
            }
        }
    };
    fill_window(t0);

    for (int64_t t = t0; t < t1; ++t) {
        if (t >= seq_end) {  // next non-empty sequence starts exactly at t
            while (seq + 1 < a.nseq && a.cu[seq + 1] <= t) ++seq;
            seq_start = a.cu[seq];
            seq_end = a.cu[seq + 1];
            slot = pool_slot(a.idx[seq], a.num_slots, a.err, false);
            fill_window(t);
        }
        float u[8], o[8];
        load_k<AT, 8>(in + t * cdim, u);
        if (slot < 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = 0.0f;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float v = bias[j];
#pragma unroll
                for (int k = 0; k < W - 1; ++k) v += w[j * W + k] * win[k][j];
                v += w[j * W + W - 1] * u[j];
                o[j] = silu_fast(v);
            }
        }
        store_k<XT, 8>(out + t * cdim, o);
#pragma unroll
        for (int k = 0; k < W - 2; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j) win[k][j] = win[k + 1][j];
#pragma unroll
        for (int j = 0; j < 8; ++j) win[W - 2][j] = u[j];
    }
}

// New cache of each sequence: entries [len, len + W-1) of [old cache || tokens].
template <typename AT, typename ST, int W>
__global__ __launch_bounds__(256) void conv_state_kernel(ConvFwdArgs a, int64_t cdim) {
    const int seq = blockIdx.y;
    const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
    if (c0 >= cdim) return;
    // Two round trips: the sequence's slot, bounds and flag together, then every row either
    // source may give (the cached rows and the sequence's last W - 1 tokens, clamped into the
    // packed rows), selected once they arrive. Loads behind the slot test and behind per-row
    // branches went out one round trip after another.
    const int idx = a.idx[seq];
    const int64_t start = a.cu[seq];
    const int64_t len = a.cu[seq + 1] - start;
    const bool init = a.has_init && a.has_init[seq];
    const int slot = pool_slot(idx, a.num_slots, a.err, c0 == 0);
    if (slot < 0) return;
    ST *cache = static_cast<ST *>(a.pool) + (int64_t)slot * (W - 1) * cdim + c0;
    const AT *in = static_cast<const AT *>(a.xbc) + c0;
    Raw<ST, 8> oldr[W - 1];
    Raw<AT, 8> tokr[W - 1];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) oldr[k].load(cache + k * cdim);
    if (a.T > 0) {
#pragma unroll
        for (int k = 0; k < W - 1; ++k) {
            int64_t row = start + len + k - (W - 1);  // the token for entry k when len + k >= W - 1
            row = row < 0 ? 0 : (row > a.T - 1 ? a.T - 1 : row);
            tokr[k].load(in + row * cdim);
        }
    } else {
#pragma unroll
        for (int k = 0; k < W - 1; ++k)
#pragma unroll
            for (int i = 0; i < Raw<AT, 8>::kW; ++i) tokr[k].w[i] = 0u;  // (never selected: no tokens)
    }
    float nw[W - 1][8];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int64_t pos = len + k;  // index into [old cache (W-1) || tokens (len)]
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float o = 0.0f;
#pragma unroll
            for (int kk = 0; kk < W - 1; ++kk) o = (pos == kk && init) ? oldr[kk][j] : o;
            nw[k][j] = pos < W - 1 ? o : tokr[k][j];
        }
    }
#pragma unroll
    for (int k = 0; k < W - 1; ++k) store_k<ST, 8>(cache + k * cdim, nw[k]);
}

// mode 0: conv of every channel, then the cache update; mode 2: the cache update alone.
template <typename AT, typename ST, typename XT, int W>
static hipError_t launch_cf(const LayerShape &s, const ConvFwdArgs &a, hipStream_t stream, int mode) {
    constexpr int TT = 16;
    const int64_t cdim = s.cdim();
    if (a.T > 0 && mode == 0) {
        dim3 grid((unsigned)((cdim / 8 + 63) / 64), (unsigned)((a.T + 4 * TT - 1) / (4 * TT)));
        hipLaunchKernelGGL((conv_fwd_kernel<AT, ST, XT, W, TT>), grid, dim3(256), 0, stream, a, cdim);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    dim3 g2((unsigned)((cdim / 8 + 255) / 256), a.nseq);
    hipLaunchKernelGGL((conv_state_kernel<AT, ST, W>), g2, dim3(256), 0, stream, a, cdim);
    return hipGetLastError();
}

template <typename AT, typename ST, typename XT>
static hipError_t launch_cf_w(const LayerShape &s, const ConvFwdArgs &a, hipStream_t stream, int mode) {
    switch (s.W) {
        case 2: return launch_cf<AT, ST, XT, 2>(s, a, stream, mode);
        case 3: return launch_cf<AT, ST, XT, 3>(s, a, stream, mode);
        case 4: return launch_cf<AT, ST, XT, 4>(s, a, stream, mode);
        default: return hipErrorInvalidValue;
    }
}

template <typename AT, typename ST>
static hipError_t launch_cf_x(const LayerShape &s, const ConvFwdArgs &a, hipStream_t stream, int mode) {
    return s.xbc_dt == DT_BF16 ? launch_cf_w<AT, ST, bf16>(s, a, stream, mode)
                               : launch_cf_w<AT, ST, float>(s, a, stream, mode);
}

template <typename AT>
static hipError_t launch_cf_s(const LayerShape &s, const ConvFwdArgs &a, hipStream_t stream, int mode) {
    return s.state_dt == DT_BF16 ? launch_cf_x<AT, bf16>(s, a, stream, mode)
                                 : launch_cf_x<AT, float>(s, a, stream, mode);
}

static hipError_t launch_cf_a(const LayerShape &s, const ConvFwdArgs &a, hipStream_t stream, int mode) {
    if (a.nseq == 0) return hipSuccess;
    return s.act_dt == DT_BF16 ? launch_cf_s<bf16>(s, a, stream, mode) : launch_cf_s<float>(s, a, stream, mode);
}

bool conv_supported(const LayerShape &s) { return s.W >= 2 && s.W <= 4 && s.cdim() % 8 == 0; }

hipError_t launch_conv_fwd(const LayerShape &s, const ConvFwdArgs &a, hipStream_t stream) {
    return launch_cf_a(s, a, stream, 0);
}

hipError_t launch_conv_state(const LayerShape &s, const ConvFwdArgs &a, hipStream_t stream) {
    return launch_cf_a(s, a, stream, 2);
}

}  // namespace m2
