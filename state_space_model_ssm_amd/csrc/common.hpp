// Shared device helpers for the gfx950 Mamba-2 kernels: storage types, bf16
// conversion, 16-byte vector access and the scalar activations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum Dt : int { DT_F32 = 0, DT_BF16 = 1 };

// Pool slot for an index read from the caller's table: the index itself when it lies in
// [0, num_slots) or is negative (padding), -1 when it is >= num_slots (the row or sequence is
// then skipped like padding and, by the one thread that `reports`, counted in *err).
__device__ __forceinline__ int pool_slot(int s, int num_slots, unsigned *err, bool reports) {
    if (s >= num_slots) {
        if (reports && err) atomicAdd(err, 1u);
        return -1;
    }
    return s;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float -> bf16, round to nearest even (the conversion clang defines for __bf16).
__device__ __forceinline__ bf16 f32_to_bf16(float v) { return (bf16)v; }

template <typename T> struct Io;

template <> struct Io<float> {
    static constexpr int kVec = 4;  // elements per 16-byte access
    __device__ static __forceinline__ void load(const float *p, float *out) {
        f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    }
    __device__ static __forceinline__ void store(float *p, const float *in) {
        f32x4 v = {in[0], in[1], in[2], in[3]};
        *reinterpret_cast<f32x4 *>(p) = v;
    }
    __device__ static __forceinline__ float get(const float *p, int64_t i) { return p[i]; }
    __device__ static __forceinline__ void put(float *p, int64_t i, float v) { p[i] = v; }
};

template <> struct Io<bf16> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ void load(const bf16 *p, float *out) {
        uint4 v = *reinterpret_cast<const uint4 *>(p);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static __forceinline__ void store(bf16 *p, const float *in) {
        bf16x8 v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = f32_to_bf16(in[i]);
        *reinterpret_cast<bf16x8 *>(p) = v;
    }
    __device__ static __forceinline__ float get(const bf16 *p, int64_t i) { return (float)p[i]; }
    __device__ static __forceinline__ void put(bf16 *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// K consecutive elements (K a multiple of 4) with the widest aligned vector access.
template <typename T, int K> __device__ __forceinline__ void load_k(const T *p, float *out) {
    static_assert(K % 4 == 0, "load_k: K must be a multiple of 4");
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < K / 4; ++i) Io<float>::load(reinterpret_cast<const float *>(p) + 4 * i, out + 4 * i);
    } else if constexpr (K % 8 == 0) {
#pragma unroll
        for (int i = 0; i < K / 8; ++i) Io<bf16>::load(p + 8 * i, out + 8 * i);
    } else {
#pragma unroll
        for (int i = 0; i < K / 4; ++i) {
            uint2 v = *reinterpret_cast<const uint2 *>(p + 4 * i);
            out[4 * i + 0] = __uint_as_float(v.x << 16);
            out[4 * i + 1] = __uint_as_float(v.x & 0xffff0000u);
            out[4 * i + 2] = __uint_as_float(v.y << 16);
            out[4 * i + 3] = __uint_as_float(v.y & 0xffff0000u);
        }
    }
}

template <typename T, int K> __device__ __forceinline__ void store_k(T *p, const float *in) {
    static_assert(K % 4 == 0, "store_k: K must be a multiple of 4");
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < K / 4; ++i) Io<float>::store(reinterpret_cast<float *>(p) + 4 * i, in + 4 * i);
    } else if constexpr (K % 8 == 0) {
#pragma unroll
        for (int i = 0; i < K / 8; ++i) Io<bf16>::store(p + 8 * i, in + 8 * i);
    } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int i = 0; i < K / 4; ++i) {
            bf16x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = f32_to_bf16(in[4 * i + j]);
            *reinterpret_cast<bf16x4 *>(p + 4 * i) = v;  // one 8-byte store
        }
    }
}

// K elements of T held as their raw bits after one vector load and widened to
// float only where used: converting right at the load would make the compiler
// wait for that load (and, loads completing in order, for every earlier one).
template <typename T, int K> struct Raw {
    static_assert((K * sizeof(T)) % 8 == 0, "Raw: 8-byte multiple");
    static constexpr int kW = (int)(K * sizeof(T) / 4);
    uint32_t w[kW];
    __device__ __forceinline__ void load(const T *p) {
        if constexpr (kW % 4 == 0) {
#pragma unroll
            for (int i = 0; i < kW / 4; ++i) {
                const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
                w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kW / 2; ++i) {
                const uint2 v = reinterpret_cast<const uint2 *>(p)[i];
                w[2 * i] = v.x; w[2 * i + 1] = v.y;
            }
        }
    }
    __device__ __forceinline__ float operator[](int i) const {
        if constexpr (sizeof(T) == 4) return __uint_as_float(w[i]);
        else return __uint_as_float((i & 1) ? (w[i >> 1] & 0xffff0000u) : (w[i >> 1] << 16));
    }
};

// 16-byte streaming (nontemporal) access: data touched once per launch should
// not displace reusable lines from L2 / the memory-side cache.
template <typename T> __device__ __forceinline__ void nt_load16(const T *p, float *out) {
    if constexpr (sizeof(T) == 4) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(v[i] << 16);
            out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
}
// The 16 bytes of nt_load16 as fp32 values, from raw bits loaded earlier.
template <typename T> __device__ __forceinline__ void unpack16(const u32x4 &v, float *out) {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(v[i] << 16);
            out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
}
template <typename T> __device__ __forceinline__ void nt_store16(T *p, const float *in) {
    if constexpr (sizeof(T) == 4) {
        const f32x4 v = {in[0], in[1], in[2], in[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
    } else {
        bf16x8 b;
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = f32_to_bf16(in[i]);
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(&b), reinterpret_cast<u32x4 *>(p));
    }
}

// Runtime-dtype scalar access for small per-row tensors (dt_raw, z, y, x).
__device__ __forceinline__ float ld(const void *p, int dt, int64_t i) {
    return dt == DT_BF16 ? (float)static_cast<const bf16 *>(p)[i] : static_cast<const float *>(p)[i];
}
__device__ __forceinline__ void st(void *p, int dt, int64_t i, float v) {
    if (dt == DT_BF16) static_cast<bf16 *>(p)[i] = f32_to_bf16(v);
    else static_cast<float *>(p)[i] = v;
}

// Sum over each aligned group of K lanes (K a power of two, 2..32), left in the
// group's last lane (the others hold partial sums): DPP shifts inside rows of
// 16 lanes (a window sum ending at each lane), then for K = 32 a broadcast of
// lane 15 into the next row. VALU only, no LDS round trips.
template <int CTRL, int ROWS> __device__ __forceinline__ float dpp_add_src(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, true));
}
template <int K> __device__ __forceinline__ float group_sum_last(float v) {
    static_assert(K >= 1 && K <= 32 && (K & (K - 1)) == 0, "group of 1..32 lanes");
    if constexpr (K >= 2) v += dpp_add_src<0x111, 0xF>(v);   // row_shr:1
    if constexpr (K >= 4) v += dpp_add_src<0x112, 0xF>(v);   // row_shr:2
    if constexpr (K >= 8) v += dpp_add_src<0x114, 0xF>(v);   // row_shr:4
    if constexpr (K >= 16) v += dpp_add_src<0x118, 0xF>(v);  // row_shr:8
    if constexpr (K >= 32) v += dpp_add_src<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    return v;
}

// Four sums over each row of 16 lanes, reduce-scattered: on return every lane of
// quad k of the row (lanes 4k .. 4k + 3) holds the row's total of v[k]. Lanes
// l and l ^ 8 first trade halves (rows {0, 1} stay with bit 3 clear, {2, 3}
// with it set), then lanes l and 7 - l of each half row (they differ in bit 2),
// then the quad sums its four partials: 11 VALU instructions for four totals,
// against 20 for four window sums and their final adds.
__device__ __forceinline__ float row16_sum4_scatter(const float v[4], bool bit3, bool bit2) {
    const float k0 = bit3 ? v[2] : v[0], s0 = bit3 ? v[0] : v[2];
    const float k1 = bit3 ? v[3] : v[1], s1 = bit3 ? v[1] : v[3];
    const float a0 = k0 + dpp_add_src<0x128, 0xF>(s0);  // row_ror:8 (the partner l ^ 8)
    const float a1 = k1 + dpp_add_src<0x128, 0xF>(s1);
    const float k = bit2 ? a1 : a0, s = bit2 ? a0 : a1;
    float t = k + dpp_add_src<0x141, 0xF>(s);           // row_half_mirror (the partner 7 - l)
    t += dpp_add_src<0xB1, 0xF>(t);                     // quad_perm [1, 0, 3, 2]
    t += dpp_add_src<0x4E, 0xF>(t);                     // quad_perm [2, 3, 0, 1]
    return t;
}

// Inclusive prefix sum over the 64 lanes with DPP: shifts within rows of 16,
// then row broadcasts of lane 15 and lane 31 (no LDS round trips).
__device__ __forceinline__ float wave_prefix_sum(float v) {
    v = group_sum_last<16>(v);              // window sums inside each row of 16
    v += dpp_add_src<0x142, 0xA>(v);        // row_bcast:15 into rows 1 and 3
    v += dpp_add_src<0x143, 0xC>(v);        // row_bcast:31 into rows 2 and 3
    return v;
}

// Sequence of packed token t: the largest i with cu[i] <= t (sequences may be empty).
__device__ __forceinline__ int find_seq(const int32_t *cu, int nseq, int64_t t) {
    int lo = 0, hi = nseq;  // answer in [0, nseq-1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Sequence taken by the workgroups in grid row r of a (…, nseq) grid whose workgroups
// each carry one sequence from start to end: with 2..kRankMax sequences, the r-th
// longest (ties by index), so long sequences are dispatched first and do not leave a
// tail of few busy CUs after the short ones finish; otherwise sequence r. The result
// does not depend on which workgroup takes which sequence. Every thread of the
// workgroup calls it (it synchronises the workgroup once when it reorders).
constexpr int kRankMax = 256;
__device__ __forceinline__ int seq_longest_first(const int32_t *cu, int nseq, int r, int tid, int nthreads,
                                                 int *shared_seq) {
    if (nseq <= 1 || nseq > kRankMax) return r;
    for (int i = tid; i < nseq; i += nthreads) {
        const int li = cu[i + 1] - cu[i];
        int rank = 0;
        for (int j = 0; j < nseq; ++j) {
            const int lj = cu[j + 1] - cu[j];
            rank += (lj > li) | ((lj == li) & (j < i));
        }
        if (rank == r) *shared_seq = i;  // ranks are a permutation: one writer
    }
    __syncthreads();
    return *shared_seq;
}

__device__ __forceinline__ float softplus_f(float v) { return fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v))); }
__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + expf(-v)); }
// softplus(v) = max(v, 0) + log1p(exp(-|v|)) from the hardware exp2/log2, with
// log1p(e) evaluated as log(1 + e) * e / ((1 + e) - 1), which cancels the
// rounding of 1 + e (the classic compensated form; e itself when 1 + e rounds to
// 1). A few fp32 ulp; for per-element use where the library softplus (a long
// polynomial with a float64 step) would dominate the instruction count.
__device__ __forceinline__ float softplus_fast(float v) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(v) * 1.4426950408889634f);
    const float u = 1.0f + e;
    const float l = (u == 1.0f) ? e : __builtin_amdgcn_logf(u) * 0.6931471805599453f * e * __builtin_amdgcn_rcpf(u - 1.0f);
    return fmaxf(v, 0.0f) + l;
}

// SiLU from the hardware exp2 and reciprocal (each about 1 ulp): a few
// instructions instead of the accurate exp and IEEE divide, for the per-element
// conv outputs of prefill. Relative error of a few fp32 ulp; the limits hold
// (large negative v: exp2 -> inf, rcp -> 0, result -> 0; large positive: v).
__device__ __forceinline__ float silu_fast(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v * -1.4426950408889634f));
}

}  // namespace m2
