// device_common.h -- types and small device helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geometry.h"

namespace hstu {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Relative-bias bucket of a distance (exact integer rule: identity below 16, then four buckets
// per octave, last bucket 127).  Any distance >= 2^32 lands in bucket 127, so callers may
// saturate 64-bit distances to 0xffffffff.
HSTU_HD int bucket_of(uint32_t x) {
    if (x < 16u) return (int)x;
#if defined(__HIP_DEVICE_COMPILE__)
    int e = 31 - (int)__clz(x);
#else
    int e = 31 - __builtin_clz(x);
#endif
    int b = 16 + 4 * (e - 4) + (int)((x >> (e - 2)) & 3u);
    return b < kNumBuckets - 1 ? b : kNumBuckets - 1;
}

// "Bucket class" of a distance: 8 * clz(x) + the three bits after the leading one.  Every class
// lies inside one bucket, so a 264-entry table indexed by class replaces the bucket arithmetic in
// the inner loops.  clz(0) = 32 gives class 256.
constexpr int kNumClasses = 264;

__device__ __forceinline__ uint32_t bucket_class(uint32_t x) {
    uint32_t c = __clz(x);
    uint32_t y = x << (c & 31u);
    return c * 8u + ((y >> 28) & 7u);
}

// A representative distance of a class (any member gives the same bucket).
HSTU_HD uint32_t class_representative(int cls) {
    int c = cls >> 3, m = cls & 7;
    if (c <= 28) return (uint32_t)(8 + m) << (28 - c);
    if (c == 29) return 4u + (uint32_t)(m >> 1);
    if (c == 30) return 2u + (uint32_t)(m >> 2);
    if (c == 31) return 1u;
    return 0u;
}

HSTU_HD int bucket_of_class(int cls) { return bucket_of(class_representative(cls)); }

__device__ __forceinline__ uint32_t absdiff_u32(uint32_t a, uint32_t b) {
    return a > b ? a - b : b - a;
}

// |a - b| for 64-bit timestamps, saturated to 32 bits (exact for bucketing, see bucket_of).
__device__ __forceinline__ uint32_t absdiff_sat(int64_t a, int64_t b) {
    uint64_t d = a >= b ? (uint64_t)(a - b) : (uint64_t)(b - a);
    return d > 0xffffffffull ? 0xffffffffu : (uint32_t)d;
}

// Timestamps relative to a sequence base, biased into uint32 so that |a - b| is exact on 32-bit
// unsigned values when both relatives fit in int32.
__device__ __forceinline__ bool rel_time_fits(int64_t t, int64_t base) {
    int64_t r = t - base;
    return r >= -(int64_t)0x80000000ll && r <= (int64_t)0x7fffffffll;
}
__device__ __forceinline__ uint32_t rel_time_u32(int64_t t, int64_t base) {
    return (uint32_t)(t - base) + 0x80000000u;
}

// SiLU pieces with hardware exp2 / reciprocal (about 1 ulp each).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float fast_sigmoid(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * x));
}

// Scores are carried as t = -log2(e) * S, so sigmoid(S) = 1 / (1 + 2^t) and
// SiLU(S) = -ln(2) * t * sigmoid(S): the caller folds -ln(2) into one final scale.
__device__ __forceinline__ float silu_scaled(float t) {
    return t * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// Bucket range of the distances |x| for x in [lo, hi] when one bucket covers them all, else -1.
HSTU_HD int uniform_bucket(int64_t lo, int64_t hi) {
    if (lo < 0 && hi > 0) return -1;
    uint64_t a = (uint64_t)(lo < 0 ? -hi : lo), b = (uint64_t)(lo < 0 ? -lo : hi);
    uint32_t sa = a > 0xffffffffull ? 0xffffffffu : (uint32_t)a;
    uint32_t sb = b > 0xffffffffull ? 0xffffffffu : (uint32_t)b;
    int ba = bucket_of(sa);
    return ba == bucket_of(sb) ? ba : -1;
}

// Smallest distance whose bucket is b.
HSTU_HD uint32_t bucket_start(int b) {
    if (b < 16) return (uint32_t)b;
    const int e = 4 + (b - 16) / 4, m = (b - 16) % 4;
    return (1u << e) + (uint32_t)m * (1u << (e - 2));
}

// How one bias term behaves over a (wavefront, tile), decided from the range [lo, hi] of the
// signed distances it covers:
//   kind 0: one bucket (b_lo) for every pair;
//   kind 1: two adjacent buckets b_lo < b_hi, split at |x| >= thr;
//   kind 3: three adjacent buckets b_lo, b_lo + 1, b_hi = b_lo + 2, split at thr and thr2;
//   kind 2: anything else (per-element bucket lookup).
struct BiasSpan {
    int kind, b_lo, b_hi;
    uint32_t thr, thr2;
};
HSTU_HD BiasSpan bias_span(int64_t lo, int64_t hi) {
    BiasSpan r{2, 0, 0, 0, 0xffffffffu};
    if (lo < 0 && hi > 0) return r;
    uint64_t a = (uint64_t)(lo < 0 ? -hi : lo), b = (uint64_t)(lo < 0 ? -lo : hi);
    const uint32_t sa = a > 0xffffffffull ? 0xffffffffu : (uint32_t)a;
    const uint32_t sb = b > 0xffffffffull ? 0xffffffffu : (uint32_t)b;
    r.b_lo = bucket_of(sa);
    r.b_hi = bucket_of(sb);
    if (r.b_lo == r.b_hi) r.kind = 0;
    else if (r.b_hi == r.b_lo + 1) { r.kind = 1; r.thr = bucket_start(r.b_hi); }
    else if (r.b_hi == r.b_lo + 2) {
        r.kind = 3;
        r.thr = bucket_start(r.b_lo + 1);
        r.thr2 = bucket_start(r.b_hi);
    }
    return r;
}

// Scalar part of a tile's bias plus the time-bias selection of modes 1 and 4 (see BiasSpan);
// set() returns the time mode: 0 one bucket, 1 two buckets, 4 three buckets, 2 / 3 per-element
// class lookup with 32-bit / 64-bit times.
struct TimeSel {
    float b0, b1, b2;
    uint32_t thr, thr2;
    __device__ __forceinline__ void set_const(float b) {
        b0 = b1 = b2 = b;
        thr = thr2 = 0xffffffffu;
    }
    __device__ __forceinline__ int set(const BiasSpan& st, bool fit, float bpos, const float* wtb) {
        if (st.kind == 0) { set_const(bpos + wtb[st.b_lo]); return 0; }
        set_const(bpos);
        if (!fit) return 3;
        if (st.kind == 2) return 2;
        b0 = bpos + wtb[st.b_lo];
        b1 = bpos + wtb[st.b_lo + 1];
        b2 = bpos + wtb[st.b_hi];
        thr = st.thr;
        thr2 = st.thr2;
        return st.kind == 1 ? 1 : 4;
    }
};

// The per-element selector of a TimeSel, built once per tile.  The third bucket is reached by
// adding e2 = b2 - b1 (within one rounding of b2): a nested select among three values is turned
// by the compiler into an indexed load from a scratch copy of them.
struct TimePick {
    float b0, b1, e2;
    uint32_t thr, thr2;
    __device__ __forceinline__ explicit TimePick(const TimeSel& t)
        : b0(t.b0), b1(t.b1), e2(t.b2 - t.b1), thr(t.thr), thr2(t.thr2) {}
    template <int TM>
    __device__ __forceinline__ float get(uint32_t ti, uint32_t tj) const {
        if (TM == 1) return absdiff_u32(ti, tj) >= thr ? b1 : b0;
        if (TM == 4) {
            const uint32_t d = absdiff_u32(ti, tj);
            const float lo = d >= thr ? b1 : b0;
            return lo + (d >= thr2 ? e2 : 0.0f);
        }
        return b0;
    }
};

// Cross-lane reductions with DPP inside each row of 16 lanes (quad swaps, then half-row and row
// mirrors: afterwards every lane of a row holds the row's result), then the four rows combined
// from lanes 0, 16, 32, 48 with readlane.  Every lane of the wavefront must be active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = umin(v, dpp_u32<kDppXor1>(v));
    v = umin(v, dpp_u32<kDppXor2>(v));
    v = umin(v, dpp_u32<kDppHalfMirror>(v));
    v = umin(v, dpp_u32<kDppMirror>(v));
    return umin(umin(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                umin(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = umax(v, dpp_u32<kDppXor1>(v));
    v = umax(v, dpp_u32<kDppXor2>(v));
    v = umax(v, dpp_u32<kDppHalfMirror>(v));
    v = umax(v, dpp_u32<kDppMirror>(v));
    return umax(umax(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                umax(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ float fdpp_add(float v, uint32_t moved) {
    return v + __builtin_bit_cast(float, moved);
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
    v = fdpp_add(v, dpp_u32<kDppXor1>(__builtin_bit_cast(uint32_t, v)));
    v = fdpp_add(v, dpp_u32<kDppXor2>(__builtin_bit_cast(uint32_t, v)));
    v = fdpp_add(v, dpp_u32<kDppHalfMirror>(__builtin_bit_cast(uint32_t, v)));
    v = fdpp_add(v, dpp_u32<kDppMirror>(__builtin_bit_cast(uint32_t, v)));
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(u, 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ int64_t wave_min64(int64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        int64_t o = __shfl_xor(v, m);
        v = o < v ? o : v;
    }
    return v;
}
__device__ __forceinline__ int64_t wave_max64(int64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        int64_t o = __shfl_xor(v, m);
        v = o > v ? o : v;
    }
    return v;
}

// Time range and 32-bit fit of one tile's timestamps, held one per lane by a whole wavefront
// (lanes with real = false are ignored for the range).  When every relative time fits in 32 bits
// the range is reduced on the biased 32-bit values with DPP, else on the 64-bit values.
struct TimeRange {
    int64_t lo, hi;
    bool fit;
};
__device__ __forceinline__ TimeRange wave_time_range(int64_t t, bool real, int64_t base) {
    TimeRange r;
    r.fit = __all(rel_time_fits(t, base));
    if (r.fit) {
        const uint32_t u = rel_time_u32(t, base);
        const uint32_t lo = wave_min_u32(real ? u : 0xffffffffu);
        const uint32_t hi = wave_max_u32(real ? u : 0u);
        r.lo = base + (int64_t)(int32_t)(lo - 0x80000000u);
        r.hi = base + (int64_t)(int32_t)(hi - 0x80000000u);
    } else {
        r.lo = wave_min64(real ? t : INT64_MAX);
        r.hi = wave_max64(real ? t : INT64_MIN);
    }
    return r;
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = (bf16)v[t];
    return r;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of key k (0..63) inside a transposed tile row: bits 2 and 3 of k are swapped so that a
// lane's eight P^T operands (keys 16s + 8(t/4) + 4g + t%4) are contiguous (16s + 8g + t).
__device__ __forceinline__ int perm_key(int k) {
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

// Scheduling hint for a block of N MFMAs, each fed by one LDS read: issue LA reads first, then
// alternate one MFMA and one read, so each read has LA matrix instructions to land.
template <int N, int LA>
__device__ __forceinline__ void sched_mfma_lds() {
    __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < N - LA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

}  // namespace hstu
