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
// The same in one instruction (v_sad_u32 computes |a - b| + c); as inline assembly it constrains
// register allocation, so kernels at the register limit use absdiff_u32.
__device__ __forceinline__ uint32_t absdiff_sad(uint32_t a, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
    uint32_t r;
    asm("v_sad_u32 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
#else
    return a > b ? a - b : b - a;
#endif
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
// d SiLU(h) / dh = s (1 + h (1 - s)), s = sigmoid(h)
__device__ __forceinline__ float silu_deriv(float h) {
    const float sg = fast_sigmoid(h);
    return sg * (1.0f + h * (1.0f - sg));
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

// Wavefront-uniform values (read from LDS, hence in vector registers) moved to scalar registers,
// so that the per-tile decisions built on them run on the scalar unit.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A wavefront-uniform float kept in a scalar register.
__device__ __forceinline__ float uniform(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// Scalar part of a tile's bias plus the time-bias selection of modes 1 and 4 (see BiasSpan);
// set() returns the time mode: 0 one bucket, 1 two buckets, 4 three buckets, 2 / 3 per-element
// class lookup with 32-bit / 64-bit times.
//
// Modes 1 and 4 only arise when the time differences of the tile have one sign (bias_span
// gives per-element mode otherwise), so |t_lane - t_elem| >= thr is a one-sided comparison of
// the element's time with a per-lane limit: `later` = every lane's time >= every element's.
// lane_tmax (the largest lane time, 32-bit relative) guards the limit t_lane + thr against
// overflow in the other case (such tiles fall back to per-element mode).
struct TimeSel {
    float b0, b1, b2;
    uint32_t thr, thr2;
    bool later;
    __device__ __forceinline__ void set_const(float b) {
        b0 = b1 = b2 = b;
        thr = thr2 = 0xffffffffu;
        later = true;
    }
    __device__ __forceinline__ int set(const BiasSpan& st, bool fit, float bpos, const float* wtb,
                                       bool lane_later, uint32_t lane_tmax) {
        if (st.kind == 0) { set_const(bpos + wtb[st.b_lo]); return 0; }
        set_const(bpos);
        if (!fit) return 3;
        if (st.kind == 2) return 2;
        if (!lane_later &&
            (uint64_t)lane_tmax + (st.kind == 1 ? st.thr : st.thr2) > 0xffffffffull)
            return 2;
        b0 = uniform(bpos + wtb[st.b_lo]);
        b1 = uniform(bpos + wtb[st.b_lo + 1]);
        b2 = uniform(bpos + wtb[st.b_hi]);
        thr = st.thr;
        thr2 = st.thr2;
        later = lane_later;
        return st.kind == 1 ? 1 : 4;
    }
};

// The per-element selector of a TimeSel for one lane's time tl, built once per tile:
//   mode 1: bias = te < l1 ? x1 : y1;  mode 4: that plus (te < l2 ? x2 : y2).
// With later, |tl - te| >= thr <=> te <= tl - thr <=> te < tl - thr + 1 (0 when tl < thr);
// otherwise |tl - te| >= thr <=> te >= tl + thr, the same comparison with the values swapped.
// The third bucket is reached by adding e2 = b2 - b1 (within one rounding of b2): a nested
// select among three values is turned by the compiler into an indexed load from scratch.
struct TimePick {
    float b0, x1, y1, x2, y2;
    uint32_t l1, l2;
    __device__ __forceinline__ TimePick(const TimeSel& t, uint32_t tl) : b0(t.b0) {
        const float e2 = t.b2 - t.b1;
        if (t.later) {
            l1 = tl >= t.thr ? tl - t.thr + 1u : 0u;
            l2 = tl >= t.thr2 ? tl - t.thr2 + 1u : 0u;
        } else {
            l1 = tl + t.thr;   // no overflow in modes 1 and 4 (see TimeSel::set)
            l2 = tl + t.thr2;
        }
        x1 = uniform(t.later ? t.b1 : t.b0);
        y1 = uniform(t.later ? t.b0 : t.b1);
        x2 = uniform(t.later ? e2 : 0.0f);
        y2 = uniform(t.later ? 0.0f : e2);
    }
    template <int TM>
    __device__ __forceinline__ float get(uint32_t te) const {
        if (TM == 1) return te < l1 ? x1 : y1;
        if (TM == 4) return (te < l1 ? x1 : y1) + (te < l2 ? x2 : y2);
        return b0;
    }
};

// The same selection from |tl - te| itself (one more instruction per element, but no per-lane
// limits to keep: for kernels short of registers).
struct TimePickAbs {
    float b0, b1, e2;
    uint32_t thr, thr2;
    __device__ __forceinline__ explicit TimePickAbs(const TimeSel& t)
        : b0(t.b0), b1(t.b1), e2(uniform(t.b2 - t.b1)), thr(t.thr), thr2(t.thr2) {}
    template <int TM>
    __device__ __forceinline__ float get(uint32_t tl, uint32_t te) const {
        if (TM == 1) return absdiff_u32(tl, te) >= thr ? b1 : b0;
        if (TM == 4) {
            const uint32_t d = absdiff_u32(tl, te);
            return (d >= thr ? b1 : b0) + (d >= thr2 ? e2 : 0.0f);
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

// Minimum / maximum over each half (lanes 0..31, 32..63) of the wavefront.
__device__ __forceinline__ void half_min_max_u32(uint32_t lo_in, uint32_t hi_in, uint32_t (&lo)[2],
                                                 uint32_t (&hi)[2]) {
    uint32_t a = lo_in, b = hi_in;
    a = umin(a, dpp_u32<kDppXor1>(a));
    b = umax(b, dpp_u32<kDppXor1>(b));
    a = umin(a, dpp_u32<kDppXor2>(a));
    b = umax(b, dpp_u32<kDppXor2>(b));
    a = umin(a, dpp_u32<kDppHalfMirror>(a));
    b = umax(b, dpp_u32<kDppHalfMirror>(b));
    a = umin(a, dpp_u32<kDppMirror>(a));
    b = umax(b, dpp_u32<kDppMirror>(b));
    lo[0] = umin(__builtin_amdgcn_readlane(a, 0), __builtin_amdgcn_readlane(a, 16));
    lo[1] = umin(__builtin_amdgcn_readlane(a, 32), __builtin_amdgcn_readlane(a, 48));
    hi[0] = umax(__builtin_amdgcn_readlane(b, 0), __builtin_amdgcn_readlane(b, 16));
    hi[1] = umax(__builtin_amdgcn_readlane(b, 32), __builtin_amdgcn_readlane(b, 48));
}

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

// Time range of each half (rows 0..31, 32..63) of one tile's timestamps, held one per lane by a
// whole wavefront (lanes with real = false are ignored; a half with no real lane gets an empty
// range lo > hi), and whether every relative time fits in 32 bits.  When they fit the ranges are
// reduced on the biased 32-bit values with DPP, else on the 64-bit values.
struct TimeRange {
    int64_t lo[2], hi[2];
    bool fit;
};
__device__ __forceinline__ TimeRange wave_time_range(int64_t t, bool real, int64_t base) {
    TimeRange r;
    r.fit = __all(rel_time_fits(t, base));
    if (r.fit) {
        const uint32_t u = rel_time_u32(t, base);
        uint32_t lo[2], hi[2];
        half_min_max_u32(real ? u : 0xffffffffu, real ? u : 0u, lo, hi);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            r.lo[h] = base + (int64_t)(int32_t)(lo[h] - 0x80000000u);
            r.hi[h] = base + (int64_t)(int32_t)(hi[h] - 0x80000000u);
        }
    } else {
        const int half = (int)(__lane_id() >> 5);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            r.lo[h] = wave_min64(real && half == h ? t : INT64_MAX);
            r.hi[h] = wave_max64(real && half == h ? t : INT64_MIN);
        }
    }
    return r;
}

// Minimum and maximum of the real lanes' times over the whole wavefront (through
// wave_time_range: DPP on 32-bit relative times when they fit, instead of 64-bit shuffles).  A
// wavefront without real lanes gets an empty range (min > max).
__device__ __forceinline__ void wave_time_minmax(int64_t t, bool real, int64_t base, int64_t& mn,
                                                 int64_t& mx) {
    const TimeRange r = wave_time_range(t, real, base);
    mn = r.lo[0] < r.lo[1] ? r.lo[0] : r.lo[1];
    mx = r.hi[0] > r.hi[1] ? r.hi[0] : r.hi[1];
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

// ---- LDS tiles --------------------------------------------------------------------------------
// A tile is kKeyTile (64) rows of D bf16, row-major without padding.  Row r is D / 8 chunks of 16
// bytes; logical chunk c sits at chunk position c ^ tile_swz(r).  With 64 LDS banks of 4 bytes
// this XOR pattern keeps three accesses free of bank conflicts: the 16-byte DMA writes of
// consecutive chunks, 16-byte reads of one chunk from 16 consecutive rows (MFMA operands with
// tile rows on lanes) and the transposing 8-byte reads of 4 rows x 64 bytes per 32 lanes (MFMA
// operands with tile columns on lanes).  tile_swz depends on bits 0..3 of r only.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
    static_assert(D == 32 || D == 64 || D == 128, "head dim");
    if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else if constexpr (D == 64) return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
    else return (r >> 2) & 3;
}
// Element offset of (row r, column col) in a tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {
    return r * D + (((col >> 3) ^ tile_swz<D>(r)) << 3) + (col & 7);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource (device pass); the host pass of a kernel only needs a placeholder of the type,
// since kernel bodies are compiled for the device only.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t buffer_rsrc;
#else
struct buffer_rsrc {
    uint32_t w[4];
};
#endif

// Transposing LDS read: within each group of 16 lanes, lane 4e + m supplies the address of 4
// consecutive bf16 of one row, and lane i receives element i % 4 of lane 4e + i / 4 as its
// element e (e = 0..3).
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
#if defined(__HIP_DEVICE_COMPILE__)
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
#else
    return bf16x4{};
#endif
}

// Per-lane element offsets of an MFMA A operand taken transposed from a tile: A (32 x 16) has
// A[m][k] = T[16 st + key(k)][m0 + m], where the k-slot order key(8g + t) = 8 (t / 4) + 4g + t % 4
// matches the C layout of a 32 x 32 MFMA result (a lane's 4r + c entries are rows 8r + 4g + c).
// Offsets are for st = 0 and one 32-column block m0; add 16 * st * D for slice st.
template <int D>
struct TrOperand {
    int off[D / 32][2];
    __device__ __forceinline__ explicit TrOperand(int lane) {
        const int s = lane & 15, q = (lane >> 4) & 1, rr = 4 * (lane >> 5) + (s >> 2);
#pragma unroll
        for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
            for (int h = 0; h < 2; ++h) off[mb][h] = tile_off<D>(rr + 8 * h, 32 * mb + 16 * q + 4 * (s & 3));
    }
    __device__ __forceinline__ bf16x8 read(const bf16* tile, int st, int mb) const {
        const bf16x4 lo = lds_read_tr4(tile + 16 * st * D + off[mb][0]);
        const bf16x4 hi = lds_read_tr4(tile + 16 * st * D + off[mb][1]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

// The same transposed read for one fixed 32-column block mb of the tile (an MFMA B operand
// B[k][n] = T[16 st + key(k)][32 mb + n] has the same per-lane layout as the A operand above).
template <int D>
struct TrBlock {
    int off[2];
    __device__ __forceinline__ TrBlock(int lane, int mb) {
        const int s = lane & 15, q = (lane >> 4) & 1, rr = 4 * (lane >> 5) + (s >> 2);
#pragma unroll
        for (int h = 0; h < 2; ++h) off[h] = tile_off<D>(rr + 8 * h, 32 * mb + 16 * q + 4 * (s & 3));
    }
    __device__ __forceinline__ bf16x8 read(const bf16* tile, int st) const {
        const bf16x4 lo = lds_read_tr4(tile + 16 * st * D + off[0]);
        const bf16x4 hi = lds_read_tr4(tile + 16 * st * D + off[1]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

// Per-lane element offsets of an MFMA A operand read along tile rows: lane (lr = l % 32, g = l / 32)
// takes row 32 blk + lr, columns 16 ks + 8g .. + 7.  Add 32 * blk * D for row block blk.
template <int D>
struct RowOperand {
    int off[D / 16];
    __device__ __forceinline__ explicit RowOperand(int lane) {
        const int lr = lane & 31, g = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) off[ks] = tile_off<D>(lr, 16 * ks + 8 * g);
    }
    __device__ __forceinline__ bf16x8 read(const bf16* tile, int blk, int ks) const {
        return *reinterpret_cast<const bf16x8*>(tile + 32 * blk * D + off[ks]);
    }
};

// Buffer resource over rows [0, n) of a bf16 slice with row stride ld (elements) starting at base:
// buffer loads past the last row return zeros.  The host guarantees the byte size fits 31 bits.
__device__ __forceinline__ buffer_rsrc rows_rsrc(const bf16* base, int n, int64_t ld, int width) {
    const int64_t bytes = n > 0 ? ((int64_t)(n - 1) * ld + width) * 2 : 0;
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, (int)bytes,
                                             0x00020000);
#else
    (void)base;
    (void)bytes;
    return buffer_rsrc{};
#endif
}

// Buffer resource over `bytes` bytes at base (raw addressing; accesses past the end are dropped
// or read zero).
__device__ __forceinline__ buffer_rsrc bytes_rsrc(const bf16* base, int64_t bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, (int)bytes, 0x00020000);
#else
    (void)base;
    (void)bytes;
    return buffer_rsrc{};
#endif
}

// Copies into LDS issued from inline assembly: the compiler then does not know that LDS is
// being written behind its back, so it neither waits for these copies before later LDS reads nor
// counts them -- the caller waits for each copy itself (wait_vmcnt / wait_vmcnt_upto, then a
// barrier) before anything reads its destination.  Used where several tiles stay in flight;
// with the builtin, every LDS read would wait for all copies.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource words over `bytes` bytes at base (loads past the end return zeros).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int32_t)((a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
    r[3] = 0x00020000;
    return r;
}

// rsrc_words over rows [0, n) of a bf16 slice with row stride ld (elements), as rows_rsrc.
__device__ __forceinline__ i32x4 rows_words(const bf16* base, int n, int64_t ld, int width) {
    return rsrc_words(base, n > 0 ? ((int64_t)(n - 1) * ld + width) * 2 : 0);
}

// LDS byte address of a pointer into __shared__ memory (the low half of its generic address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)reinterpret_cast<uintptr_t>(p));
}

// Lane l copies 4 bytes at byte offset voff to LDS address lds + 4 l.
__device__ __forceinline__ void copy4_lds_asm(i32x4 rs, uint32_t lds, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
#else
    (void)rs;
    (void)lds;
    (void)voff;
#endif
}

// Lane l copies 16 bytes at byte offset voff to LDS address lds + 16 l.
__device__ __forceinline__ void copy16_lds_asm(i32x4 rs, uint32_t lds, int voff) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rs) : "memory", "m0");
#else
    (void)rs;
    (void)lds;
    (void)voff;
#endif
}

// Copies tile rows [r0, r0 + 64) of one slice from memory straight into an LDS tile (buffer
// loads with the LDS-write option, 16 bytes per lane): instruction u of wavefront w fills the
// 1 KB block u * W + w of the tile (W wavefronts; blocks past the tile's D / 8 are skipped), lane
// l its chunk position l, so each lane reads the logical chunk that the swizzle puts there.  The
// copy is asynchronous: it is complete once the issuing wavefront has waited for vmcnt(0).
template <int D, int THREADS>
struct TileDma {
    static constexpr int C = D / 8;            // 16-byte chunks per row = 1 KB blocks per tile
    static constexpr int W = THREADS / 64;
    static constexpr int N = (C + W - 1) / W;  // blocks per wavefront
    static_assert(kKeyTile == 64, "a 1 KB block is 64 chunks");
    int off[N];  // byte offset of this lane's chunk, relative to tile row 0
    int wave;
    __device__ __forceinline__ TileDma(int tid, int64_t ld) {
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int pos = (u * W + wave) * 64 + lane;
            const int row = pos / C, c = (pos % C) ^ tile_swz<D>(row);
            off[u] = (int)(((int64_t)row * ld + 8 * c) * 2);
        }
    }
    // The same copy issued from inline assembly (see copy16_lds_asm).
    __device__ __forceinline__ void issue_asm(i32x4 rs, bf16* tile, int row_bytes) const {
#pragma unroll
        for (int u = 0; u < N; ++u)
            if (C % W == 0 || u * W + wave < C)
                copy16_lds_asm(rs, lds_addr(tile + (u * W + wave) * 512), off[u] + row_bytes);
    }
    // row_bytes = r0 * ld * 2
    __device__ __forceinline__ void issue(buffer_rsrc rs, bf16* tile, int row_bytes) const {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
        for (int u = 0; u < N; ++u)
            if (C % W == 0 || u * W + wave < C)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (lds_void*)(tile + (u * W + wave) * 512), 16, off[u] + row_bytes, 0, 0, 0);
#else
        (void)rs;
        (void)tile;
        (void)row_bytes;
#endif
    }
};

// 8-byte buffer store of 4 bf16 at byte offset voff + soff (soff wavefront-uniform); stores past
// the resource's size are dropped.
__device__ __forceinline__ void store_bf16x4(bf16x4 v, buffer_rsrc rs, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef int i32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), rs, voff, soff, 0);
#else
    (void)v;
    (void)rs;
    (void)voff;
    (void)soff;
#endif
}

// Waits for all of this wavefront's vector memory operations.  Written with the builtin (not
// inline assembly) so that the compiler's own wait tracking sees it: otherwise it still counts
// loads issued before this point as outstanding and waits for them again inside the next loop,
// where that wait would also cover copies into LDS issued since.
__device__ __forceinline__ void wait_tile_dma() {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15
    asm volatile("" ::: "memory");
}

// Waits until at most N of this wavefront's vector memory loads are outstanding (they complete in
// issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only: waits for this wavefront's LDS operations, then
// s_barrier, without the vector-memory wait that __syncthreads() implies (copies into LDS that
// are still in flight stay in flight; each wavefront waits for its own with wait_vmcnt first).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// wait_vmcnt with a wavefront-uniform count (counts above 15 wait for all).
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
    switch (n) {
        case 15: wait_vmcnt<15>(); break;
        case 14: wait_vmcnt<14>(); break;
        case 13: wait_vmcnt<13>(); break;
        case 12: wait_vmcnt<12>(); break;
        case 11: wait_vmcnt<11>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 9: wait_vmcnt<9>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 1: wait_vmcnt<1>(); break;
        default: wait_vmcnt<0>(); break;
    }
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
