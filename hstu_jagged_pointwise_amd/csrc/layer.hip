// layer.hip -- the row-wise parts of an HSTU layer on gfx950 (page 1 section 2.1.2, equation (3):
// pointwise transformation LayerNorm(A) * U; page 1 section 2.1.3: fused elementwise work) and
// of its backward.  The matrix products are in gemm.hip.
//
// ln_gate_kernel: one wavefront per token; mean and biased variance over the row in fp32 with
// cross-lane reductions, then (a - mean) * rsqrt(var + eps) * u.
//
// ln_gate_bwd_kernel: one wavefront per token.  With xhat = (a - mean) * rstd and the incoming
// gradient dg of g = xhat * u: du = dg * xhat, dxhat = dg * u and the LayerNorm backward
// da = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)).  The same pass writes g (for
// dW2 = G^T dY) and turns du into the gradient before the U projection's SiLU (the V, Q and K
// blocks get theirs in the attention backward's stores).
#include "device_common.h"
#include "kernels.h"

namespace hstu {
namespace {

// ---- LayerNorm x gate ------------------------------------------------------------------------

constexpr int kLnRowsPerBlock = 4;
constexpr int kLnMaxChunks = 8;  // width <= 64 lanes * 8 * 8

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out) {
    if constexpr (sizeof(T) == 2) {
        bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
    } else {
        f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { out[e] = a[e]; out[4 + e] = b[e]; }
    }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v) {
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<bf16x8*>(p) = pack8(v);
    } else {
        f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        *reinterpret_cast<f32x4*>(p) = a;
        *reinterpret_cast<f32x4*>(p + 4) = b;
    }
}

template <typename T>
__global__ __launch_bounds__(64 * kLnRowsPerBlock) void ln_gate_kernel(
    const T* a, const T* __restrict__ u, int64_t ldu, T* out, int64_t rows, int width, float eps) {
    const int64_t row = (int64_t)blockIdx.x * kLnRowsPerBlock + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const T* ar = a + row * width;
    float x[kLnMaxChunks][8];
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kLnMaxChunks; ++k) {
        const int c = 8 * (lane + 64 * k);
        if (c < width) {
            load8(ar + c, x[k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += x[k][e];
        }
    }
    const float mean = wave_sum(s) / (float)width;
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < kLnMaxChunks; ++k) {
        const int c = 8 * (lane + 64 * k);
        if (c < width)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = x[k][e] - mean;
                v = fmaf(d, d, v);
            }
    }
    const float rstd = rsqrtf(wave_sum(v) / (float)width + eps);
    const T* ur = u + row * ldu;
    T* orow = out + row * width;
#pragma unroll
    for (int k = 0; k < kLnMaxChunks; ++k) {
        const int c = 8 * (lane + 64 * k);
        if (c < width) {
            float uu[8], y[8];
            load8(ur + c, uu);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = (x[k][e] - mean) * rstd * uu[e];
            store8(orow + c, y);
        }
    }
}


__global__ __launch_bounds__(64 * kLnRowsPerBlock) void ln_gate_bwd_kernel(
    const bf16* a, const bf16* __restrict__ u, const bf16* __restrict__ hu, int64_t ldz,
    const float* __restrict__ dg, bf16* __restrict__ g, bf16* __restrict__ da,
    bf16* __restrict__ dhu, int64_t lddh, int64_t rows, int width, float eps) {
    const int64_t row = (int64_t)blockIdx.x * kLnRowsPerBlock + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const bf16* ar = a + row * width;
    float x[kLnMaxChunks][8], dx[kLnMaxChunks][8];
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kLnMaxChunks; ++k) {
        const int c = 8 * (lane + 64 * k);
        if (c < width) {
            load8(ar + c, x[k]);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += x[k][e];
        }
    }
    const float mean = wave_sum(s) / (float)width;
    float v = 0.0f;
#pragma unroll
    for (int k = 0; k < kLnMaxChunks; ++k) {
        const int c = 8 * (lane + 64 * k);
        if (c < width)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = x[k][e] - mean;
                v = fmaf(d, d, v);
            }
    }
    const float rstd = rsqrtf(wave_sum(v) / (float)width + eps);
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int k = 0; k < kLnMaxChunks; ++k) {
        const int c = 8 * (lane + 64 * k);
        if (c < width) {
            float uu[8], hh[8], gg[8], gout[8], dh[8];
            load8(u + row * ldz + c, uu);
            load8(hu + row * ldz + c, hh);
            load8(dg + row * width + c, gg);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xh = (x[k][e] - mean) * rstd;
                x[k][e] = xh;
                gout[e] = xh * uu[e];
                dx[k][e] = gg[e] * uu[e];
                dh[e] = gg[e] * xh * silu_deriv(hh[e]);
                s1 += dx[k][e];
                s2 = fmaf(dx[k][e], xh, s2);
            }
            store8(g + row * width + c, gout);
            store8(dhu + row * lddh + c, dh);
        }
    }
    const float m1 = wave_sum(s1) / (float)width, m2 = wave_sum(s2) / (float)width;
#pragma unroll
    for (int k = 0; k < kLnMaxChunks; ++k) {
        const int c = 8 * (lane + 64 * k);
        if (c < width) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = (dx[k][e] - m1 - x[k][e] * m2) * rstd;
            store8(da + row * width + c, o);
        }
    }
}

template <typename T>
hipError_t launch_ln(const void* a, const void* u, int64_t ldu, void* out, int64_t rows, int width,
                     float eps, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (width % 8 != 0 || width > 64 * 8 * kLnMaxChunks) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((rows + kLnRowsPerBlock - 1) / kLnRowsPerBlock);
    hipLaunchKernelGGL(ln_gate_kernel<T>, dim3(blocks), dim3(64 * kLnRowsPerBlock), 0, s,
                       static_cast<const T*>(a), static_cast<const T*>(u), ldu,
                       static_cast<T*>(out), rows, width, eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ln_gate_bf16(const void* a, const void* u, int64_t ldu, void* out, int64_t rows,
                               int32_t width, float eps, hipStream_t s) {
    return launch_ln<bf16>(a, u, ldu, out, rows, width, eps, s);
}

hipError_t launch_ln_gate_f32(const void* a, const void* u, int64_t ldu, void* out, int64_t rows,
                              int32_t width, float eps, hipStream_t s) {
    return launch_ln<float>(a, u, ldu, out, rows, width, eps, s);
}

hipError_t launch_ln_gate_bwd_bf16(const void* a, const void* u, const void* hu, int64_t ldz,
                                   const float* dg, void* g, void* da, void* dhu, int64_t lddh,
                                   int64_t rows, int32_t width, float eps, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (width % 8 != 0 || width > 64 * 8 * kLnMaxChunks) return hipErrorInvalidValue;
    const unsigned blocks = (unsigned)((rows + kLnRowsPerBlock - 1) / kLnRowsPerBlock);
    hipLaunchKernelGGL(ln_gate_bwd_kernel, dim3(blocks), dim3(64 * kLnRowsPerBlock), 0, s,
                       static_cast<const bf16*>(a), static_cast<const bf16*>(u),
                       static_cast<const bf16*>(hu), ldz, dg, static_cast<bf16*>(g),
                       static_cast<bf16*>(da), static_cast<bf16*>(dhu), lddh, rows, width, eps);
    return hipGetLastError();
}


}  // namespace hstu
