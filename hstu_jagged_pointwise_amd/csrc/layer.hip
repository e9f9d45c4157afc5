// layer.hip -- the dense parts of an HSTU layer on gfx950 (page 1 section 2.1.2, equations (1)
// and (3): pointwise projection Z = SiLU(X W1), pointwise transformation
// Y = (LayerNorm(A) * U) W2 + X; page 1 section 2.1.3: only two linear layers, fused
// elementwise work).
//
// gemm_kernel: C = epilogue(A B), A (M x K) and B (K x N) row-major bf16, fp32 accumulation with
// v_mfma_f32_32x32x16_bf16.  128 x 128 output tile per workgroup (4 wavefronts, 64 x 64 each),
// K advanced 64 at a time through two LDS buffers.  B tiles are stored transposed (n-major) so
// both MFMA operands read 16 contiguous bytes per lane.  The epilogue applies SiLU (projection)
// or adds the residual before the single bf16 store.
//
// ln_gate_kernel: one wavefront per token; mean and biased variance over the row in fp32 with
// cross-lane reductions, then (a - mean) * rsqrt(var + eps) * u.
#include "device_common.h"
#include "kernels.h"

namespace hstu {
namespace {

constexpr int kGT = 256;  // threads
constexpr int kGM = 128, kGN = 128, kGK = 64;
constexpr int kGP = kGK + 8;  // LDS pitch (elements) of both tiles

struct GemmSmem {
    bf16 a[2][kGM * kGP];
    bf16 b[2][kGN * kGP];  // transposed: [n][k]
};

template <int EPI>
__global__ __launch_bounds__(kGT, 2) void gemm_kernel(const bf16* __restrict__ A,
                                                      const bf16* __restrict__ B,
                                                      bf16* __restrict__ C,
                                                      const bf16* __restrict__ R, int64_t M,
                                                      int N, int K) {
    __shared__ __attribute__((aligned(16))) GemmSmem sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, lr = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * kGM;
    const int n0 = blockIdx.x * kGN;

    bf16x8 ar[4], br[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int id = tid + kGT * u, row = id >> 3, ch = id & 7;
            const int64_t m = m0 + row;
            ar[u] = m < M ? load_bf16x8(A + m * K + k0 + 8 * ch) : bf16x8{};
        }
        const int kg = tid & 15, ch = tid >> 4;  // 4 k-rows x 8 columns
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            br[kk] = load_bf16x8(B + (int64_t)(k0 + 4 * kg + kk) * N + n0 + 8 * ch);
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int id = tid + kGT * u, row = id >> 3, ch = id & 7;
            *reinterpret_cast<bf16x8*>(&sm.a[buf][row * kGP + 8 * ch]) = ar[u];
        }
        const int kg = tid & 15, ch = tid >> 4;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 w = {br[0][e], br[1][e], br[2][e], br[3][e]};
            *reinterpret_cast<bf16x4*>(&sm.b[buf][(8 * ch + e) * kGP + 4 * kg]) = w;
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{};

    const int nk = K / kGK;
    load(0);
    store(0);
    if (nk > 1) load(kGK);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const int buf = t & 1;
#pragma unroll
        for (int ks = 0; ks < kGK / 16; ++ks) {
            bf16x8 a[2], b[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                a[mb] = *reinterpret_cast<const bf16x8*>(
                    &sm.a[buf][(64 * wm + 32 * mb + lr) * kGP + 16 * ks + 8 * g]);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                b[nb] = *reinterpret_cast<const bf16x8*>(
                    &sm.b[buf][(64 * wn + 32 * nb + lr) * kGP + 16 * ks + 8 * g]);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(a[mb], b[nb], acc[mb][nb]);
        }
        if (t + 1 < nk) store(buf ^ 1);
        if (t + 2 < nk) load((t + 2) * kGK);
        __syncthreads();
    }

#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t m = m0 + 64 * wm + 32 * mb + 8 * r + 4 * g + c;
                    const int nn = n0 + 64 * wn + 32 * nb + lr;
                    if (m < M) {
                        float x = acc[mb][nb][4 * r + c];
                        if (EPI == 0) x = x * fast_sigmoid(x);
                        else x += (float)R[m * N + nn];
                        C[m * N + nn] = (bf16)x;
                    }
                }
}

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

hipError_t launch_gemm_bf16(const void* A, const void* B, void* C, const void* R, int64_t M,
                            int32_t N, int32_t K, int32_t epilogue, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (N % kGN != 0 || K % kGK != 0 || (epilogue == 1 && !R)) return hipErrorInvalidValue;
    dim3 grid(N / kGN, (unsigned)((M + kGM - 1) / kGM));
    if (epilogue == 0)
        hipLaunchKernelGGL(gemm_kernel<0>, grid, dim3(kGT), 0, s, static_cast<const bf16*>(A),
                           static_cast<const bf16*>(B), static_cast<bf16*>(C), nullptr, M, N, K);
    else
        hipLaunchKernelGGL(gemm_kernel<1>, grid, dim3(kGT), 0, s, static_cast<const bf16*>(A),
                           static_cast<const bf16*>(B), static_cast<bf16*>(C),
                           static_cast<const bf16*>(R), M, N, K);
    return hipGetLastError();
}

hipError_t launch_ln_gate_bf16(const void* a, const void* u, int64_t ldu, void* out, int64_t rows,
                               int32_t width, float eps, hipStream_t s) {
    return launch_ln<bf16>(a, u, ldu, out, rows, width, eps, s);
}

hipError_t launch_ln_gate_f32(const void* a, const void* u, int64_t ldu, void* out, int64_t rows,
                              int32_t width, float eps, hipStream_t s) {
    return launch_ln<float>(a, u, ldu, out, rows, width, eps, s);
}

}  // namespace hstu
