// jagged.hip -- Stochastic Length compaction on gfx950 (page 1 section 2.1.3, algorithm-level
// optimisation: training sequences are cut to a randomly drawn length, which makes the batch
// sparser and the encoder cheaper).  The draw is the caller's; this kernel moves the kept tokens:
// sequence b keeps dst_len_b = dst_off[b + 1] - dst_off[b] consecutive rows starting at
// keep_start[b] within it (the last dst_len_b rows when keep_start is NULL) and they are packed
// into a new jagged tensor with offsets dst_off.
//
// One thread per 16-byte (or 8-byte) piece of an output row: a streaming copy, bound by HBM.
// The owning sequence of an output row is found by binary search in dst_off.  Source rows that
// fall outside their sequence or the source tensor are written as zeros instead of read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace hstu {
namespace {

constexpr int kSelThreads = 256;

template <typename Chunk>
__global__ __launch_bounds__(kSelThreads) void jagged_select_kernel(
    int32_t B, const int64_t* __restrict__ so, int64_t src_rows, const int64_t* __restrict__ dof,
    int64_t dst_rows, const int64_t* __restrict__ keep_start, int64_t chunks,
    const Chunk* __restrict__ src, Chunk* __restrict__ dst) {
    const int64_t idx = (int64_t)blockIdx.x * kSelThreads + threadIdx.x;
    if (idx >= dst_rows * chunks) return;
    const int64_t r = idx / chunks, c = idx - r * chunks;
    int lo = 0, hi = B - 1;  // last b with dof[b] <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (dof[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    const int64_t n = so[lo + 1] - so[lo], m = dof[lo + 1] - dof[lo];
    const int64_t j = (keep_start ? keep_start[lo] : n - m) + (r - dof[lo]);
    const int64_t sr = so[lo] + j;
    Chunk v{};
    if (j >= 0 && j < n && sr >= 0 && sr < src_rows) v = src[sr * chunks + c];
    dst[idx] = v;
}

template <typename Chunk>
hipError_t launch_t(int32_t B, const int64_t* so, int64_t src_rows, const int64_t* dof,
                    int64_t dst_rows, const int64_t* keep_start, int64_t row_bytes,
                    const void* src, void* dst, hipStream_t s) {
    const int64_t chunks = row_bytes / (int64_t)sizeof(Chunk);
    const int64_t total = dst_rows * chunks;
    hipLaunchKernelGGL((jagged_select_kernel<Chunk>),
                       dim3((unsigned)((total + kSelThreads - 1) / kSelThreads)), dim3(kSelThreads),
                       0, s, B, so, src_rows, dof, dst_rows, keep_start, chunks,
                       static_cast<const Chunk*>(src), static_cast<Chunk*>(dst));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_jagged_select(int32_t B, const int64_t* so, int64_t src_rows, const int64_t* dof,
                                int64_t dst_rows, const int64_t* keep_start, int64_t row_bytes,
                                const void* src, void* dst, hipStream_t s) {
    if (dst_rows <= 0) return hipSuccess;
    if (B <= 0 || row_bytes <= 0 || row_bytes % 8 != 0) return hipErrorInvalidValue;
    if ((dst_rows * row_bytes / 8) / kSelThreads >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    const bool wide = row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
                      (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
    return wide ? launch_t<uint4>(B, so, src_rows, dof, dst_rows, keep_start, row_bytes, src, dst, s)
                : launch_t<uint2>(B, so, src_rows, dof, dst_rows, keep_start, row_bytes, src, dst, s);
}

}  // namespace hstu
