// kernels.h -- launch interface between the C-ABI layer and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geometry.h"

namespace hstu {

// Everything a jagged-attention kernel needs; pointers are device pointers.
struct AttnParams {
    const SeqInfo* seqs;
    const WorkUnit* units;
    int32_t num_units;
    const FwdItem* items;   // bf16 forward: work items (row blocks, the longest split by key tiles)
    int32_t num_items;
    const FixItem* fix;     // bf16 forward: split row blocks to sum
    int32_t num_fix;
    float* part;            // bf16 forward: partial slots, [slot][128 rows][head_dim] fp32
    int32_t heads;
    int32_t head_dim;
    int64_t ld_in;    // token stride of q, k, v (elements)
    int64_t ld_out;   // token stride of out / dout / dq / dk / dv (elements)
    float alpha;
    float inv_n;      // 1 / max_seqlen
    const int64_t* ts;
    const float* rab_pos;
    const float* rab_ts;
    const void* q;
    const void* k;
    const void* v;
    void* out;        // forward output
    const void* dout; // backward input
    void* dq;
    void* dk;
    void* dv;
    float* drab_pos;
    float* drab_ts;
};

hipError_t launch_attn_fwd_bf16(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_fwd_f32(const AttnParams& p, hipStream_t s);
// Backward passes: dK/dV over `units` = key-block units; dQ (and bias gradients, which the
// caller has zeroed) over `units` = row-block units.
hipError_t launch_attn_bwd_dkdv_bf16(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_bwd_dq_bf16(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_bwd_dkdv_f32(const AttnParams& p, hipStream_t s);
hipError_t launch_attn_bwd_dq_f32(const AttnParams& p, hipStream_t s);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);

// LayerNorm over `width` features of each row of a (bf16), times gate u (token stride ldu),
// written to out (dense, may alias a).
hipError_t launch_ln_gate_bf16(const void* a, const void* u, int64_t ldu, void* out,
                               int64_t rows, int32_t width, float eps, hipStream_t s);
hipError_t launch_ln_gate_f32(const void* a, const void* u, int64_t ldu, void* out,
                              int64_t rows, int32_t width, float eps, hipStream_t s);

// C = epilogue(A (M x K) * B (K x N)); row-major bf16; epilogue 0 = SiLU, 1 = + R (residual,
// M x N).  Requires K % 64 == 0 and N % 128 == 0.
hipError_t launch_gemm_bf16(const void* A, const void* B, void* C, const void* R, int64_t M,
                            int32_t N, int32_t K, int32_t epilogue, hipStream_t s);

}  // namespace hstu
