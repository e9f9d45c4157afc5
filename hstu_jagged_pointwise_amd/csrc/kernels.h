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
    int32_t item_rows;      // bf16 forward: rows per item, 128 or 64 (64: key-half layout)
    float* part;            // bf16 forward: partial slots, [slot][item_rows][head_dim] fp32
    int32_t heads;
    int32_t head_dim;
    int64_t ld_in;    // token stride of q, k, v (elements)
    int64_t ld_out;   // token stride of out / dout (elements)
    int64_t ld_grad;  // token stride of dq / dk / dv (elements)
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
    // Candidate scoring against cached history (bf16 forward only).  When cache is set, seqs[b]
    // describes user b's candidates (start, n) and cache[b] its cached history; keys and values
    // come from kc / vc (token stride ld_cache) with times ts_cache, and each candidate row also
    // sees its own k and v.
    const CacheSeq* cache;
    const void* kc;
    const void* vc;
    const int64_t* ts_cache;
    int64_t ld_cache;
    // bf16 backward with stored dS (head_dim 64 and 128): when ds is set, the dK/dV pass also
    // writes dS * N of every pair it visits to ds, and the dQ pass reads it back instead of
    // recomputing S and dP.  Sequence b's chunks (geometry.h: one 128 x 64 block per key block
    // and query tile, row = key, column = query) start at ds + ds_off[b].
    void* ds;
    const int64_t* ds_off;
    // With ds, the dK/dV pass also sums the bias-table gradients ([H][128] fp32, already zeroed,
    // either may be NULL) and the dQ pass does not.
    float* gpos;
    float* gts;
    // With ds: the bias-mode records the dK/dV pass launch writes in a pass of its own before
    // the products (32 bytes per sequence, 128-key block, query tile and wavefront: dS chunk
    // count / heads x 256 bytes) and the query times relative to each sequence's first (uint32
    // per token; with a time bias only).
    void* modes;
    uint32_t* tq_rel;
    // Layer backward: when nonzero, dQ, dK and dV leave multiplied by SiLU'(h), the derivative of
    // the projection's SiLU at its pre-activation h (bf16), found gate_delta bytes after each
    // output element (dQ, dK, dV are blocks of dH, and H has the same layout).
    int64_t gate_delta;
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
// Clears up to four fp32 buffers (NULL entries or zero counts are skipped) with one launch.
hipError_t launch_zero_f32_list(float* const* ptrs, const int64_t* counts, int k, hipStream_t s);

// LayerNorm over `width` features of each row of a (bf16), times gate u (token stride ldu),
// written to out (dense, may alias a).
hipError_t launch_ln_gate_bf16(const void* a, const void* u, int64_t ldu, void* out,
                               int64_t rows, int32_t width, float eps, hipStream_t s);
hipError_t launch_ln_gate_f32(const void* a, const void* u, int64_t ldu, void* out,
                              int64_t rows, int32_t width, float eps, hipStream_t s);

// Layer backward, per token row of width Hd: recomputes LayerNorm(a), writes the gate product
// g = xhat * u (bf16), the attention-output gradient da (bf16) and the U-slot gradient before
// the projection, dhu = dg * xhat * SiLU'(hu) (bf16, token stride lddh).  u and hu have token
// stride ldz; a, g, da stride width; dg is fp32 with stride width.
hipError_t launch_ln_gate_bwd_bf16(const void* a, const void* u, const void* hu, int64_t ldz,
                                   const float* dg, void* g, void* da, void* dhu, int64_t lddh,
                                   int64_t rows, int32_t width, float eps, hipStream_t s);

// C (M x N) = epilogue(op(A) op(B)), bf16 operands, fp32 accumulation.
enum GemmEpilogue : int32_t {
    kEpiSilu = 0,       // C = SiLU(acc) (bf16); if c2, also c2 = acc (bf16, stride ldc)
    kEpiResidual = 1,   // C = acc + R (bf16)
    kEpiStoreF32 = 2,   // C = acc (fp32)
    kEpiAtomicF32 = 3,  // C += acc (fp32, atomic; K may be split over workgroups)
};
struct GemmArgs {
    const void* a;      // at ? A^T (K x M) : A (M x K), row stride lda
    int64_t lda;
    const void* b;      // bt ? B^T (N x K) : B (K x N), row stride ldb
    int64_t ldb;
    int64_t M;
    int32_t N;          // multiple of 128
    int64_t K;          // multiple of 64 unless (at && !bt)
    int64_t kchunk;     // K per workgroup (0 = all); a split needs at && !bt and kEpiAtomicF32
    void* c;
    int64_t ldc;
    void* c2;
    const void* r;
    int64_t ldr;
    bool at;
    bool bt;            // at && bt is not supported
    int32_t epilogue;
    int32_t compute_units;           // for the persistent grid (0: 256)
    int32_t mtiles, ntiles, splits;  // set by launch_gemm
    int32_t rounds;                  // set by launch_gemm: tile numbers per workgroup
};
hipError_t launch_gemm(const GemmArgs& g, hipStream_t s);

// Stochastic Length compaction: rows of jagged src (offsets so, src_rows rows of row_bytes)
// gathered into jagged dst (offsets dof); sequence b keeps the rows starting at keep_start[b]
// (NULL: its last rows).  Offsets and keep_start are device arrays.
hipError_t launch_jagged_select(int32_t B, const int64_t* so, int64_t src_rows, const int64_t* dof,
                                int64_t dst_rows, const int64_t* keep_start, int64_t row_bytes,
                                const void* src, void* dst, hipStream_t s);

}  // namespace hstu
