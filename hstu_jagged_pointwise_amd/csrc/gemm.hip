// gemm.hip -- the dense products of an HSTU layer and of its backward on gfx950 (page 1 section
// 2.1.2, equations (1) and (3): Z = SiLU(X W1) and Y = (LayerNorm(A) * U) W2 + X; their
// gradients dW1 = X^T dH, dX = dH W1^T + dY, dW2 = G^T dY and dG = dY W2^T).
//
// C (M x N) = epilogue(op(A) op(B)) in bf16 with fp32 accumulation on v_mfma_f32_32x32x16_bf16.
// Each workgroup (4 wavefronts, 64 x 64 outputs each) computes 128 x 128 tiles over a range of
// K, 64 at a time; workgroups are persistent (two per compute unit) and run sequences of tiles.  Operand tiles go from memory straight into LDS with buffer loads that write
// LDS (no register staging), double buffered, in the XOR-swizzled tile layout of the attention
// kernels:
//   * an operand whose rows are the MFMA's row index and whose columns are K (A row-major,
//     or B given as B^T row-major) is stored as 128 rows x 64 K and read 16 bytes per lane;
//   * an operand stored K-major (A given as A^T, or B row-major) is stored as 64 K rows x 128
//     and read with transposing 8-byte LDS reads in natural K order.
// K-major operands may have any K (rows past the end read as zero), so the token dimension of
// the weight gradients can be the reduction dimension and can be split over blockIdx.z; those
// launches add their fp32 partial results atomically into an output the caller has cleared.
// bf16 results leave through LDS (the operand buffer the last K step read) so that every store
// instruction writes whole row segments.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace hstu {
namespace {

constexpr int kGT = 256;               // threads
constexpr int kXcds = 8;
constexpr int kGM = 128, kGN = 128, kGK = 64;
constexpr int kGTile = kGM * kGK;      // elements of one operand stage (either form)

// Transposed operand in natural K order: lane (lr = l % 32, g = l / 32) receives columns
// c0 + lr of K rows 16 st + 8g + 0..7 from a 64 x D tile.  In each group of 16 lanes, lane s
// supplies the address of row 8g + 4h + s / 4, columns 16 q + 4 (s % 4) .. + 3 (q = bit 4 of
// the lane), so that after the transposing read lane i holds row 8g + 4h + e, column 16 q + i.
template <int D, int NB>
struct TrOperandNat {
    // Offsets for the wavefront's own column blocks cb0 .. cb0 + NB - 1 (32 columns each), so
    // that the reads index this array with constants only (an array indexed at run time is
    // moved to LDS by the compiler, and every K step then waits for an extra LDS round trip).
    int off[NB][2];
    __device__ __forceinline__ TrOperandNat(int lane, int cb0) {
        const int s = lane & 15, q = (lane >> 4) & 1, g = lane >> 5;
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                off[i][h] = tile_off<D>(8 * g + 4 * h + (s >> 2), 32 * ((cb0 + i) & (D / 32 - 1)) + 16 * q + 4 * (s & 3));
    }
    __device__ __forceinline__ bf16x8 read(const bf16* tile, int st, int i) const {
        const bf16x4 lo = lds_read_tr4(tile + 16 * st * D + off[i][0]);
        const bf16x4 hi = lds_read_tr4(tile + 16 * st * D + off[i][1]);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

struct GemmSmem {
    bf16 a[2][kGTile];
    bf16 b[2][kGTile];
};

__device__ __forceinline__ float silu_f(float x) { return x * fast_sigmoid(x); }

// Orders a wavefront's LDS accesses: its earlier LDS writes and reads complete before any later
// one issues, and the compiler moves no LDS access across this point (lanes read what other lanes
// of the same wavefront wrote).
__device__ __forceinline__ void lds_wave_sync() {
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// One output tile: rows [m0, m0 + 128), columns [n0, n0 + 128), K range [kbeg, kend).
struct GemmTile {
    int64_t m0, kbeg, kend;
    int n0, nk;
};

// Tile number -> tile, XCD-aware.  Workgroups are dispatched to the 8 XCDs round robin
// (workgroup w runs on XCD w % 8), and the persistent workgroup w takes tile numbers w, w + G,
// ... (G, the grid, a multiple of 8), so all its tiles have numbers of one residue mod 8.  The
// numbering puts all tiles that share one A block (same row tile and K range: a "group") on
// consecutive numbers of one residue, i.e. on one XCD at about the same time: the A block is
// fetched into that XCD's L2 once.  Numbers past the last group are skipped.
__device__ __forceinline__ bool gemm_tile(const GemmArgs& g, int id, GemmTile& t) {
    const int xcd = id % kXcds, slot = id / kXcds;
    const int group = (slot / g.ntiles) * kXcds + xcd;
    if (group >= g.mtiles * g.splits) return false;
    t.m0 = (int64_t)(group % g.mtiles) * kGM;
    t.n0 = (slot % g.ntiles) * kGN;
    t.kbeg = (int64_t)(group / g.mtiles) * g.kchunk;
    t.kend = min(g.K, t.kbeg + g.kchunk);
    t.nk = (int)((t.kend - t.kbeg + kGK - 1) / kGK);
    return t.kbeg < t.kend;
}

// AT: A is given as A^T (K x M, row stride lda); else A is M x K.  BT: B is given as B^T (N x K,
// row stride ldb); else B is K x N.
//
// Persistent: each workgroup runs a sequence of tiles and keeps one K step in flight across tile
// boundaries (the first step of the next tile loads while the current tile's last step and its
// epilogue run), so a tile's first load does not stall the matrix units.
template <bool AT, bool BT, int EPI>
__global__ __launch_bounds__(kGT, 2) void gemm_kernel(const GemmArgs g) {
    __shared__ __attribute__((aligned(16))) GemmSmem sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 5, lr = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;
    const bf16* A = static_cast<const bf16*>(g.a);
    const bf16* B = static_cast<const bf16*>(g.b);
    const TileDma<AT ? 128 : 64, kGT> adma(tid, g.lda);
    const TileDma<BT ? 64 : 128, kGT> bdma(tid, g.ldb);

    // starts the copy of K step st of tile t into buffer buf.  The copies are issued from inline
    // assembly: with the copy builtin the compiler waits for every copy in flight before the
    // step's LDS reads, i.e. for the next step's copy; each step waits for its own copy
    // explicitly (wait_tile_dma, then the barrier).
    auto issue = [&](const GemmTile& t, int st, int buf) {
        const int64_t kk = (int64_t)st * kGK;  // relative to kbeg
        const int krows = (int)(t.kend - t.kbeg);
        if constexpr (AT) {
            const i32x4 rs = rows_words(A + t.kbeg * g.lda + t.m0, krows, g.lda, kGM);
            adma.issue_asm(rs, sm.a[buf], (int)(kk * g.lda * 2));
        } else {
            const i32x4 rs = rows_words(A + t.m0 * g.lda, (int)min<int64_t>(g.M - t.m0, kGM), g.lda, (int)g.K);
            adma.issue_asm(rs, sm.a[buf], (int)((t.kbeg + kk) * 2));
            adma.issue_asm(rs, sm.a[buf] + 64 * kGK, (int)((t.kbeg + kk + 64 * g.lda) * 2));
        }
        if constexpr (BT) {
            const i32x4 rs = rows_words(B + (int64_t)t.n0 * g.ldb, kGN, g.ldb, (int)g.K);
            bdma.issue_asm(rs, sm.b[buf], (int)((t.kbeg + kk) * 2));
            bdma.issue_asm(rs, sm.b[buf] + 64 * kGK, (int)((t.kbeg + kk + 64 * g.ldb) * 2));
        } else {
            const i32x4 rs = rows_words(B + t.kbeg * g.ldb + t.n0, krows, g.ldb, kGN);
            bdma.issue_asm(rs, sm.b[buf], (int)(kk * g.ldb * 2));
        }
    };
    // next tile of this workgroup at or after number id (id advanced past it), if any
    const int total = (int)gridDim.x * g.rounds;
    auto next_tile = [&](int& id, GemmTile& t) {
        for (; id < total; id += gridDim.x)
            if (gemm_tile(g, id, t)) { id += gridDim.x; return true; }
        return false;
    };

    const RowOperand<64> rowop(lane);
    const TrOperandNat<128, 2> tra(lane, 2 * wm), trb(lane, 2 * wn);
    int id = blockIdx.x;
    GemmTile cur, nxt;
    if (!next_tile(id, cur)) return;  // uniform: whole workgroup
    bool more = next_tile(id, nxt);
    issue(cur, 0, 0);
    int buf = 0;
    for (;;) {
        f32x16 acc[2][2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = f32x16{};
        for (int t = 0; t < cur.nk; ++t) {
            wait_tile_dma();
            __syncthreads();
            // operand fragments of 16-wide K slices, two slices in registers at a time
            bf16x8 a[2][2], b[2][2];
            auto load = [&](int ks, int slot) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
                    a[slot][mb] = AT ? tra.read(sm.a[buf], ks, mb)
                                     : rowop.read(sm.a[buf], 2 * wm + mb, ks);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    b[slot][nb] = BT ? rowop.read(sm.b[buf], 2 * wn + nb, ks)
                                     : trb.read(sm.b[buf], ks, nb);
            };
            load(0, 0);
            if (t + 1 < cur.nk) issue(cur, t + 1, buf ^ 1);
            else if (more) issue(nxt, 0, buf ^ 1);
#pragma unroll
            for (int ks = 0; ks < kGK / 16; ++ks) {
                if (ks + 1 < kGK / 16) load(ks + 1, (ks + 1) & 1);
                const int sl = ks & 1;
                // Stored results come out transposed (C^T = B^T A^T: a lane holds one row of C
                // and 4 consecutive columns per entry group, for vector stores); atomic results
                // keep C's layout (consecutive lanes on consecutive columns: coalesced atomics).
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        acc[mb][nb] = EPI == kEpiAtomicF32 ? mfma32(a[sl][mb], b[sl][nb], acc[mb][nb])
                                                           : mfma32(b[sl][nb], a[sl][mb], acc[mb][nb]);
            }
            buf ^= 1;
        }
        const int64_t m0 = cur.m0;
        const int n0 = cur.n0;
        if constexpr (EPI == kEpiAtomicF32) {
            // lane holds C[64 wm + 32 mb + 8 r + 4 gq + c][64 wn + 32 nb + lr]
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int64_t m = m0 + 64 * wm + 32 * mb + 8 * r + 4 * gq + c;
                            const int64_t n = n0 + 64 * wn + 32 * nb + lr;
                            if (m < g.M)
                                unsafeAtomicAdd(static_cast<float*>(g.c) + m * g.ldc + n,
                                                acc[mb][nb][4 * r + c]);
                        }
        } else if constexpr (EPI == kEpiStoreF32) {
            // lane holds C[64 wm + 32 mb + lr][64 wn + 32 nb + 8 r + 4 gq + c], c = 0..3: fp32
            // results are stored from there, 16 bytes per lane (staged through LDS they were
            // slower on the layer shapes)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int64_t m = m0 + 64 * wm + 32 * mb + lr;
                if (m >= g.M) continue;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        *reinterpret_cast<f32x4*>(static_cast<float*>(g.c) + m * g.ldc + n0 + 64 * wn + 32 * nb + 8 * r + 4 * gq) =
                            f32x4{acc[mb][nb][4 * r], acc[mb][nb][4 * r + 1], acc[mb][nb][4 * r + 2], acc[mb][nb][4 * r + 3]};
            }
        } else {
            // The wavefront's 64 x 64 results go out through LDS, 32 rows at a time in fp32, so
            // that a store instruction writes 8 whole 128-byte row segments (from the MFMA
            // layout a lane holds 4 columns of one row: 32 rows per store instruction).  The
            // staging area is the operand buffer the last K step read, 8 KB per wavefront, free
            // once every wavefront is past that step; the next tile's copies go to the other
            // buffer until its first step's barrier.  16-byte chunks of a staged row are
            // XOR-swizzled by the row's low 4 bits: conflict-free writes and reads.
            __syncthreads();
            float* const stage = reinterpret_cast<float*>(wave < 2 ? sm.a[buf ^ 1] : sm.b[buf ^ 1]) + (wave & 1) * 2048;
            const int cp = lane & 7;  // read-back: 8 consecutive columns 8 cp .. 8 cp + 7 of a row
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int64_t mrow = m0 + 64 * wm + 32 * mb;  // first row of this half
                const int n = n0 + 64 * wn + 8 * cp;
                // the residual values first: the compiler may not move a load of r above a store
                // to c, which it cannot prove apart
                bf16x8 res[4];
                if constexpr (EPI == kEpiResidual)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t m = mrow + (lane >> 3) + 8 * i;
                        if (m < g.M)
                            res[i] = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(g.r) + m * g.ldr + n);
                    }
                // lane holds C[mrow + lr][64 wn + 32 nb + 8 r + 4 gq + c], c = 0..3
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int chunk = 8 * nb + 2 * r + gq;
                        *reinterpret_cast<f32x4*>(stage + lr * 64 + 4 * (chunk ^ (lr & 15))) =
                            f32x4{acc[mb][nb][4 * r], acc[mb][nb][4 * r + 1], acc[mb][nb][4 * r + 2],
                                  acc[mb][nb][4 * r + 3]};
                    }
                lds_wave_sync();
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = (lane >> 3) + 8 * i;
                    const f32x4 lo = *reinterpret_cast<const f32x4*>(stage + row * 64 + 4 * ((2 * cp) ^ (row & 15)));
                    const f32x4 hi = *reinterpret_cast<const f32x4*>(stage + row * 64 + 4 * ((2 * cp + 1) ^ (row & 15)));
                    const int64_t m = mrow + row;
                    if (m >= g.M) continue;
                    const float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    if constexpr (EPI == kEpiSilu) {
                        bf16x8 y, z;
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            y[c] = (bf16)silu_f(x[c]);
                            z[c] = (bf16)x[c];
                        }
                        *reinterpret_cast<bf16x8*>(static_cast<bf16*>(g.c) + m * g.ldc + n) = y;
                        if (g.c2) *reinterpret_cast<bf16x8*>(static_cast<bf16*>(g.c2) + m * g.ldc + n) = z;
                    } else {
                        bf16x8 y;
#pragma unroll
                        for (int c = 0; c < 8; ++c) y[c] = (bf16)(x[c] + (float)res[i][c]);
                        *reinterpret_cast<bf16x8*>(static_cast<bf16*>(g.c) + m * g.ldc + n) = y;
                    }
                }
                lds_wave_sync();  // the next half overwrites what this one read
            }
        }
        if (!more) break;
        cur = nxt;
        more = next_tile(id, nxt);
    }
}

template <bool AT, bool BT>
hipError_t launch_t(const GemmArgs& g, dim3 grid, hipStream_t s) {
    switch (g.epilogue) {
        case kEpiSilu: hipLaunchKernelGGL((gemm_kernel<AT, BT, kEpiSilu>), grid, dim3(kGT), 0, s, g); break;
        case kEpiResidual: hipLaunchKernelGGL((gemm_kernel<AT, BT, kEpiResidual>), grid, dim3(kGT), 0, s, g); break;
        case kEpiStoreF32: hipLaunchKernelGGL((gemm_kernel<AT, BT, kEpiStoreF32>), grid, dim3(kGT), 0, s, g); break;
        case kEpiAtomicF32: hipLaunchKernelGGL((gemm_kernel<AT, BT, kEpiAtomicF32>), grid, dim3(kGT), 0, s, g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
    if (g.M <= 0 || g.K <= 0) return hipSuccess;
    if (!g.a || !g.b || !g.c || g.N <= 0 || g.N % kGN != 0) return hipErrorInvalidValue;
    if (g.epilogue == kEpiResidual && !g.r) return hipErrorInvalidValue;
    // operands read along K (row form) need whole 64-wide K steps and no K split
    const bool k_ragged_ok = g.at && !g.bt;
    int64_t kchunk = g.kchunk <= 0 ? g.K : g.kchunk;
    if (!k_ragged_ok && (g.K % kGK != 0 || kchunk < g.K)) return hipErrorInvalidValue;
    if (kchunk % kGK != 0 && kchunk < g.K) return hipErrorInvalidValue;
    if (g.at && g.M % kGM != 0) return hipErrorInvalidValue;
    if (kchunk < g.K && g.epilogue != kEpiAtomicF32) return hipErrorInvalidValue;
    // 32-bit buffer offsets: a K-major operand spans kchunk rows, a row-form operand 128 rows
    const int64_t kspan_a = g.at ? kchunk * g.lda : kGM * g.lda + g.K;
    const int64_t kspan_b = g.bt ? kGN * g.ldb + g.K : kchunk * g.ldb;
    if ((kspan_a + kGK * g.lda) * 2 >= (int64_t(1) << 31) ||
        (kspan_b + kGK * g.ldb) * 2 >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    const int64_t splits = (g.K + kchunk - 1) / kchunk;
    if (splits > 65535) return hipErrorInvalidValue;
    GemmArgs a = g;
    a.kchunk = kchunk;
    a.mtiles = (int32_t)((g.M + kGM - 1) / kGM);
    a.ntiles = g.N / kGN;
    a.splits = (int32_t)splits;
    const int64_t groups = (int64_t)a.mtiles * a.splits;
    const int64_t numbers = (groups + kXcds - 1) / kXcds * kXcds * a.ntiles;  // tile numbers
    if (numbers >= (int64_t(1) << 31)) return hipErrorInvalidValue;
    // persistent grid: two workgroups per compute unit (a multiple of 8), each taking every
    // grid-th tile number
    const int64_t slots = 2 * (int64_t)(g.compute_units > 0 ? g.compute_units : 256);
    const int64_t gsize = std::min<int64_t>((numbers + kXcds - 1) / kXcds * kXcds,
                                            (slots + kXcds - 1) / kXcds * kXcds);
    a.rounds = (int32_t)((numbers + gsize - 1) / gsize);
    dim3 grid((unsigned)gsize);
    if (!g.at && !g.bt) return launch_t<false, false>(a, grid, s);
    if (!g.at && g.bt) return launch_t<false, true>(a, grid, s);
    if (g.at && !g.bt) return launch_t<true, false>(a, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace hstu
