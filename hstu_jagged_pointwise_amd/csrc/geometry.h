// geometry.h -- which (row block, key tile) pairs of a jagged sequence hold visible pairs.
//
// Shared by the host planner (work costs) and the kernels (iteration ranges), so both agree.
// The composite mask follows page 2 ("RecSDK supports generative recommendation", HSTU
// acceleration operator: causal + context/target masks, with whole blocks skipped) and page 1
// section 2.1.2 (ranking: candidates at the end see the history and themselves only):
//   nc = min(num_contexts, n), nt = min(num_targets, n - nc), nh = n - nt
//   row i < nh (history) sees keys j <= max(i, nc - 1);  row i >= nh (candidate) sees j < nh
//   and j == i.
// Every key tile is BN = 64 keys wide and aligned to multiples of 64 within the sequence.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define HSTU_HD __host__ __device__ __forceinline__
#else
#define HSTU_HD inline
#endif

namespace hstu {

constexpr int kNumBuckets = 128;
constexpr int kKeyTile = 64;     // keys per tile in the forward / dQ kernels
constexpr int kQueryTile = 64;   // queries per tile in the dK/dV kernel
constexpr int kWaveRows = 32;    // rows (or keys) owned by one wavefront

struct SeqInfo {
    int32_t start;  // first token of the sequence in the packed token dimension
    int32_t n;      // length
    int32_t nc;     // effective number of context tokens
    int32_t nh;     // effective number of non-candidate tokens (n - candidates)
};

// Cached history of one user for candidate scoring: rows [start, start + n) of the cache.
struct CacheSeq {
    int32_t start;
    int32_t n;
};

struct WorkUnit {
    int32_t seq, head, row0, cost;
};

// A forward work item: key tiles [t0, t1) of the list key_tiles_for_rows() gives for one row
// block.  part < 0: the item covers the whole list and writes the output rows itself; otherwise
// it writes its fp32 partial sums to partial slot `part`, and a FixItem adds the slots up.  The
// item carries its sequence's SeqInfo (and the cached history's CacheSeq for candidate scoring)
// so that a workgroup needs one 64-byte load, not two dependent ones, before it can start.
struct FwdItem {
    int32_t seq, head, row0, cost, t0, t1, part, pad0;
    int32_t start, n, nc, nh;  // SeqInfo of seq
    int32_t cstart, cn;        // CacheSeq of seq (candidate scoring)
    int32_t pad1, pad2;
};
// A row block whose key tiles were split over items with slots [part0, part0 + nparts).
struct FixItem {
    int32_t seq, head, row0, part0, nparts, pad0, pad1, pad2;
};

HSTU_HD int imax(int a, int b) { return a > b ? a : b; }
HSTU_HD int imin(int a, int b) { return a < b ? a : b; }
HSTU_HD int cdiv(int a, int b) { return (a + b - 1) / b; }

HSTU_HD void split_sequence(int n, int num_contexts, int num_targets, int* nc, int* nh) {
    int c = imin(imax(num_contexts, 0), n);
    int t = imin(imax(num_targets, 0), n - c);
    *nc = c;
    *nh = n - t;
}

// Key tiles visible to query rows [rlo, rhi) (rhi <= n): tiles [0, main_tiles) followed by
// tiles [diag_first, diag_first + diag_tiles), the candidates' own diagonal.
struct KeyTiles {
    int main_tiles, diag_first, diag_tiles;
    HSTU_HD int count() const { return main_tiles + diag_tiles; }
    HSTU_HD int tile(int t) const { return t < main_tiles ? t : diag_first + (t - main_tiles); }
};

HSTU_HD KeyTiles key_tiles_for_rows(int rlo, int rhi, int nc, int nh) {
    KeyTiles r{0, 0, 0};
    if (rhi <= rlo) return r;
    int kmain = 0;
    if (rlo < nh) kmain = imax(imin(rhi, nh), nc);  // history rows: up to the last row, contexts
    if (rhi > nh) kmain = imax(kmain, nh);          // candidate rows: the whole history
    r.main_tiles = cdiv(kmain, kKeyTile);
    if (rhi > nh) {
        int first = imax(imax(rlo, nh) / kKeyTile, r.main_tiles);
        int last = cdiv(rhi, kKeyTile);
        r.diag_first = first;
        r.diag_tiles = imax(0, last - first);
    }
    return r;
}

// Classification of the block rows [rlo, rhi) x keys [j0, j0 + keys) (rhi <= n).
enum TileKind { kEmpty = 0, kPartial = 1, kFull = 2 };

HSTU_HD int classify_row_tile(int rlo, int rhi, int j0, int n, int nc, int nh,
                              int keys = kKeyTile) {
    if (rhi <= rlo) return kEmpty;
    int j1 = j0 + keys - 1;
    bool any = false;
    int hhi = imin(rhi, nh);
    if (rlo < hhi && j0 <= imax(hhi - 1, nc - 1)) any = true;          // history rows
    int tlo = imax(rlo, nh);
    if (tlo < rhi && (j0 < nh || (j0 < rhi && j1 >= tlo))) any = true;  // candidate rows
    if (!any) return kEmpty;
    if (j1 >= n) return kPartial;
    if (rhi <= nh && j1 <= imax(rlo, nc - 1)) return kFull;             // all history rows
    if (rlo >= nh && j1 < nh) return kFull;                             // all candidate rows
    return kPartial;
}

// Query rows that see keys [klo, khi) (khi <= n): one contiguous range [qlo, qhi).
HSTU_HD void rows_for_keys(int klo, int khi, int n, int nc, int nh, int* qlo, int* qhi) {
    if (khi <= klo) { *qlo = 0; *qhi = 0; return; }
    *qlo = klo < nc ? 0 : klo;
    *qhi = klo < nh ? n : imin(khi, n);
}

// Stored-dS layout of one sequence (bf16 backward).  Key block kb (keys [128 kb, 128 kb + 128))
// owns chunks of kDsChunk elements, one per 64-query tile from ds_first_qtile() on: chunk c holds
// dS of the block's 128 keys (rows) and queries [64 (q0 + c), + 64) (columns), q0 the first
// tile.  The chunks cover the 128-row-aligned range of the queries that see the block (the rows
// rows_for_keys() gives, rounded out to 128), so every 128-row block that visits one of the
// block's key tiles finds its two query tiles as two consecutive chunks.  A sequence's blocks
// are stored in order, each block's heads one after another: head h of block kb starts at
//   kDsChunk * (H * ds_chunks_before(kb) + h * ds_chunks(kb))
// elements from the sequence's start.
constexpr int kDsChunk = 128 * 64;

HSTU_HD int ds_first_qtile(int kb, int nc) { return 128 * kb < nc ? 0 : 2 * kb; }

// Chunks of key block kb (the sequence has nc contexts and nh non-candidates, nc <= nh).
HSTU_HD int ds_chunks(int kb, int n, int nc, int nh) {
    const int klo = 128 * kb;
    if (klo < nc) return 2 * cdiv(n, 128);               // every query sees a context key
    if (klo < nh) return 2 * cdiv(n, 128) - 2 * kb;      // history keys: queries from klo on
    return 2;                                            // candidates: only themselves
}

// Chunks of key blocks 0 .. kb - 1, in closed form: blocks below ceil(nc / 128) hold the whole
// query range, blocks below ceil(nh / 128) the range from their own first key, the rest 2.
HSTU_HD int64_t ds_chunks_before(int kb, int n, int nc, int nh) {
    const int64_t cn = 2 * cdiv(n, 128);
    const int64_t k1 = imin(kb, cdiv(nc, 128)), k2 = imin(kb, cdiv(nh, 128));
    const int64_t m2 = k2 - k1;                          // blocks k1 .. k2 - 1
    return k1 * cn + m2 * cn - m2 * (k1 + k2 - 1) + 2 * (int64_t)(kb - k2);
}

// Classification of the block queries [i0, i0 + rows) x keys [klo, khi) (khi <= n).
HSTU_HD int classify_key_tile(int klo, int khi, int i0, int n, int nc, int nh,
                              int rows = kQueryTile) {
    if (khi <= klo) return kEmpty;
    int i1 = i0 + rows - 1;
    bool any = false;
    if (klo < nc && i0 < n) any = true;                                  // context keys
    int hlo = imax(klo, nc), hhi = imin(khi, nh);
    if (hlo < hhi && i1 >= hlo && i0 < n) any = true;                    // history keys
    int tlo = imax(klo, nh);
    if (tlo < khi && i0 < khi && i1 >= tlo) any = true;                  // candidate keys
    if (!any) return kEmpty;
    if (i1 >= n) return kPartial;
    if (khi <= nc) return kFull;                                         // all context keys
    if (khi <= nh && i0 >= khi - 1) return kFull;                        // all history keys
    return kPartial;
}

}  // namespace hstu
