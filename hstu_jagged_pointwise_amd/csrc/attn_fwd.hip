// attn_fwd.hip -- HSTU pointwise attention forward on gfx950.
//
// O_i = sum_j vis(i, j) * SiLU(alpha * q_i.k_j + rab_pos[h, bucket(|i-j|)]
//                                + rab_ts[h, bucket(|t_i-t_j|)]) / N * v_j
// (page 1 section 2.1.2, HSTU spatial aggregation, equation (2); no softmax).
//
// bf16 path.  A work unit is (sequence, head, 128 query rows); each of the 4 wavefronts owns 32
// rows.  Key tiles of 64 keys are visited in the order given by key_tiles_for_rows(): tiles that
// the composite causal/context/candidate mask leaves empty for the whole unit are never loaded,
// and a wavefront skips the arithmetic of tiles that are empty for its own rows (page 2, HSTU
// acceleration operator: composite-mask skipping).  K and V tiles are copied from memory straight
// into LDS by buffer loads (rows past the sequence end read as zero), into two LDS buffers, so
// the copy of tile t+1 runs while tile t is computed (page 2: move one block while computing
// another).
//
// Per tile and wavefront:
//   S^T (64 keys x 32 rows) = K . Q^T        2 x (D/16) v_mfma_f32_32x32x16_bf16
//   P = SiLU(alpha S + bias), masked          fp32 in registers
//   O^T (D x 32 rows) += V^T . P^T           (D/32) x 4 v_mfma_f32_32x32x16_bf16
// The C layout of S^T gives each lane one query row and 16 keys per 32-key block, which is the
// B-operand layout P^T needs; the matching V^T operand is read from the row-major V tile with
// transposing LDS reads, so P never leaves registers.  Scores are carried as -log2(e) * S (folded
// into alpha and the staged bias tables), so SiLU costs one fma, exp2, add, rcp and mul; the
// remaining factor -ln(2) / N is applied once to O.  Whenever every pair of a (wavefront, tile)
// falls into one position bucket (or one time bucket), that bias is a single scalar for the tile
// and the per-element bias work disappears -- the common case away from the diagonal.
#include "device_common.h"
#include "kernels.h"

namespace hstu {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4 * kWaveRows;  // 128 query rows per unit
constexpr int kBN = kKeyTile;         // 64 keys per tile
constexpr int kToep = kRows + kBN - 1;  // 191 distinct i - j per (unit, tile)

// Time bias by the bit pattern of a float distance.  For an integer distance 1 <= x < 2^24 the
// float's exponent and first three fraction bits, (bits >> 20) = 8 * (127 + e) + m3, name a
// class of width 2^(e-3) that lies inside one bucket (the bucket rule is exact on quarter octaves
// and the identity below 16), so ((bits >> 18) & 0x1ffc) is a byte offset into a table of
// kFloatClasses entries that starts kFloatClassBase bytes after the bucket table's entry for
// distance 0 -- which is where the pattern of +-0.0 points.  Four instructions from two 32-bit
// times to a table address (subtract, convert, shift, mask; the sign bit is masked off),
// against eight for |difference| and the integer class (bucket_class).
constexpr int kFloatClasses = 192;               // exponents 0 .. 23
constexpr int kFloatClassBase = (127 * 8) * 4;   // byte offset of the class of 1.0f
constexpr int64_t kFloatExact = 1 << 24;         // time differences below this: exact floats

template <int D>
struct FwdSmem {
    // Small tables first, so their offsets fit the 16-bit LDS instruction offset field (the
    // Toeplitz table at offset 0, so its per-element reads need no address arithmetic).  Bias
    // values are stored multiplied by -log2(e) (see silu_scaled).
    float rp[2][kToep + 1];             // position bias by (i - j) for the tile
    float wp[kNumBuckets];              // position bias by bucket
    float wtb[kNumBuckets];             // time bias by bucket
    float wt[kNumClasses];              // time bias by bucket class
    uint32_t tk[2][kBN];                // key timestamps, biased 32-bit relative
    int64_t tk64[2][kBN];               // key timestamps (fallback)
    int64_t tkmin[2], tkmax[2];         // time range of the tile's real keys
    int fits[2];
    char pad_[kFloatClassBase - sizeof(float) * (kNumBuckets + kNumClasses) -
              sizeof(uint32_t) * 2 * kBN - sizeof(int64_t) * (2 * kBN + 4) - sizeof(int) * 2];
    float wtf[kFloatClasses];           // time bias by float class (see kFloatClassBase)
    alignas(16) bf16 k[2][kBN * D];     // swizzled tiles (tile_off)
    bf16 v[2][kBN * D];
};

// Time bias of the distance between two biased 32-bit relative times whose difference is below
// 2^24 in magnitude (see kFloatClassBase): the byte offset from the bucket table, then the
// lookup.
__device__ __forceinline__ uint32_t float_class_offset(uint32_t ti, uint32_t tk) {
    return (__float_as_uint((float)(int32_t)(ti - tk)) >> 18) & 0x1ffcu;
}
template <int D>
__device__ __forceinline__ float float_class_at(const FwdSmem<D>& sm, uint32_t off) {
    return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(sm.wtb) + off);
}

// Bias handling of one (wavefront, tile), decided once per tile from the distance ranges:
//   PM 0: position bias absent or one bucket (inside b0/b1); 1: Toeplitz table per element.
//   TM 0: time bias absent or one bucket (inside tb.b0); 1: two buckets, tb.b1 where
//      |dt| >= thr; 4: three buckets (tb.b2 where |dt| >= thr2); 2: per-element bucket class,
//      32-bit relative times; 3: the same with 64-bit times; 5: per-element float class
//      (float_class_offset) when every time difference of the tile is below 2^24.
// In the per-element time modes tb.b0 is the position bucket's bias, zero when PM is 1.
// s[x] holds the 32-key block kb0 + x of the tile (x < NKB); on return, the scores
// t = -log2(e) (alpha q.k + bias) that silu_scaled takes.
template <int D, int PM, int TM, int NKB>
__device__ __forceinline__ void epilogue(f32x16 (&s)[NKB], const FwdSmem<D>& sm, int buf, int u0,
                                         int g, float alpha2, const TimeSel tb, uint32_t ti,
                                         int64_t ti64, int kb0) {
    const TimePick pick(tb, ti);
    constexpr bool kPerElem = TM == 2 || TM == 3 || TM == 5;
    if constexpr (TM == 5) {
        // per 32-key block: the 16 table addresses, then all 16 lookups (with the Toeplitz
        // reads), then the sums -- so the lookups are in flight together
#pragma unroll
        for (int x = 0; x < NKB; ++x) {
            const int kb = kb0 + x;
            uint32_t a[16];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const u32x4 tq = *reinterpret_cast<const u32x4*>(&sm.tk[buf][32 * kb + 8 * r + 4 * g]);
#pragma unroll
                for (int c = 0; c < 4; ++c) a[4 * r + c] = float_class_offset(ti, tq[c]);
            }
            __builtin_amdgcn_sched_barrier(0);
            float bt[16], bp[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                bt[e] = float_class_at(sm, a[e]);
                if (PM == 1) bp[e] = sm.rp[buf][u0 + 32 * kb + 8 * (e >> 2) + (e & 3)];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                s[x][e] = fmaf(alpha2, s[x][e], (PM == 1 ? bp[e] : tb.b0) + bt[e]);
        }
        return;
    }
#pragma unroll
    for (int x = 0; x < NKB; ++x) {
        const int kb = kb0 + x;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jj = 32 * kb + 8 * r + 4 * g;  // first of this lane's 4 keys
            u32x4 tq;
            if (TM == 1 || TM == 2 || TM == 4) tq = *reinterpret_cast<const u32x4*>(&sm.tk[buf][jj]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int e = 4 * r + c;
                float bt;  // time part
                if (TM == 2) bt = sm.wt[bucket_class(absdiff_sad(ti, tq[c]))];
                else if (TM == 3) bt = sm.wt[bucket_class(absdiff_sat(ti64, sm.tk64[buf][jj + c]))];
                else bt = pick.get<TM>(tq[c]);
                float b;
                if (PM == 1) b = sm.rp[buf][u0 + 32 * kb + 8 * r + c] + bt;
                else b = kPerElem ? tb.b0 + bt : bt;
                s[x][e] = fmaf(alpha2, s[x][e], b);
            }
        }
    }
}

template <int D, int PM, int NKB>
__device__ __forceinline__ void epilogue_tm(int tm, f32x16 (&s)[NKB], const FwdSmem<D>& sm, int buf,
                                            int u0, int g, float alpha2, const TimeSel tb,
                                            uint32_t ti, int64_t ti64, int kb0) {
    switch (tm) {
        case 0: epilogue<D, PM, 0, NKB>(s, sm, buf, u0, g, alpha2, tb, ti, ti64, kb0); break;
        case 1: epilogue<D, PM, 1, NKB>(s, sm, buf, u0, g, alpha2, tb, ti, ti64, kb0); break;
        case 4: epilogue<D, PM, 4, NKB>(s, sm, buf, u0, g, alpha2, tb, ti, ti64, kb0); break;
        case 5: epilogue<D, PM, 5, NKB>(s, sm, buf, u0, g, alpha2, tb, ti, ti64, kb0); break;
        case 2: epilogue<D, PM, 2, NKB>(s, sm, buf, u0, g, alpha2, tb, ti, ti64, kb0); break;
        default: epilogue<D, PM, 3, NKB>(s, sm, buf, u0, g, alpha2, tb, ti, ti64, kb0); break;
    }
}

// Zero the entries of keys this lane's row does not see (partial tiles only); s[x] holds the
// 32-key block kb0 + x of the tile.
template <int NKB>
__device__ __forceinline__ void mask_keys(f32x16 (&s)[NKB], int g, int j0, int lim, int dg, int kb0) {
#pragma unroll
    for (int x = 0; x < NKB; ++x)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int j = j0 + 32 * (kb0 + x) + 8 * (e >> 2) + 4 * g + (e & 3);
            s[x][e] = (j <= lim || j == dg) ? s[x][e] : 0.0f;
        }
}

// CACHED: candidate scoring.  The item's rows are candidates (positions nk + i, where nk is the
// user's cached history length) and its key tiles run over the cache; every cached key is
// visible (rows past the cache end read as zero, and zero V rows add nothing), and each row's
// own key is added after the tiles by the item that holds the first tile.
// KH: items of 64 rows, and the 4 wavefronts are 2 row groups x 2 key halves (wavefront w: rows
// 32 (w % 2) .. + 31 of the item, keys 32 (w / 2) .. + 31 of each tile): half the work per
// wavefront and tile for candidate lists and small batches, where the items do not fill the
// GPU; the key halves' partial outputs are added through LDS.  Otherwise items of 128 rows, 4
// row groups of 32 over whole tiles.
template <int D, bool RP, bool RT, bool CACHED, bool KH>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(const AttnParams p) {
    __shared__ __attribute__((aligned(16))) FwdSmem<D> sm;
    static_assert(offsetof(FwdSmem<D>, wtf) == offsetof(FwdSmem<D>, wtb) + kFloatClassBase,
                  "float-class table placement");

    constexpr int kItemRows = KH ? 2 * kWaveRows : kRows;
    constexpr int NKB = KH ? 1 : 2;                  // 32-key blocks per wavefront and tile
    const FwdItem wu = p.items[blockIdx.x];
    const int tid = threadIdx.x, wave = uniform_i(tid >> 6), lane = tid & 63, g = lane >> 5,
              lr = lane & 31;
    const int rg = KH ? (wave & 1) : wave, kh = KH ? (wave >> 1) : 0;  // row group, key half
    const int n = wu.n, nc = wu.nc, nh = wu.nh, r0 = wu.row0, h = wu.head;
    const int64_t tok0 = wu.start;
    const bf16* __restrict__ qg = static_cast<const bf16*>(p.q) + tok0 * p.ld_in + h * D;
    const CacheSeq cs = CACHED ? CacheSeq{wu.cstart, wu.cn} : CacheSeq{0, 0};
    const int64_t ktok0 = CACHED ? cs.start : tok0;
    const int64_t ld = CACHED ? p.ld_cache : p.ld_in;  // key / value token stride
    const bf16* __restrict__ kg = static_cast<const bf16*>(CACHED ? p.kc : p.k) + ktok0 * ld + h * D;
    const bf16* __restrict__ vg = static_cast<const bf16*>(CACHED ? p.vc : p.v) + ktok0 * ld + h * D;
    const int nk = CACHED ? cs.n : n;     // keys
    const int rpos0 = CACHED ? cs.n : 0;  // position of row 0
    const int64_t* __restrict__ tsk = (CACHED ? p.ts_cache : p.ts) + ktok0;

    const int64_t tbase = RT ? (nk > 0 ? tsk[0] : p.ts[tok0]) : 0;
    const int rhi = imin(r0 + kItemRows, n);
    const KeyTiles kl = key_tiles_for_rows(r0, rhi, nc, nh);
    const int tbeg = wu.t0, ntiles = wu.t1 - wu.t0;  // this item's part of the tile list
    auto tile_at = [&](int t) { return CACHED ? tbeg + t : kl.tile(tbeg + t); };

    // The tile copies are issued from inline assembly (TileDma::issue_asm): with the builtin the
    // compiler would wait for the next tile's copy before every LDS read of the current tile.
    // Each iteration waits for its copy explicitly (wait_tile_dma, then the barrier).
    const i32x4 krs = rows_words(kg, nk, ld, D), vrs = rows_words(vg, nk, ld, D);
    const TileDma<D, kThreads> dma(tid, ld);
    const RowOperand<D> kop(lane);
    const TrOperand<D> vop(lane);
    int64_t tkr = 0;

    // loads a tile's timestamps and starts the copy of its K and V rows into buffer buf (the
    // timestamp load goes first: the compiler's wait for its register then finds no copy in
    // flight)
    auto load_tile = [&](int buf, int tile) {
        const int j0 = tile * kBN;
        const int row_bytes = (int)((int64_t)j0 * ld * 2);
        if (RT && tid < kBN) {  // keys past the end take the last key's time (within the tile's range)
            const int j = j0 + tid;
            tkr = tsk[j < nk ? j : nk - 1];
        }
        dma.issue_asm(krs, sm.k[buf], row_bytes);
        dma.issue_asm(vrs, sm.v[buf], row_bytes);
    };

    // the tile's small tables: key times and their range, position bias by (i - j)
    auto store_tile = [&](int buf, int tile) {
        const int j0 = tile * kBN;
        if (RT && tid < kBN) {  // exactly wavefront 0
            const bool real = j0 + tid < nk;
            sm.tk64[buf][tid] = tkr;
            sm.tk[buf][tid] = rel_time_u32(tkr, tbase);
            const TimeRange tr = wave_time_range(tkr, real, tbase);
            if (tid == 0) {
                sm.fits[buf] = tr.fit ? 1 : 0;
                sm.tkmin[buf] = tr.lo[0] < tr.lo[1] ? tr.lo[0] : tr.lo[1];
                sm.tkmax[buf] = tr.hi[0] > tr.hi[1] ? tr.hi[0] : tr.hi[1];
            }
        }
        if (RP)
            for (int u = tid; u < kToep; u += kThreads) {
                const int delta = (r0 + rpos0 - j0) + (kRows - 1) - u;  // i - j for table slot u
                sm.rp[buf][u] = sm.wp[bucket_of((uint32_t)(delta < 0 ? -delta : delta))];
            }
    };

    // the first tile's copy runs while the bias tables, Q and the row times load
    if (ntiles > 0) load_tile(0, tile_at(0));

    if (RP)
        for (int e = tid; e < kNumBuckets; e += kThreads)
            sm.wp[e] = -kLog2e * p.rab_pos[h * kNumBuckets + e];
    if (RT) {
        for (int e = tid; e < kNumClasses; e += kThreads)
            sm.wt[e] = -kLog2e * p.rab_ts[h * kNumBuckets + bucket_of_class(e)];
        for (int e = tid; e < kNumBuckets; e += kThreads)
            sm.wtb[e] = -kLog2e * p.rab_ts[h * kNumBuckets + e];
        for (int e = tid; e < kFloatClasses; e += kThreads)  // a member of float class e
            sm.wtf[e] = -kLog2e * p.rab_ts[h * kNumBuckets + bucket_of(((8u + (e & 7)) << (e >> 3)) >> 3)];
    }

    // this wavefront's rows and this lane's row
    const int wlo = r0 + kWaveRows * rg, whi = imin(wlo + kWaveRows, rhi);
    const int i = wlo + lr;
    const bool row_ok = i < rhi;
    int lim = -1, dg = -1;  // visible keys: j <= lim or j == dg
    if (row_ok && !CACHED) {
        if (i < nh) lim = imax(i, nc - 1);
        else { lim = nh - 1; dg = i; }
    }

    bf16x8 qf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        if (row_ok) qf[ks] = load_bf16x8(qg + (int64_t)i * ld + 16 * ks + 8 * g);
        else qf[ks] = bf16x8{};
    }
    uint32_t ti = 0, timax_rel = 0;
    int64_t ti64 = 0, timin = 0, timax = 0;
    bool wave_qfit = true;
    if (RT) {
        ti64 = row_ok ? p.ts[tok0 + i] : tbase;
        wave_qfit = __all(rel_time_fits(ti64, tbase));
        ti = rel_time_u32(ti64, tbase);
        {
            int64_t lo, hi;
            wave_time_minmax(ti64, row_ok, tbase, lo, hi);
            timin = uniform64(lo);
            timax = uniform64(hi);
        }
        timax_rel = rel_time_u32(timax, tbase);  // used only when every row time fits
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};

    __syncthreads();  // bias tables ready
    if (ntiles > 0) store_tile(0, tile_at(0));
    wait_tile_dma();
    __syncthreads();

    // slot of (row i, key j0 + jj) in rp is u0 + jj - 4g; see store_tile
    const int u0 = 4 * g - (kWaveRows * rg + lr) + (kRows - 1);
    const float alpha2 = -kLog2e * p.alpha;

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1, j0 = tile_at(t) * kBN;
        if (t + 1 < ntiles) load_tile(buf ^ 1, tile_at(t + 1));
        // this wavefront's keys of the tile: [jw, jw + 32 NKB)
        const int jw = j0 + kWaveRows * kh;
        const int kind = wlo >= rhi || jw >= nk ? kEmpty
                         : CACHED ? kFull : classify_row_tile(wlo, whi, jw, n, nc, nh, kWaveRows * NKB);
        if (kind != kEmpty) {
            f32x16 s[NKB];
#pragma unroll
            for (int x = 0; x < NKB; ++x) s[x] = f32x16{};
#pragma unroll
            for (int y = 0; y < NKB * (D / 16); ++y) {
                const int ks = y / NKB, x = y % NKB;
                s[x] = mfma32(kop.read(sm.k[buf], kh + x, ks), qf[ks], s[x]);
            }
            sched_mfma_lds<NKB * (D / 16), 2 * NKB>();
            // bias mode of this (wavefront, tile): one bucket for the whole tile when possible
            float bpos = 0.0f;
            int pm = 0;
            if (RP) {
                const int jhi = imin(jw + kWaveRows * NKB, nk) - 1;
                const BiasSpan sp = bias_span((int64_t)wlo + rpos0 - jhi, (int64_t)(whi - 1 + rpos0) - jw);
                if (sp.kind == 0) bpos = sm.wp[sp.b_lo];
                else pm = 1;
            }
            TimeSel tb;
            int tm = 0;
            if (RT) {
                const int64_t dlo = timin - uniform64(sm.tkmax[buf]);
                const BiasSpan st = bias_span(dlo, timax - uniform64(sm.tkmin[buf]));
                tm = tb.set(st, wave_qfit && uniform_i(sm.fits[buf]), bpos, sm.wtb, dlo >= 0, timax_rel);
                // every |t_i - t_j| of the tile below 2^24: exact as a float
                if (tm == 2 && dlo > -kFloatExact && timax - uniform64(sm.tkmin[buf]) < kFloatExact) tm = 5;
            } else tb.set_const(bpos);
            if (pm) epilogue_tm<D, 1, NKB>(tm, s, sm, buf, u0, g, alpha2, tb, ti, ti64, kh);
            else epilogue_tm<D, 0, NKB>(tm, s, sm, buf, u0, g, alpha2, tb, ti, ti64, kh);
            // the mode branches only form the scores; the SiLU is common code after them
#pragma unroll
            for (int x = 0; x < NKB; ++x)
#pragma unroll
                for (int e = 0; e < 16; ++e) s[x][e] = silu_scaled(s[x][e]);
            if (kind == kPartial) mask_keys<NKB>(s, g, j0, lim, dg, kh);
#pragma unroll
            for (int st = 0; st < 2 * NKB; ++st) {
                float tmp[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) tmp[x] = s[st >> 1][8 * (st & 1) + x];
                const bf16x8 pb = pack8(tmp);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) o[db] = mfma32(vop.read(sm.v[buf], 2 * kh + st, db), pb, o[db]);
            }
        }
        if (t + 1 < ntiles) store_tile(buf ^ 1, tile_at(t + 1));
        wait_tile_dma();
        __syncthreads();
    }

    if (CACHED && row_ok && wu.t0 == 0 && kh == 0) {  // the row's own key and value
        const bf16* kr = static_cast<const bf16*>(p.k) + (tok0 + i) * p.ld_in + h * D;
        const bf16* vr = static_cast<const bf16*>(p.v) + (tok0 + i) * p.ld_in + h * D;
        float dot = 0.0f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const bf16x8 kv = load_bf16x8(kr + 16 * ks + 8 * g);
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf((float)qf[ks][e], (float)kv[e], dot);
        }
        dot += __shfl_xor(dot, 32);
        float b = 0.0f;  // distance 0 in position and time: bucket 0
        if (RP) b += sm.wp[0];
        if (RT) b += sm.wtb[0];
        const float pw = silu_scaled(fmaf(alpha2, dot, b));
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bf16x4 vv = *reinterpret_cast<const bf16x4*>(vr + 32 * db + 8 * r + 4 * g);
#pragma unroll
                for (int c = 0; c < 4; ++c) o[db][4 * r + c] = fmaf(pw, (float)vv[c], o[db][4 * r + c]);
            }
    }

    if constexpr (KH) {
        // the second key half's partial outputs into the first's, through the (then idle) K
        // tiles laid out [row group][db][element][lane]
        static_assert(sizeof(sm.k) >= 2 * (D / 32) * 16 * 64 * sizeof(float), "reduction buffer");
        float* mine = reinterpret_cast<float*>(&sm.k[0][0]) + (size_t)rg * (D / 32) * 16 * 64 + lane;
        if (kh == 1)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) mine[(db * 16 + e) * 64] = o[db][e];
        __syncthreads();
        if (kh == 0)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) o[db][e] += mine[(db * 16 + e) * 64];
        if (kh != 0) return;
    }
    if (row_ok && wu.part >= 0) {  // one piece of a split row block: fp32 partial sums
        float* pg = p.part + ((size_t)wu.part * kItemRows + (i - r0)) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<f32x4*>(pg + 32 * db + 8 * r + 4 * g) =
                    f32x4{o[db][4 * r], o[db][4 * r + 1], o[db][4 * r + 2], o[db][4 * r + 3]};
    } else if (wu.part < 0) {
        // this wavefront's 32 rows go through LDS (the idle V tiles, swizzled like a tile) so
        // that each store instruction writes whole row segments
        bf16* stage = sm.v[0] + (size_t)rg * kWaveRows * D;
        const float oscale = -kLn2 * p.inv_n;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bf16x4 w;
#pragma unroll
                for (int c = 0; c < 4; ++c) w[c] = (bf16)(o[db][4 * r + c] * oscale);
                *reinterpret_cast<bf16x4*>(stage + tile_off<D>(lr, 32 * db + 8 * r + 4 * g)) = w;
            }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        constexpr int kChunks = D / 8, kRowsPer = 64 / kChunks;  // 16-byte chunks per row
#pragma unroll
        for (int it = 0; it < kWaveRows / kRowsPer; ++it) {
            const int row = kRowsPer * it + lane / kChunks, ch = lane % kChunks;
            if (wlo + row < rhi) {
                const bf16x8 v = *reinterpret_cast<const bf16x8*>(stage + tile_off<D>(row, 8 * ch));
                *reinterpret_cast<bf16x8*>(static_cast<bf16*>(p.out) + (tok0 + wlo + row) * p.ld_out +
                                           h * D + 8 * ch) = v;
            }
        }
    }
}

// ---- fp32 path: one thread per query row, keys streamed through the cache --------------------

constexpr int kF32Rows = 64;

template <int D>
__global__ __launch_bounds__(kF32Rows) void fwd_f32_kernel(const AttnParams p) {
    __shared__ float wp[kNumBuckets];
    __shared__ float wt[kNumClasses];
    const WorkUnit wu = p.units[blockIdx.x];
    const SeqInfo si = p.seqs[wu.seq];
    const int n = si.n, nc = si.nc, nh = si.nh, h = wu.head;
    const int64_t tok0 = si.start, ld = p.ld_in;
    const int i = wu.row0 + threadIdx.x;
    const bool row_ok = i < n;
    const bool has_rp = p.rab_pos != nullptr, has_rt = p.rab_ts != nullptr;
    if (has_rp)
        for (int e = threadIdx.x; e < kNumBuckets; e += kF32Rows) wp[e] = p.rab_pos[h * kNumBuckets + e];
    if (has_rt)
        for (int e = threadIdx.x; e < kNumClasses; e += kF32Rows)
            wt[e] = p.rab_ts[h * kNumBuckets + bucket_of_class(e)];
    __syncthreads();

    int lim = -1, dg = -1;
    if (row_ok) {
        if (i < nh) lim = imax(i, nc - 1);
        else { lim = nh - 1; dg = i; }
    }
    const float* qg = static_cast<const float*>(p.q) + tok0 * ld + h * D;
    const float* kg = static_cast<const float*>(p.k) + tok0 * ld + h * D;
    const float* vg = static_cast<const float*>(p.v) + tok0 * ld + h * D;
    float q[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        q[c] = row_ok ? qg[(int64_t)i * ld + c] : 0.0f;
        acc[c] = 0.0f;
    }
    const int64_t ti = (has_rt && row_ok) ? p.ts[tok0 + i] : 0;
    const int jend = __reduce_max_sync(~0ull, imax(lim, dg)) + 1;  // keys any lane sees
    for (int j = 0; j < jend; ++j) {
        const bool vis = j <= lim || j == dg;
        if (!__any(vis)) continue;
        float dot = 0.0f;
#pragma unroll
        for (int c = 0; c < D; ++c) dot = fmaf(q[c], kg[(int64_t)j * ld + c], dot);
        float bias = 0.0f;
        if (has_rp) bias += wp[bucket_of((uint32_t)(i > j ? i - j : j - i))];
        if (has_rt && row_ok) bias += wt[bucket_class(absdiff_sat(ti, p.ts[tok0 + j]))];
        const float x = fmaf(p.alpha, dot, bias);
        const float w = vis ? x / (1.0f + expf(-x)) : 0.0f;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(w, vg[(int64_t)j * ld + c], acc[c]);
    }
    if (row_ok) {
        float* og = static_cast<float*>(p.out) + (tok0 + i) * p.ld_out + h * D;
#pragma unroll
        for (int c = 0; c < D; ++c) og[c] = acc[c] * p.inv_n;
    }
}

// Sums the partial slots of each split row block of ROWS rows and writes its output rows (scaled
// like the unsplit rows).  Workgroup (x, y) takes rows [y * kFixRows, + kFixRows) of split block
// x; each thread owns 4 columns of one row.
constexpr int kFixRows = 4 * kThreads / 128;
template <int D, int ROWS>
__global__ __launch_bounds__(kThreads) void fwd_fix_kernel(const AttnParams p) {
    constexpr int RPT = kThreads / (D / 4);  // rows per pass of the workgroup
    const FixItem f = p.fix[blockIdx.x];
    const SeqInfo si = p.seqs[f.seq];
    const int rows = imin(ROWS, si.n - f.row0);
    const float oscale = -kLn2 * p.inv_n;
    const int c = 4 * (threadIdx.x % (D / 4));
#pragma unroll
    for (int pass = 0; pass < kFixRows / RPT + (kFixRows % RPT != 0); ++pass) {
        const int r = blockIdx.y * kFixRows + pass * RPT + threadIdx.x / (D / 4);
        if (r >= rows || r >= (int)(blockIdx.y + 1) * kFixRows) continue;
        f32x4 acc = f32x4{};
        for (int k = 0; k < f.nparts; ++k)
            acc += *reinterpret_cast<const f32x4*>(p.part + ((size_t)(f.part0 + k) * ROWS + r) * D + c);
        bf16x4 w;
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = (bf16)(acc[x] * oscale);
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(p.out) + (si.start + f.row0 + r) * p.ld_out +
                                   f.head * D + c) = w;
    }
}

template <int D, bool RP, bool RT>
hipError_t launch_bf16_t(const AttnParams& p, hipStream_t s) {
    const bool kh = p.item_rows == 2 * kWaveRows;  // else kRows (checked by the caller)
    const dim3 grid(p.num_items), block(kThreads);
    if (p.cache)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, RP, RT, true, true>), grid, block, 0, s, p);
    else if (kh)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, RP, RT, false, true>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, RP, RT, false, false>), grid, block, 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.num_fix == 0) return e;
    if (kh)
        hipLaunchKernelGGL((fwd_fix_kernel<D, 2 * kWaveRows>), dim3(p.num_fix, 2 * kWaveRows / kFixRows), block, 0, s, p);
    else
        hipLaunchKernelGGL((fwd_fix_kernel<D, kRows>), dim3(p.num_fix, kRows / kFixRows), block, 0, s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_d(const AttnParams& p, hipStream_t s) {
    const bool rp = p.rab_pos != nullptr, rt = p.rab_ts != nullptr;
    if (rp && rt) return launch_bf16_t<D, true, true>(p, s);
    if (rp) return launch_bf16_t<D, true, false>(p, s);
    if (rt) return launch_bf16_t<D, false, true>(p, s);
    return launch_bf16_t<D, false, false>(p, s);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnParams& p, hipStream_t s) {
    if (p.num_items == 0) return hipSuccess;
    if (p.num_fix > 0 && p.part == nullptr) return hipErrorInvalidValue;
    if (p.item_rows != kRows && p.item_rows != 2 * kWaveRows) return hipErrorInvalidValue;
    if (p.cache && p.item_rows != 2 * kWaveRows) return hipErrorInvalidValue;
    switch (p.head_dim) {
        case 32: return launch_bf16_d<32>(p, s);
        case 64: return launch_bf16_d<64>(p, s);
        case 128: return launch_bf16_d<128>(p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_f32(const AttnParams& p, hipStream_t s) {
    if (p.num_units == 0) return hipSuccess;
    switch (p.head_dim) {
        case 32: hipLaunchKernelGGL(fwd_f32_kernel<32>, dim3(p.num_units), dim3(kF32Rows), 0, s, p); break;
        case 64: hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(p.num_units), dim3(kF32Rows), 0, s, p); break;
        case 128: hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(p.num_units), dim3(kF32Rows), 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hstu
