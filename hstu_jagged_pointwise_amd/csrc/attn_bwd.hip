// attn_bwd.hip -- HSTU pointwise attention backward on gfx950.
//
// With S = alpha q.k + bias, s = sigmoid(S), P = S s / N on visible pairs (page 1 section 2.1.2,
// equation (2)), and dO given:
//   dV_j = sum_i P_ij dO_i                 dP_ij = dO_i . v_j
//   dS_ij = dP_ij s (1 + S (1 - s)) / N    dQ_i = alpha sum_j dS_ij k_j
//   dK_j = alpha sum_i dS_ij q_i           d rab_pos[h, b] = sum over pairs with bucket b of dS
//   (and likewise d rab_ts over time buckets).
//
// Two passes, no atomics on dQ/dK/dV:
//   pass A (key-stationary): unit = (sequence, head, 128 keys), 8 wavefronts: wavefront w owns
//     keys 32 (w % 4) .. + 31 and the query half 32 (w / 4) .. + 31 of each visited 64-query tile
//     (two wavefronts per SIMD; the two halves' dK, dV partial sums are added through LDS at the
//     end).  The unit's K and V rows stay in LDS and are read as MFMA B operands, which keeps a
//     wavefront within the 256 registers that two wavefronts per SIMD allow.  S = Q K^T and
//     dP = dO V^T put one key per lane, which is the B-operand layout for dV^T += dO^T P and
//     dK^T += Q^T dS; the Q and dO tiles are read along their rows for the A operands of the
//     first two products and with transposing LDS reads for the last two.  With a workspace,
//     pass A also writes dS (bf16) for pass B and sums the bias-table gradients from it.
//   pass B (query-stationary): unit = (sequence, head, 128 rows) like the forward, 8 wavefronts:
//     wavefront w owns rows 32 (w % 4) .. + 31 and the key half 32 (w / 4) .. + 31 of each
//     64-key tile; S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T (K^T read transposed from the K
//     tile), and the bias-table gradients.  The unit's Q and dO rows stay in LDS (B operands),
//     two wavefronts per SIMD; the key halves' dQ partial sums are added through LDS at the end.
//     With the stored dS, pass B only reads dS and K (bwd_dq_stored_kernel).
// Tiles are copied from memory straight into LDS by buffer loads, double-buffered, as in the
// forward.
// Bias-gradient sums: when all pairs of a (wavefront, tile) fall into one bucket -- the common
// case away from the diagonal -- each lane only adds its dS values to a running sum, and the
// wavefront flushes that sum into an LDS histogram when the tile bucket changes; other tiles add
// each dS to an LDS histogram indexed by bucket class.  At the end of the unit each non-zero
// histogram entry goes to the global table with one atomic add.
// Scores are carried as -log2(e) S (folded into alpha and the staged bias tables), as in the
// forward, so sigmoid costs one exp2 and one rcp.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace hstu {
namespace {

constexpr int kThreads = 256;           // pass B
constexpr int kThreadsA = 512;          // pass A: 8 wavefronts
constexpr int kBlk = 4 * kWaveRows;      // 128 keys (pass A) or rows (pass B) per unit
constexpr int kTile = 64;                // queries (pass A) or keys (pass B) per tile
constexpr int kToep = kBlk + kTile - 1;  // 191 distinct i - j per (unit, tile)
constexpr int kReadAhead = 2;            // dK/dV pass: matrix instructions between a read and its use

struct ToepEntry {
    float bias;     // -log2(e) * position bias
    float bucket;   // bucket of |i - j|, as a float
};

// sigmoid(S) and dL/dS * N from t = -log2(e) S and dP:  P' = t s gives SiLU(S) = -ln(2) P', and
// dS N = dP (s + x s (1 - s)) with x s = -ln(2) P'.
struct Grad {
    float p, ds;
};
__device__ __forceinline__ Grad silu_grad(float t, float dp) {
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
    const float pv = t * sg;
    return Grad{pv, dp * fmaf(kLn2, fmaf(pv, sg, -pv), sg)};
}

// The layer backward's pre-activations for one lane's part of a gradient row (C layout of D / 32
// accumulators: columns 32 db + 8 r + 4 g + c), gate_delta bytes after each output element
// (AttnParams).  Loaded before the unit's final reduction, so their latency overlaps it.
template <int D>
struct GateRow {
    bf16x4 hv[D / 32][4];
    __device__ __forceinline__ void load(const bf16* row, int g, int64_t gate_delta) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                hv[db][r] = *reinterpret_cast<const bf16x4*>(
                    reinterpret_cast<const char*>(row + 32 * db + 8 * r + 4 * g) + gate_delta);
    }
};

// One lane's part of a gradient row leaving the backward: scaled, and in the layer backward
// (gate_delta != 0, gr loaded) multiplied by SiLU'(h).
template <int D>
__device__ __forceinline__ void store_grad_row(bf16* row, const f32x16 (&acc)[D / 32], int g,
                                               float scale, int64_t gate_delta,
                                               const GateRow<D>& gr) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bf16x4 w;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float x = acc[db][4 * r + c] * scale;
                w[c] = (bf16)(gate_delta != 0 ? x * silu_deriv((float)gr.hv[db][r][c]) : x);
            }
            *reinterpret_cast<bf16x4*>(row + 32 * db + 8 * r + 4 * g) = w;
        }
}



// ---------------------------------------------------------------------------------------------
// pass A: dK, dV
// ---------------------------------------------------------------------------------------------

// LDS operand reads by byte address.  In a 256-byte aligned tile (rows of 2D bytes, 16-byte
// chunks XOR-swizzled within a row), the chunk index occupies address bits 4 .. 3 + log2(D / 8):
// the row read at k-step ks is the ks = 0 address with bits 5.. flipped by ks, and the transposing
// read of 32-column block mb is the mb = 0 address with bits 6.. flipped by mb.  One register per
// lane and stream then addresses every k-step (one XOR each) instead of one register per k-step.
typedef __attribute__((address_space(3))) const char lds_cchar;
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(lds_cchar*)p;
}
__device__ __forceinline__ bf16x8 lds_b128(uint32_t a) {
#if defined(__HIP_DEVICE_COMPILE__)
    return *(__attribute__((address_space(3))) const bf16x8*)(uintptr_t)a;
#else
    (void)a;
    return bf16x8{};
#endif
}
__device__ __forceinline__ bf16x4 lds_tr4_at(uint32_t a) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_bit_cast(
        bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(uintptr_t)a));
#else
    (void)a;
    return bf16x4{};
#endif
}
// Byte offset in a tile of lane (lr = l % 32, g = l / 32)'s row read at ks = 0 (RowOperand).
template <int D>
__device__ __forceinline__ uint32_t row_read_off(int lane) {
    return 2u * (uint32_t)tile_off<D>(lane & 31, 8 * (lane >> 5));
}
// Byte offsets in a tile of the lane's two transposing reads at mb = 0 (TrOperand).
template <int D>
__device__ __forceinline__ uint32_t tr_read_off(int lane, int h) {
    const int s = lane & 15, q = (lane >> 4) & 1, rr = 4 * (lane >> 5) + (s >> 2);
    return 2u * (uint32_t)tile_off<D>(rr + 8 * h, 16 * q + 4 * (s & 3));
}
// Issue order for the dK/dV pass's product blocks: N MFMAs, each fed by two LDS reads; the reads
// run LA matrix instructions ahead.
template <int N, int LA>
__device__ __forceinline__ void sched_mfma_2lds() {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < N - LA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, LA, 0);
}

// Bias modes of one (wavefront, query tile) of the dK/dV pass, the same for every head: the tile
// kind, the position and time modes with their buckets and thresholds.  With the stored-dS
// workspace the modes pass (bwd_modes_kernel) writes them for every (sequence, key block, query
// tile) ahead of the dK/dV pass, which copies each tile's eight records into LDS with its rows;
// without it eight lanes of wavefront 0 decide them from the tile's times.  Each wavefront turns
// its record into bias values with its head's tables (mode_timesel).
struct ModeRec {
    uint32_t bits;  // kind | pm << 2 | tm << 3 | later << 6 | pkind << 7 | pneg << 9
    uint32_t bk;    // position buckets lo | hi << 8, time buckets lo << 16 | hi << 24
    uint32_t thr, thr2;  // time thresholds (modes 1 and 4)
    uint32_t pthr;       // position threshold (two position buckets)
    uint32_t pad[3];
};
static_assert(sizeof(ModeRec) == 32, "eight records make one 256-byte copy");

// The record of key group [mk0, mk1) (key times tkmin .. tkmax; kfit: all fit in 32 bits relative
// to the sequence's first time; kmax_rel: tkmax so) against query rows mq0 .. mq1 (times
// tlo .. thi; qfit as kfit) of a sequence of n rows with nc contexts and nh = n - candidates.
//   pm: position bias one bucket (0) or per element (1); pkind, buckets, pthr, pneg: the position
//   span for the bias-gradient sums (pneg: every i - j <= 0).
//   tm (as TimeSel::set): 0 one time bucket, 1 / 4 two / three buckets by threshold (key minus
//   query has one sign; later: key times not below query times), 2 / 3 per-element class with
//   32-bit / 64-bit times.
__device__ __forceinline__ ModeRec make_mode_rec(bool rp, bool rt, int mk0, int mk1, int mq0,
                                                 int mq1, int n, int nc, int nh, int64_t tkmin,
                                                 int64_t tkmax, bool kfit, uint32_t kmax_rel,
                                                 int64_t tlo, int64_t thi, bool qfit) {
    ModeRec m{};
    const uint32_t kind = mk0 < mk1 && mq0 < n ? classify_key_tile(mk0, mk1, mq0, n, nc, nh, kWaveRows)
                                               : kEmpty;
    uint32_t pm = 0, tm = 0, later = 1, pkind = 0, pneg = 0, pb_lo = 0, pb_hi = 0, tb_lo = 0,
             tb_hi = 0;
    m.thr = m.thr2 = m.pthr = 0xffffffffu;
    if (rp) {
        const BiasSpan sp = bias_span((int64_t)mq0 - (mk1 - 1), (int64_t)mq1 - mk0);
        pkind = (uint32_t)sp.kind;
        pb_lo = (uint32_t)sp.b_lo;
        pb_hi = (uint32_t)sp.b_hi;
        m.pthr = sp.thr;
        pneg = mq1 - mk0 <= 0 ? 1u : 0u;
        pm = sp.kind != 0 ? 1u : 0u;
    }
    if (rt) {
        const int64_t dlo = tkmin - thi;
        const BiasSpan st = bias_span(dlo, tkmax - tlo);
        tb_lo = (uint32_t)st.b_lo;
        tb_hi = (uint32_t)st.b_hi;
        const bool lat = dlo >= 0;
        if (st.kind == 0) tm = 0;
        else if (!(kfit && qfit)) tm = 3;
        else if (st.kind == 2) tm = 2;
        else if (!lat && (uint64_t)kmax_rel + (st.kind == 1 ? st.thr : st.thr2) > 0xffffffffull)
            tm = 2;
        else {
            tm = st.kind == 1 ? 1u : 4u;
            m.thr = st.thr;
            m.thr2 = st.thr2;
            later = lat ? 1u : 0u;
        }
    }
    m.bits = kind | pm << 2 | tm << 3 | later << 6 | pkind << 7 | pneg << 9;
    m.bk = pb_lo | pb_hi << 8 | tb_lo << 16 | tb_hi << 24;
    return m;
}

template <int D>
struct SmemA {
    float wt[kNumClasses];               // -log2(e) * time bias by class
    float wp[kNumBuckets];               // -log2(e) * position bias by bucket
    float wtb[kNumBuckets];              // -log2(e) * time bias by bucket
    float rp[2][kToep + 1];
    uint32_t tq[2][kTile];
    int64_t tq64[2][kTile];
    ModeRec modes[2][8];                 // by tile buffer, 4 * query half + key group
    int64_t kgmin[4], kgmax[4];          // key times of each key group: range, whether all fit
    uint32_t kgmax_rel[4];               // in 32 bits relative to the sequence's first time
    int kgfit[4];
    // bias-table gradient sums of the unit (stored-dS pass only), by bucket; time sums by
    // (bucket, lane % 32) so that per-lane additions rarely share an address
    float hbp[kNumBuckets];
    float hbt[kNumBuckets][32];
    int64_t kt64[kBlk];                  // the unit's key times (read by the 64-bit time mode)
    alignas(256) bf16 q[2][kTile * D];   // swizzled tiles (tile_off), 256-byte aligned (lds_b128)
    bf16 dout[2][kTile * D];
    alignas(256) bf16 kb[kBlk * D];      // the unit's keys and values, swizzled like the tiles
    bf16 vb[kBlk * D];
};

// A record's bias values for this head: TimeSel with the position bias folded in when it is one
// bucket (bits, bk, thresholds wavefront-uniform).
template <int D, bool RP, bool RT>
__device__ __forceinline__ TimeSel mode_timesel(uint32_t bits, uint32_t bk, uint32_t thr,
                                                uint32_t thr2, const SmemA<D>& sm) {
    const uint32_t pm = (bits >> 2) & 1u, tm = (bits >> 3) & 7u;
    const float bpos = RP && pm == 0 ? sm.wp[bk & 0xffu] : 0.0f;
    TimeSel tb;
    tb.set_const(bpos);
    if (RT) {
        const int lo = (int)((bk >> 16) & 0xffu), hi = (int)(bk >> 24);
        if (tm == 0) tb.set_const(bpos + sm.wtb[lo]);
        else if (tm == 1 || tm == 4) {
            tb.b0 = bpos + sm.wtb[lo];
            tb.b1 = bpos + sm.wtb[imin(lo + 1, kNumBuckets - 1)];
            tb.b2 = bpos + sm.wtb[hi];
            tb.thr = thr;
            tb.thr2 = thr2;
            tb.later = ((bits >> 6) & 1u) != 0;
        }
    }
    return tb;
}

// Bias modes of a (wavefront, tile) as in the forward:
//   PM 0: position bias absent or one bucket (inside b0/b1); 1: Toeplitz table per element.
//   TM 0: time bias absent or one bucket; 1: two buckets, b1 where |dt| >= thr; 2 / 3: per-element
//      bucket class with 32-bit / 64-bit times.
// One wavefront's 32 x 32 block: queries q0 + (8r + 4g + c) of the tile (C layout), its key per
// lane; u0 is the Toeplitz slot of the block's first query for this lane.  The modes only form
// the scores t = -log2(e) S in place; the sigmoid and gradient arithmetic that follows is common
// (silu_grad_all), so the mode branches rejoin with one register set.
template <int D, int PM, int TM>
__device__ __forceinline__ void scores_a(f32x16& s, const SmemA<D>& sm, int buf, int q0, int u0,
                                         int g, float alpha2, const TimeSel tb, uint32_t tj,
                                         int kl) {
    const TimePick pick(tb, tj);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ii = q0 + 8 * r + 4 * g;
        u32x4 tq4;
        if (TM == 1 || TM == 2 || TM == 4) tq4 = *reinterpret_cast<const u32x4*>(&sm.tq[buf][ii]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * r + c;
            float b = pick.get<TM>(tq4[c]);
            if (PM == 1) b += sm.rp[buf][u0 + 8 * r + c];
            if (TM == 2) b += sm.wt[bucket_class(absdiff_u32(tj, tq4[c]))];
            if (TM == 3) b += sm.wt[bucket_class(absdiff_sat(sm.kt64[kl], sm.tq64[buf][ii + c]))];
            s[e] = fmaf(alpha2, s[e], b);
        }
    }
}

template <int D, int PM>
__device__ __forceinline__ void scores_a_tm(int tm, f32x16& s, const SmemA<D>& sm, int buf, int q0,
                                            int u0, int g, float alpha2, const TimeSel tb,
                                            uint32_t tj, int kl) {
    switch (tm) {
        case 0: scores_a<D, PM, 0>(s, sm, buf, q0, u0, g, alpha2, tb, tj, kl); break;
        case 1: scores_a<D, PM, 1>(s, sm, buf, q0, u0, g, alpha2, tb, tj, kl); break;
        case 4: scores_a<D, PM, 4>(s, sm, buf, q0, u0, g, alpha2, tb, tj, kl); break;
        case 2: scores_a<D, PM, 2>(s, sm, buf, q0, u0, g, alpha2, tb, tj, kl); break;
        default: scores_a<D, PM, 3>(s, sm, buf, q0, u0, g, alpha2, tb, tj, kl); break;
    }
}

// P' and dS N of all sixteen elements from the scores and dP (silu_grad).
__device__ __forceinline__ void silu_grad_all(f32x16& s, f32x16& dp) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const Grad gr = silu_grad(s[e], dp[e]);
        s[e] = gr.p;
        dp[e] = gr.ds;
    }
}

// Zero P and dS of the block's queries iq0 + (8r + 4g + c) that do not see this lane's key
// (partial tiles only).
__device__ __forceinline__ void mask_queries(f32x16& s, f32x16& dp, int g, int iq0, int lo, int hi) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = iq0 + 8 * (e >> 2) + 4 * g + (e & 3);
        const bool vis = i >= lo && i <= hi;
        s[e] = vis ? s[e] : 0.0f;
        dp[e] = vis ? dp[e] : 0.0f;
    }
}

// Bias-table gradient sums of one (wavefront, tile) of the dK/dV pass: d8 holds dS * N (as
// stored, bf16; element e = 8 sl + x in d8[sl][x]) of the queries i = iq0 + (8r + 4g + c) for
// this lane's key j (zero where not visible).  The tile's
// pairs fall in the buckets the forward bias decisions found (sp: position, st / tm: time):
//   one bucket: the wavefront's sum of dS goes to it;
//   two or three adjacent buckets: per lane, the sums over pairs at or past each threshold are
//     kept too (one comparison per pair and threshold), and the splits go to the buckets;
//   more: each pair's bucket is computed and per-lane runs along the lane's queries (whose
//     buckets change rarely) are added to the histogram when the bucket changes.
// Wavefront sums go through a DPP reduction and one single-lane LDS atomic per bucket.
template <int D, bool GP, bool GT, int PG, int TM>
__device__ __forceinline__ void grads_a_t(const bf16x8 (&d8)[2], SmemA<D>& sm, int buf, int q0,
                                          int iq0, int j, int g, int lane, const BiasSpan& sp,
                                          bool pneg, const BiasSpan& st, uint32_t thr,
                                          uint32_t thr2, uint32_t tj, int kl) {
    float sum = 0.0f, thp = 0.0f, tht = 0.0f, tht2 = 0.0f;
    // position: i - j = base + 8r + c, of one sign over the tile when PG < 2 (pneg: every
    // i - j <= 0); lanes and queries outside the tile's visible pairs carry dS = 0
    const int base = iq0 + 4 * g - j;
    int pcur = -1, tcur = -1;
    float pacc = 0.0f, tacc = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int ii = q0 + 8 * r + 4 * g;
        u32x4 tq4;
        if (TM == 1 || TM == 2 || TM == 4) tq4 = *reinterpret_cast<const u32x4*>(&sm.tq[buf][ii]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * r + c;
            const float ds = (float)d8[e >> 3][e & 7];
            const int d = base + 8 * r + c;  // i - j
            sum += ds;
            if (PG == 1) thp += (uint32_t)(pneg ? -d : d) >= sp.thr ? ds : 0.0f;
            if (PG == 2) {
                const int b = bucket_of((uint32_t)(d < 0 ? -d : d));
                if (b != pcur) {
                    if (pcur >= 0) atomicAdd(&sm.hbp[pcur], pacc);
                    pcur = b;
                    pacc = 0.0f;
                }
                pacc += ds;
            }
            if (TM == 1 || TM == 4) {
                const uint32_t dt = absdiff_u32(tj, tq4[c]);
                tht += dt >= thr ? ds : 0.0f;
                if (TM == 4) tht2 += dt >= thr2 ? ds : 0.0f;
            }
            if (TM == 2 || TM == 3) {
                const int b = TM == 2 ? bucket_of(absdiff_u32(tj, tq4[c]))
                                      : bucket_of(absdiff_sat(sm.kt64[kl], sm.tq64[buf][ii + c]));
                if (b != tcur) {
                    if (tcur >= 0) atomicAdd(&sm.hbt[tcur][lane & 31], tacc);
                    tcur = b;
                    tacc = 0.0f;
                }
                tacc += ds;
            }
        }
    }
    if (PG == 2 && pcur >= 0) atomicAdd(&sm.hbp[pcur], pacc);
    if ((TM == 2 || TM == 3) && tcur >= 0) atomicAdd(&sm.hbt[tcur][lane & 31], tacc);
    constexpr bool pfew = GP && PG < 2, tfew = GT && (TM == 0 || TM == 1 || TM == 4);
    if constexpr (pfew || tfew) {
        const float tot = wave_sum_dpp(sum);
        const float tp = PG == 1 ? wave_sum_dpp(thp) : 0.0f;
        const float t1 = TM == 1 || TM == 4 ? wave_sum_dpp(tht) : 0.0f;
        const float t2 = TM == 4 ? wave_sum_dpp(tht2) : 0.0f;
        if (lane == 0) {
            if (pfew) {
                atomicAdd(&sm.hbp[sp.b_lo], tot - tp);
                if (PG == 1) atomicAdd(&sm.hbp[sp.b_hi], tp);
            }
            if (tfew) {
                atomicAdd(&sm.hbt[st.b_lo][0], tot - t1);
                if (TM == 1) atomicAdd(&sm.hbt[st.b_hi][0], t1);
                if (TM == 4) {
                    atomicAdd(&sm.hbt[st.b_lo + 1][0], t1 - t2);
                    atomicAdd(&sm.hbt[st.b_hi][0], t2);
                }
            }
        }
    }
}

template <int D, bool GP, bool GT, int PG>
__device__ __forceinline__ void grads_a_pg(int tm, const bf16x8 (&d8)[2], SmemA<D>& sm, int buf,
                                           int q0, int iq0, int j, int g, int lane,
                                           const BiasSpan& sp, bool pneg, const BiasSpan& st,
                                           uint32_t thr, uint32_t thr2, uint32_t tj, int kl) {
    switch (GT ? tm : 0) {
        case 0: grads_a_t<D, GP, GT, PG, 0>(d8, sm, buf, q0, iq0, j, g, lane, sp, pneg, st, thr, thr2, tj, kl); break;
        case 1: grads_a_t<D, GP, GT, PG, 1>(d8, sm, buf, q0, iq0, j, g, lane, sp, pneg, st, thr, thr2, tj, kl); break;
        case 4: grads_a_t<D, GP, GT, PG, 4>(d8, sm, buf, q0, iq0, j, g, lane, sp, pneg, st, thr, thr2, tj, kl); break;
        case 2: grads_a_t<D, GP, GT, PG, 2>(d8, sm, buf, q0, iq0, j, g, lane, sp, pneg, st, thr, thr2, tj, kl); break;
        default: grads_a_t<D, GP, GT, PG, 3>(d8, sm, buf, q0, iq0, j, g, lane, sp, pneg, st, thr, thr2, tj, kl); break;
    }
}

template <int D, bool GP, bool GT>
__device__ __forceinline__ void grads_a(const bf16x8 (&d8)[2], SmemA<D>& sm, int buf, int q0,
                                        int iq0, int j, int g, int lane, const BiasSpan& sp,
                                        bool pneg, const BiasSpan& st, int tm, uint32_t thr,
                                        uint32_t thr2, uint32_t tj, int kl) {
    const int pg = !GP ? -1 : sp.kind == 0 ? 0 : sp.kind == 1 ? 1 : 2;
    if (pg == 0) grads_a_pg<D, GP, GT, 0>(tm, d8, sm, buf, q0, iq0, j, g, lane, sp, pneg, st, thr, thr2, tj, kl);
    else if (pg == 1) grads_a_pg<D, GP, GT, 1>(tm, d8, sm, buf, q0, iq0, j, g, lane, sp, pneg, st, thr, thr2, tj, kl);
    else if (pg == 2) grads_a_pg<D, GP, GT, 2>(tm, d8, sm, buf, q0, iq0, j, g, lane, sp, pneg, st, thr, thr2, tj, kl);
    else grads_a_pg<D, GP, GT, 3>(tm, d8, sm, buf, q0, iq0, j, g, lane, sp, pneg, st, thr, thr2, tj, kl);
}

template <int D, bool RP, bool RT, bool DS>
__global__ __launch_bounds__(kThreadsA, 1) void bwd_dkdv_kernel(const AttnParams p) {
    constexpr int kThreads = kThreadsA;  // the helpers below stride over the whole workgroup
    __shared__ __attribute__((aligned(16))) SmemA<D> sm;

    const WorkUnit wu = p.units[blockIdx.x];
    const SeqInfo si = p.seqs[wu.seq];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lr = lane & 31;
    const int wave = (tid >> 6) & 3, qh = tid >> 8;  // key group, query half
    const int n = si.n, nc = si.nc, nh = si.nh, k0 = wu.row0, h = wu.head;
    const int64_t tok0 = si.start, ld = p.ld_in;
    const bf16* __restrict__ qg = static_cast<const bf16*>(p.q) + tok0 * ld + h * D;
    const bf16* __restrict__ kg = static_cast<const bf16*>(p.k) + tok0 * ld + h * D;
    const bf16* __restrict__ vg = static_cast<const bf16*>(p.v) + tok0 * ld + h * D;
    const bf16* __restrict__ dog = static_cast<const bf16*>(p.dout) + tok0 * p.ld_out + h * D;

    if (RP)
        for (int e = tid; e < kNumBuckets; e += kThreads)
            sm.wp[e] = -kLog2e * p.rab_pos[h * kNumBuckets + e];
    if (RT) {
        for (int e = tid; e < kNumClasses; e += kThreads)
            sm.wt[e] = -kLog2e * p.rab_ts[h * kNumBuckets + bucket_of_class(e)];
        for (int e = tid; e < kNumBuckets; e += kThreads)
            sm.wtb[e] = -kLog2e * p.rab_ts[h * kNumBuckets + e];
    }
        if constexpr (DS && (RP || RT)) {
        for (int e = tid; e < kNumBuckets; e += kThreads) sm.hbp[e] = 0.0f;
        for (int e = tid; e < kNumBuckets * 32; e += kThreads) (&sm.hbt[0][0])[e] = 0.0f;
    }
    const int64_t tbase = RT ? p.ts[tok0] : 0;  const int khi = imin(k0 + kBlk, n);
    int qlo, qhi;
    rows_for_keys(k0, khi, n, nc, nh, &qlo, &qhi);
    const int tfirst = qlo / kTile, ntiles = cdiv(qhi, kTile) - tfirst;
    // partial dK, dV of the second query half go through the (then idle) tile buffers
    static_assert(sizeof(sm.q) + sizeof(sm.dout) >= 4 * (D / 32) * 16 * 64 * sizeof(float),
                  "reduction buffer");

    const int wk0 = k0 + kWaveRows * wave;
    const int j = wk0 + lr;
    const bool key_ok = j < khi;
    int lo = 1, hi = 0;  // rows that see key j: lo <= i <= hi
    if (key_ok) {
        if (j < nc) { lo = 0; hi = n - 1; }
        else if (j < nh) { lo = j; hi = n - 1; }
        else { lo = j; hi = j; }
    }
    uint32_t tj = 0;
    int64_t tj64 = 0, tjmin = 0, tjmax = 0;
    uint32_t tjmax_rel = 0;
    bool wave_kfit = true;
    if (RT) {
        tj64 = key_ok ? p.ts[tok0 + j] : tbase;
        wave_kfit = __all(rel_time_fits(tj64, tbase));
        tj = rel_time_u32(tj64, tbase);
        {
            int64_t lo, hi;
            wave_time_minmax(tj64, key_ok, tbase, lo, hi);
            tjmin = uniform64(lo);
            tjmax = uniform64(hi);
        }
        tjmax_rel = rel_time_u32(tjmax, tbase);  // used only when every key time fits
        if (qh == 0) sm.kt64[kWaveRows * wave + lr] = tj64;  // read after the first barrier
        if (qh == 0 && lane == 0) {
            sm.kgmin[wave] = tjmin;
            sm.kgmax[wave] = tjmax;
            sm.kgmax_rel[wave] = tjmax_rel;
            sm.kgfit[wave] = wave_kfit ? 1 : 0;
        }
    }

    f32x16 dvt[D / 32], dkt[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) { dvt[db] = f32x16{}; dkt[db] = f32x16{}; }

    // query-tile copies from inline assembly (see the forward kernel): explicit waits only
    const i32x4 qrs = rows_words(qg, n, ld, D), drs = rows_words(dog, n, p.ld_out, D);
    const TileDma<D, kThreads> qdma(tid, ld), ddma(tid, p.ld_out);
    // byte offsets of this lane's operand reads (lds_b128, lds_tr4_at)
    const uint32_t roff = row_read_off<D>(lane) + (uint32_t)(qh * 64 * D);
    const uint32_t kaddr = lds_u32(sm.kb) + row_read_off<D>(lane) + (uint32_t)(wave * 64 * D);
    const uint32_t toff0 = tr_read_off<D>(lane, 0) + (uint32_t)(qh * 64 * D);
    const uint32_t toff1 = tr_read_off<D>(lane, 1) + (uint32_t)(qh * 64 * D);
    // stored dS: the unit's chunks (geometry.h), one 128-key x 64-query block per tile; this
    // lane's key row, its 4 queries 4g .. 4g + 3 of each group of 8 (byte offset); the tile's
    // chunk goes into the scalar offset
    const bf16* dsb = nullptr;
    int ds_voff = 0;
    int64_t ds_size = 0;
    if constexpr (DS) {
        const int kb = k0 / kBlk, nch = ds_chunks(kb, n, nc, nh);
        dsb = static_cast<const bf16*>(p.ds) + p.ds_off[wu.seq] +
              (int64_t)kDsChunk * ((int64_t)p.heads * ds_chunks_before(kb, n, nc, nh) + (int64_t)h * nch);
        ds_voff = ((j - k0) * kTile + kWaveRows * qh + 4 * g) * 2;
        ds_size = (int64_t)nch * kDsChunk * 2;
    }
    const buffer_rsrc dsrs = bytes_rsrc(dsb, ds_size);
    int64_t tqr = 0;
    // stored-dS workspace: the unit's mode records (one 256-byte block per tile, from the modes
    // pass) and the sequence's relative and raw query times, copied into LDS with each tile
    i32x4 mrs{}, trs{}, tsrs{};
    if constexpr (DS) {
        const int kb = k0 / kBlk;
        const ModeRec* mb = static_cast<const ModeRec*>(p.modes) +
                            8 * (p.ds_off[wu.seq] / ((int64_t)kDsChunk * p.heads) +
                                 ds_chunks_before(kb, n, nc, nh));
        mrs = rsrc_words(mb, (int64_t)ntiles * 8 * (int64_t)sizeof(ModeRec));
        trs = rsrc_words(RT ? p.tq_rel + tok0 : nullptr, RT ? (int64_t)n * 4 : 0);
        tsrs = rsrc_words(RT ? p.ts + tok0 : nullptr, RT ? (int64_t)n * 8 : 0);
    }
    // starts the copy of a query tile's Q and dO rows into buffer buf and loads its timestamps
    // (stored-dS workspace: copies its records and times too, one 256-byte copy per wavefront
    // 0 .. 3; rows past the sequence end read as zero)
    auto load_tile = [&](int buf, int tile) {
        const int i0 = tile * kTile;
        if constexpr (DS) {
            if (tid < 64) copy4_lds_asm(mrs, lds_addr(&sm.modes[buf][0]), (tile - tfirst) * 256 + 4 * lane);
            else if (RT && tid < 128) copy4_lds_asm(trs, lds_addr(&sm.tq[buf][0]), i0 * 4 + 4 * lane);
            else if (RT && tid < 256) {
                const int hf = (tid >> 6) - 2;
                copy4_lds_asm(tsrs, lds_addr(&sm.tq64[buf][32 * hf]), i0 * 8 + 256 * hf + 4 * lane);
            }
        } else if (RT && tid < kTile) {  // first: see the forward kernel's load_tile
            const int i = i0 + tid;
            tqr = i < n ? p.ts[tok0 + i] : tbase;
        }
        qdma.issue_asm(qrs, sm.q[buf], (int)((int64_t)i0 * ld * 2));
        ddma.issue_asm(drs, sm.dout[buf], (int)((int64_t)i0 * p.ld_out * 2));
    };
    // the tile's small tables: (without the workspace) query times and the eight mode records;
    // position bias by (i - j)
    auto store_tile = [&](int buf, int tile) {
        const int i0 = tile * kTile;
        if (!DS && tid < kTile) {  // exactly wavefront 0
            TimeRange tr{};
            if (RT) {
                const bool real = i0 + tid < n;
                sm.tq64[buf][tid] = tqr;
                sm.tq[buf][tid] = rel_time_u32(tqr, tbase);
                tr = wave_time_range(tqr, real, tbase);
            }
            if (tid < 8) {  // lane 4 hq + w: key group w, query half hq
                const int w = tid & 3, hq = tid >> 2;
                const int mk0 = k0 + kWaveRows * w, mk1 = imin(mk0 + kWaveRows, khi);
                const int mq0 = i0 + kWaveRows * hq, mq1 = imin(mq0 + kWaveRows, n) - 1;
                sm.modes[buf][tid] = make_mode_rec(
                    RP, RT, mk0, mk1, mq0, mq1, n, nc, nh, sm.kgmin[w], sm.kgmax[w],
                    sm.kgfit[w] != 0, sm.kgmax_rel[w], hq ? tr.lo[1] : tr.lo[0],
                    hq ? tr.hi[1] : tr.hi[0], tr.fit);
            }
        }
        if (RP)
            for (int u = tid; u < kToep; u += kThreads) {
                const int delta = (i0 - k0) - (kBlk - 1) + u;  // i - j for slot u
                sm.rp[buf][u] = sm.wp[bucket_of((uint32_t)(delta < 0 ? -delta : delta))];
            }
    };

    {  // the unit's 128 keys and values (rows past the sequence end read as zero)
        const buffer_rsrc krs = rows_rsrc(kg, n, ld, D), vrs = rows_rsrc(vg, n, ld, D);
        const TileDma<D, kThreads> kvdma(tid, ld);
#pragma unroll
        for (int half = 0; half < kBlk / kTile; ++half) {
            const int row_bytes = (int)((int64_t)(k0 + kTile * half) * ld * 2);
            kvdma.issue(krs, sm.kb + kTile * half * D, row_bytes);
            kvdma.issue(vrs, sm.vb + kTile * half * D, row_bytes);
        }
    }
    __syncthreads();
    load_tile(0, tfirst);
    store_tile(0, tfirst);
    wait_tile_dma();
    __syncthreads();

    // slot of (query i0 + ii, key j) is u0 + ii - 4g; this wavefront's queries start at ii = q0
    const int q0 = kWaveRows * qh;
    const int u0 = 4 * g - (kWaveRows * wave + lr) + (kBlk - 1) + q0;
    const float alpha2 = -kLog2e * p.alpha;
    const int mslot = uniform_i(4 * qh + wave);

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1, i0 = (tfirst + t) * kTile, iq0 = i0 + q0;
        if (t + 1 < ntiles) load_tile(buf ^ 1, tfirst + t + 1);
        const ModeRec& md = sm.modes[buf][mslot];
        const uint32_t mbits = (uint32_t)uniform_i((int)md.bits);
        const int kind = (int)(mbits & 3u);
        if (kind != kEmpty) {
            f32x16 s = f32x16{}, dp = f32x16{};
            // this lane's Q row (dO: + sizeof(sm.q)) and key row (V: + sizeof(sm.kb)) at ks = 0,
            // opaque so that the per-ks addresses are formed here rather than held in registers
            uint32_t qa = lds_u32(sm.q[buf]) + roff, ka = kaddr;
            asm volatile("" : "+v"(qa), "+v"(ka));
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                const uint32_t xq = qa ^ (uint32_t)(ks << 5), xk = ka ^ (uint32_t)(ks << 5);
                s = mfma32(lds_b128(xq), lds_b128(xk), s);
                dp = mfma32(lds_b128(xq + (uint32_t)sizeof(sm.q)), lds_b128(xk + (uint32_t)sizeof(sm.kb)), dp);
            }
            sched_mfma_2lds<D / 8, kReadAhead>();
            const int pm = RP ? (int)((mbits >> 2) & 1u) : 0, tm = RT ? (int)((mbits >> 3) & 7u) : 0;
            const uint32_t mbk = (uint32_t)uniform_i((int)md.bk);
            const TimeSel tb = mode_timesel<D, RP, RT>(mbits, mbk, md.thr, md.thr2, sm);
            if (pm) scores_a_tm<D, 1>(tm, s, sm, buf, q0, u0, g, alpha2, tb, tj, kWaveRows * wave + lr);
            else scores_a_tm<D, 0>(tm, s, sm, buf, q0, u0, g, alpha2, tb, tj, kWaveRows * wave + lr);
            silu_grad_all(s, dp);
            if (kind == kPartial) mask_queries(s, dp, g, iq0, lo, hi);
            bf16x8 pb[2], db8[2];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                float tp[8], td[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    tp[x] = s[8 * sl + x];
                    td[x] = dp[8 * sl + x];
                }
                pb[sl] = pack8(tp);
                db8[sl] = pack8(td);
            }
            if constexpr (DS) {
                // stored before the dV / dK products, so that the writes complete while those run
                // (the tile-end wait counts stores too); entries 8sl .. 8sl + 3 are queries
                // 16sl + 4g + c, then + 8
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    store_bf16x4(__builtin_shufflevector(db8[sl], db8[sl], 0, 1, 2, 3), dsrs, ds_voff + 32 * sl, t * kDsChunk * 2);
                    store_bf16x4(__builtin_shufflevector(db8[sl], db8[sl], 4, 5, 6, 7), dsrs, ds_voff + 32 * sl + 16, t * kDsChunk * 2);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            uint32_t ta0 = lds_u32(sm.q[buf]) + toff0, ta1 = lds_u32(sm.q[buf]) + toff1;
            asm volatile("" : "+v"(ta0), "+v"(ta1));
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    // Q tile at +0, dO tile at + sizeof(sm.q); 16 query rows per sl
                    const uint32_t x0 = (ta0 ^ (uint32_t)(db << 6)) + (uint32_t)(sl * 32 * D);
                    const uint32_t x1 = (ta1 ^ (uint32_t)(db << 6)) + (uint32_t)(sl * 32 * D);
                    const uint32_t dq = (uint32_t)sizeof(sm.q);
                    const bf16x4 d0 = lds_tr4_at(x0 + dq), d1 = lds_tr4_at(x1 + dq);
                    const bf16x4 q0v = lds_tr4_at(x0), q1v = lds_tr4_at(x1);
                    dvt[db] = mfma32(__builtin_shufflevector(d0, d1, 0, 1, 2, 3, 4, 5, 6, 7), pb[sl], dvt[db]);
                    dkt[db] = mfma32(__builtin_shufflevector(q0v, q1v, 0, 1, 2, 3, 4, 5, 6, 7), db8[sl], dkt[db]);
                }
            sched_mfma_2lds<D / 8, kReadAhead>();
            // from the stored values, after the products are issued (their vector work overlaps
            // the matrix instructions, and S and dP in fp32 are no longer held)
            if constexpr (DS && (RP || RT)) {
                const uint32_t gb = (uint32_t)uniform_i((int)md.bits);
                const uint32_t gk = (uint32_t)uniform_i((int)md.bk);
                const BiasSpan gsp{RP ? (int)((gb >> 7) & 3u) : 0, (int)(gk & 0xffu),
                                   (int)((gk >> 8) & 0xffu), md.pthr, 0u};
                const BiasSpan gst{0, (int)((gk >> 16) & 0xffu), (int)(gk >> 24), md.thr, md.thr2};
                grads_a<D, RP, RT>(db8, sm, buf, q0, iq0, j, g, lane, gsp, ((gb >> 9) & 1u) != 0,
                                   gst, RT ? (int)((gb >> 3) & 7u) : 0, md.thr, md.thr2, tj,
                                   kWaveRows * wave + lr);
            }
        }
        if (t + 1 < ntiles) store_tile(buf ^ 1, tfirst + t + 1);
        wait_tile_dma();
        __syncthreads();
    }

    // add the second query half's partial sums into the first's, dV then dK, through LDS laid
    // out [key group][db][element][lane] (lanes consecutive: no bank conflicts)
    float* red = reinterpret_cast<float*>(&sm.q[0][0]);
    auto exchange = [&](f32x16 (&acc)[D / 32]) {
        float* mine = red + ((size_t)wave * (D / 32) * 16) * 64 + lane;
        if (qh == 1)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) mine[(db * 16 + e) * 64] = acc[db][e];
        __syncthreads();
        if (qh == 0)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[db][e] += mine[(db * 16 + e) * 64];
        __syncthreads();
    };
    bf16* dvg = static_cast<bf16*>(p.dv) + (tok0 + j) * p.ld_grad + h * D;
    bf16* dkg = static_cast<bf16*>(p.dk) + (tok0 + j) * p.ld_grad + h * D;
    GateRow<D> gv, gk;
    if (p.gate_delta != 0 && key_ok && qh == 0) {
        gv.load(dvg, g, p.gate_delta);
        gk.load(dkg, g, p.gate_delta);
    }
    exchange(dvt);
    exchange(dkt);

    if (key_ok && qh == 0) {
        const float sv = -kLn2 * p.inv_n, sk = p.alpha * p.inv_n;
        store_grad_row<D>(dvg, dvt, g, sv, p.gate_delta, gv);
        store_grad_row<D>(dkg, dkt, g, sk, p.gate_delta, gk);
    }
    if constexpr (DS && (RP || RT)) {  // the unit's bias-table gradient sums: one global atomic
        __syncthreads();                // per non-zero bucket
        for (int b = tid; b < kNumBuckets; b += kThreads) {
            if (RP && p.gpos && sm.hbp[b] != 0.0f) atomicAdd(&p.gpos[h * kNumBuckets + b], sm.hbp[b] * p.inv_n);
            if (RT && p.gts) {
                float v = 0.0f;
#pragma unroll 8
                for (int l = 0; l < 32; ++l) v += sm.hbt[b][(l + b) & 31];
                if (v != 0.0f) atomicAdd(&p.gts[h * kNumBuckets + b], v * p.inv_n);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// pass B: dQ and the bias-table gradients
// ---------------------------------------------------------------------------------------------

template <int D>
struct SmemB {
    float wt[kNumClasses];
    float wp[kNumBuckets];
    float wtb[kNumBuckets];
    ToepEntry rp[2][kToep + 1];
    uint32_t tk[2][kTile];
    int64_t tk64[2][kTile];
    int64_t tkmin[2][2], tkmax[2][2];  // time range of the real keys of each 32-key half
    int fits[2];
    float hbp[kNumBuckets];   // position-bias gradient sums, by bucket
    // time-bias gradient sums by (bucket, lane % 32): at most two lanes of a wavefront share an
    // address, whatever their buckets
    float hbt[kNumBuckets][32];
    alignas(16) bf16 k[2][kTile * D];    // swizzled tiles (tile_off)
    bf16 v[2][kTile * D];
    bf16 qb[kBlk * D];                   // the unit's query and dO rows, swizzled like the tiles
    bf16 dob[kBlk * D];
};

// Per-element part of pass B for one wavefront's 32 x 32 block: keys k0 + (8r + 4g + c) of the
// tile (C layout), this lane's row; u0 is the Toeplitz slot of the block's first key for this
// lane.  dS (times N) into dp.  Bias modes as in pass A.
template <int D, int PM, int TM>
__device__ __forceinline__ void epilogue_b(const f32x16& s, f32x16& dp, const SmemB<D>& sm, int buf,
                                           int k0, int u0, int g, float alpha2, const TimeSel tb,
                                           uint32_t ti, int64_t ti64) {
    const TimePick pick(tb, ti);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int jj = k0 + 8 * r + 4 * g;
        u32x4 tk4;
        if (TM == 1 || TM == 2 || TM == 4) tk4 = *reinterpret_cast<const u32x4*>(&sm.tk[buf][jj]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 4 * r + c;
            float b = pick.get<TM>(tk4[c]);
            if (PM == 1) b += sm.rp[buf][u0 + 8 * r + c].bias;
            if (TM == 2) b += sm.wt[bucket_class(absdiff_sad(ti, tk4[c]))];
            if (TM == 3) b += sm.wt[bucket_class(absdiff_sat(ti64, sm.tk64[buf][jj + c]))];
            dp[e] = silu_grad(fmaf(alpha2, s[e], b), dp[e]).ds;
        }
    }
}

template <int D, int PM>
__device__ __forceinline__ void epilogue_b_tm(int tm, const f32x16& s, f32x16& dp,
                                              const SmemB<D>& sm, int buf, int k0, int u0, int g,
                                              float alpha2, const TimeSel tb, uint32_t ti,
                                              int64_t ti64) {
    switch (tm) {
        case 0: epilogue_b<D, PM, 0>(s, dp, sm, buf, k0, u0, g, alpha2, tb, ti, ti64); break;
        case 1: epilogue_b<D, PM, 1>(s, dp, sm, buf, k0, u0, g, alpha2, tb, ti, ti64); break;
        case 4: epilogue_b<D, PM, 4>(s, dp, sm, buf, k0, u0, g, alpha2, tb, ti, ti64); break;
        case 2: epilogue_b<D, PM, 2>(s, dp, sm, buf, k0, u0, g, alpha2, tb, ti, ti64); break;
        default: epilogue_b<D, PM, 3>(s, dp, sm, buf, k0, u0, g, alpha2, tb, ti, ti64); break;
    }
}

// Bias-gradient sums of one (wavefront, tile), per lane:
//   sum = sum of dS (serves every term whose tile lies in one bucket),
//   mp  = sum of dS * bucket(|i - j|) (PG 1, two position buckets: the upper bucket's share is
//         mp - b_lo * sum),
//   th  = sum of dS over pairs with |dt| >= thr, th2 the same for thr2 (TM 1 and 4: two or
//         three time buckets; one comparison per pair with TimePick's limits),
// plus, for tiles spanning more buckets, per-lane runs along the lane's keys (which come in
// increasing order): a lane adds its run sum to the LDS histogram only when its own bucket
// changes (PG 2 position, TM 2 and 3 time).  LDS float atomics cost a few cycles per active
// lane, so few changes per lane keep them cheap.
struct TileSums {
    float sum, mp, th, th2;
};
template <int D, int PG, int TM, bool GP, bool GT, class Smem>
__device__ __forceinline__ TileSums grad_sums(const f32x16& dp, Smem& sm, int buf, int k0,
                                              int u0, int g, int lane, const TimeSel tb,
                                              uint32_t ti, int64_t ti64) {
    TileSums ts{0.0f, 0.0f, 0.0f, 0.0f};
    const TimePick pick(tb, ti);
    int pcur = -1, tcur = -1;  // per-lane runs of the many-bucket modes
    float pacc = 0.0f, tacc = 0.0f;
    auto prun = [&](int b, float ds) {
        if (b != pcur) {
            if (pcur >= 0) atomicAdd(&sm.hbp[pcur], pacc);
            pcur = b;
            pacc = 0.0f;
        }
        pacc += ds;
    };
    auto trun = [&](int b, float ds) {
        if (b != tcur) {
            if (tcur >= 0) atomicAdd(&sm.hbt[tcur][lane & 31], tacc);
            tcur = b;
            tacc = 0.0f;
        }
        tacc += ds;
    };
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int jj = k0 + 8 * r + 4 * g;
            u32x4 tk4;
            if (GT && (TM == 1 || TM == 2 || TM == 4)) tk4 = *reinterpret_cast<const u32x4*>(&sm.tk[buf][jj]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float ds = dp[4 * r + c];
                const int u = u0 + 8 * r + c;
                ts.sum += ds;
                if (GP && PG == 1) ts.mp = fmaf(ds, sm.rp[buf][u].bucket, ts.mp);
                if (GP && PG == 2) prun((int)sm.rp[buf][u].bucket, ds);
                if (GT && (TM == 1 || TM == 4)) {  // sums over te < l (see TimePick)
                    ts.th += tk4[c] < pick.l1 ? ds : 0.0f;
                    if (TM == 4) ts.th2 += tk4[c] < pick.l2 ? ds : 0.0f;
                }
                if (GT && TM == 2) trun(bucket_of(absdiff_sad(ti, tk4[c])), ds);
                if (GT && TM == 3) trun(bucket_of(absdiff_sat(ti64, sm.tk64[buf][jj + c])), ds);
            }
        }
    if (GP && PG == 2 && pcur >= 0) atomicAdd(&sm.hbp[pcur], pacc);
    if (GT && (TM == 2 || TM == 3) && tcur >= 0) atomicAdd(&sm.hbt[tcur][lane & 31], tacc);
    if (GT && (TM == 1 || TM == 4) && !tb.later) {  // te < l counted the pairs below thr
        ts.th = ts.sum - ts.th;
        ts.th2 = ts.sum - ts.th2;
    }
    return ts;
}

template <int D, int PG, bool GP, bool GT, class Smem>
__device__ __forceinline__ TileSums grad_sums_tm(int tm, const f32x16& dp, Smem& sm, int buf,
                                                 int k0, int u0, int g, int lane, const TimeSel tb,
                                                 uint32_t ti, int64_t ti64) {
    switch (GT ? tm : 0) {
        case 0: return grad_sums<D, PG, 0, GP, GT>(dp, sm, buf, k0, u0, g, lane, tb, ti, ti64);
        case 1: return grad_sums<D, PG, 1, GP, GT>(dp, sm, buf, k0, u0, g, lane, tb, ti, ti64);
        case 4: return grad_sums<D, PG, 4, GP, GT>(dp, sm, buf, k0, u0, g, lane, tb, ti, ti64);
        case 2: return grad_sums<D, PG, 2, GP, GT>(dp, sm, buf, k0, u0, g, lane, tb, ti, ti64);
        default: return grad_sums<D, PG, 3, GP, GT>(dp, sm, buf, k0, u0, g, lane, tb, ti, ti64);
    }
}

// Zero dS of the block's keys jk0 + (8r + 4g + c) that this lane's row does not see (partial
// tiles only).
__device__ __forceinline__ void mask_keys_b(f32x16& dp, int g, int jk0, int lim, int dg) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int j = jk0 + 8 * (e >> 2) + 4 * g + (e & 3);
        dp[e] = (j <= lim || j == dg) ? dp[e] : 0.0f;
    }
}

// A per-lane running sum for one histogram bucket (the same bucket across the wavefront).  A
// change of bucket flushes the wavefront's total (DPP reduction) with one single-lane LDS atomic
// at hist[bucket * stride].
struct Run {
    int cur = -1;
    float acc = 0.0f;
    __device__ __forceinline__ void add(float* hist, int bucket, float v, int lane, int stride = 1) {
        if (bucket != cur) {
            const float tot = wave_sum_dpp(acc);
            if (cur >= 0 && lane == 0) atomicAdd(&hist[cur * stride], tot);
            cur = bucket;
            acc = 0.0f;
        }
        acc += v;
    }
};

template <int D, bool RP, bool RT, bool GP, bool GT>
__global__ __launch_bounds__(kThreadsA, 1) void bwd_dq_kernel(const AttnParams p) {
    constexpr int kThreads = kThreadsA;  // the helpers below stride over the whole workgroup
    __shared__ __attribute__((aligned(16))) SmemB<D> sm;

    const WorkUnit wu = p.units[blockIdx.x];
    const SeqInfo si = p.seqs[wu.seq];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lr = lane & 31;
    const int wave = uniform_i((tid >> 6) & 3), kh = uniform_i(tid >> 8);  // row group, key half
    const int n = si.n, nc = si.nc, nh = si.nh, r0 = wu.row0, h = wu.head;
    const int64_t tok0 = si.start, ld = p.ld_in;
    const bf16* __restrict__ qg = static_cast<const bf16*>(p.q) + tok0 * ld + h * D;
    const bf16* __restrict__ kg = static_cast<const bf16*>(p.k) + tok0 * ld + h * D;
    const bf16* __restrict__ vg = static_cast<const bf16*>(p.v) + tok0 * ld + h * D;
    const bf16* __restrict__ dog = static_cast<const bf16*>(p.dout) + tok0 * p.ld_out + h * D;

    if (RP)
        for (int e = tid; e < kNumBuckets; e += kThreads)
            sm.wp[e] = -kLog2e * p.rab_pos[h * kNumBuckets + e];
    if (RT) {
        for (int e = tid; e < kNumClasses; e += kThreads)
            sm.wt[e] = -kLog2e * p.rab_ts[h * kNumBuckets + bucket_of_class(e)];
        for (int e = tid; e < kNumBuckets; e += kThreads)
            sm.wtb[e] = -kLog2e * p.rab_ts[h * kNumBuckets + e];
    }
    for (int e = tid; e < kNumBuckets; e += kThreads) sm.hbp[e] = 0.0f;
    for (int e = tid; e < kNumBuckets * 32; e += kThreads) (&sm.hbt[0][0])[e] = 0.0f;
    const int64_t tbase = RT ? p.ts[tok0] : 0;

    const int rhi = imin(r0 + kBlk, n);
    const KeyTiles ktl = key_tiles_for_rows(r0, rhi, nc, nh);
    const int ntiles = ktl.count();
    const int wlo = r0 + kWaveRows * wave, whi = imin(wlo + kWaveRows, rhi);
    const int i = wlo + lr;
    const bool row_ok = i < rhi;
    int lim = -1, dg = -1;
    if (row_ok) {
        if (i < nh) lim = imax(i, nc - 1);
        else { lim = nh - 1; dg = i; }
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
    f32x16 dqt[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqt[db] = f32x16{};
    Run run_p_lo, run_p_hi, run_t_lo, run_t_mid, run_t_hi;  // bias-gradient running sums

    // key-tile copies from inline assembly (see the forward kernel): explicit waits only
    const i32x4 krs = rows_words(kg, n, ld, D), vrs = rows_words(vg, n, ld, D);
    const TileDma<D, kThreads> dma(tid, ld);
    const RowOperand<D> rowop(lane);
    const TrOperand<D> trop(lane);
    int64_t tkr = 0;
    // loads a key tile's timestamps (first: see the forward kernel's load_tile) and starts the
    // copy of its K and V rows into buffer buf
    auto load_tile = [&](int buf, int tile) {
        const int j0 = tile * kTile;
        const int row_bytes = (int)((int64_t)j0 * ld * 2);
        if (RT && tid < kTile) {
            const int jj = j0 + tid;
            tkr = jj < n ? p.ts[tok0 + jj] : tbase;
        }
        dma.issue_asm(krs, sm.k[buf], row_bytes);
        dma.issue_asm(vrs, sm.v[buf], row_bytes);
    };
    // the tile's small tables: key times and their range, position bias and bucket by (i - j)
    auto store_tile = [&](int buf, int tile) {
        const int j0 = tile * kTile;
        if (RT && tid < kTile) {  // exactly wavefront 0
            const bool real = j0 + tid < n;
            sm.tk64[buf][tid] = tkr;
            sm.tk[buf][tid] = rel_time_u32(tkr, tbase);
            const TimeRange tr = wave_time_range(tkr, real, tbase);
            if (tid == 0) {
                sm.fits[buf] = tr.fit ? 1 : 0;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    sm.tkmin[buf][hf] = tr.lo[hf];
                    sm.tkmax[buf][hf] = tr.hi[hf];
                }
            }
        }
        if (RP)
            for (int u = tid; u < kToep; u += kThreads) {
                const int delta = (r0 - j0) + (kBlk - 1) - u;
                const uint32_t ad = (uint32_t)(delta < 0 ? -delta : delta);
                const int bk = bucket_of(ad);
                sm.rp[buf][u] = ToepEntry{sm.wp[bk], (float)bk};
            }
    };

    {  // the unit's 128 query and dO rows (rows past the sequence end read as zero)
        const buffer_rsrc qrs = rows_rsrc(qg, n, ld, D), drs = rows_rsrc(dog, n, p.ld_out, D);
        const TileDma<D, kThreads> qdma(tid, ld), ddma(tid, p.ld_out);
#pragma unroll
        for (int half = 0; half < kBlk / kTile; ++half) {
            qdma.issue(qrs, sm.qb + kTile * half * D, (int)((int64_t)(r0 + kTile * half) * ld * 2));
            ddma.issue(drs, sm.dob + kTile * half * D, (int)((int64_t)(r0 + kTile * half) * p.ld_out * 2));
        }
    }
    __syncthreads();
    load_tile(0, ktl.tile(0));
    store_tile(0, ktl.tile(0));
    wait_tile_dma();
    __syncthreads();

    // slot of (row i, key j0 + jj) is u0 + jj - 4g; this wavefront's keys start at jj = k0
    const int k0 = kWaveRows * kh;
    const int u0 = 4 * g - (kWaveRows * wave + lr) + (kBlk - 1) + k0;
    const float alpha2 = -kLog2e * p.alpha;

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1, j0 = ktl.tile(t) * kTile, jk0 = j0 + k0;
        if (t + 1 < ntiles) load_tile(buf ^ 1, ktl.tile(t + 1));
        const int kind = wlo < rhi && jk0 < n ? classify_row_tile(wlo, whi, jk0, n, nc, nh, kWaveRows)
                                              : kEmpty;
        if (kind != kEmpty) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < D / 16; ++ks) {
                s = mfma32(rowop.read(sm.k[buf], kh, ks), rowop.read(sm.qb, wave, ks), s);
                dp = mfma32(rowop.read(sm.v[buf], kh, ks), rowop.read(sm.dob, wave, ks), dp);
            }
            float bpos = 0.0f;
            int pm = 0;
            BiasSpan sp{0, 0, 0, 0, 0}, st{0, 0, 0, 0, 0};
            if (RP) {
                const int jhi = imin(jk0 + kWaveRows, n) - 1;
                sp = bias_span((int64_t)wlo - jhi, (int64_t)(whi - 1) - jk0);
                if (sp.kind == 0) bpos = sm.wp[sp.b_lo];
                else pm = 1;
            }
            TimeSel tb;
            int tm = 0;
            if (RT) {
                const int64_t dlo = timin - uniform64(sm.tkmax[buf][kh]);  // row minus key
                st = bias_span(dlo, timax - uniform64(sm.tkmin[buf][kh]));
                tm = tb.set(st, wave_qfit && uniform_i(sm.fits[buf]), bpos, sm.wtb, dlo >= 0, timax_rel);
            } else tb.set_const(bpos);
            if (pm) epilogue_b_tm<D, 1>(tm, s, dp, sm, buf, k0, u0, g, alpha2, tb, ti, ti64);
            else epilogue_b_tm<D, 0>(tm, s, dp, sm, buf, k0, u0, g, alpha2, tb, ti, ti64);
            if (kind == kPartial) mask_keys_b(dp, g, jk0, lim, dg);
            if (GP || GT) {
                const int pg = !GP ? 0 : (sp.kind == 0 ? 0 : (sp.kind == 1 ? 1 : 2));
                TileSums ts;
                if (pg == 0) ts = grad_sums_tm<D, 0, GP, GT>(tm, dp, sm, buf, k0, u0, g, lane, tb, ti, ti64);
                else if (pg == 1) ts = grad_sums_tm<D, 1, GP, GT>(tm, dp, sm, buf, k0, u0, g, lane, tb, ti, ti64);
                else ts = grad_sums_tm<D, 2, GP, GT>(tm, dp, sm, buf, k0, u0, g, lane, tb, ti, ti64);
                if (GP && pg == 0) run_p_lo.add(sm.hbp, sp.b_lo, ts.sum, lane);
                if (GP && pg == 1) {
                    const float hi_part = ts.mp - (float)sp.b_lo * ts.sum;
                    run_p_lo.add(sm.hbp, sp.b_lo, ts.sum - hi_part, lane);
                    run_p_hi.add(sm.hbp, sp.b_hi, hi_part, lane);
                }
                if (GT && tm == 0) run_t_lo.add(&sm.hbt[0][0], st.b_lo, ts.sum, lane, 32);
                if (GT && tm == 1) {
                    run_t_lo.add(&sm.hbt[0][0], st.b_lo, ts.sum - ts.th, lane, 32);
                    run_t_hi.add(&sm.hbt[0][0], st.b_hi, ts.th, lane, 32);
                }
                if (GT && tm == 4) {
                    run_t_lo.add(&sm.hbt[0][0], st.b_lo, ts.sum - ts.th, lane, 32);
                    run_t_mid.add(&sm.hbt[0][0], st.b_lo + 1, ts.th - ts.th2, lane, 32);
                    run_t_hi.add(&sm.hbt[0][0], st.b_hi, ts.th2, lane, 32);
                }
            }
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                float td[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) td[x] = dp[8 * sl + x];
                const bf16x8 db8 = pack8(td);
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
                    dqt[db] = mfma32(trop.read(sm.k[buf], 2 * kh + sl, db), db8, dqt[db]);
            }
        }
        if (t + 1 < ntiles) store_tile(buf ^ 1, ktl.tile(t + 1));
        wait_tile_dma();
        __syncthreads();
    }

    bf16* dqg = static_cast<bf16*>(p.dq) + (tok0 + i) * p.ld_grad + h * D;
    GateRow<D> gq;
    if (p.gate_delta != 0 && row_ok && kh == 0) gq.load(dqg, g, p.gate_delta);
    // add the second key half's partial dQ into the first's through the idle K and V tile
    // buffers (adjacent), laid out [row group][db][element][lane]
    static_assert(sizeof(sm.k) + sizeof(sm.v) >= 4 * (D / 32) * 16 * 64 * sizeof(float),
                  "reduction buffer");
    {
        float* mine = reinterpret_cast<float*>(&sm.k[0][0]) + ((size_t)wave * (D / 32) * 16) * 64 + lane;
        if (kh == 1)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) mine[(db * 16 + e) * 64] = dqt[db][e];
        __syncthreads();
        if (kh == 0)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int e = 0; e < 16; ++e) dqt[db][e] += mine[(db * 16 + e) * 64];
    }

    if (row_ok && kh == 0) {
        const float sq = p.alpha * p.inv_n;
        store_grad_row<D>(dqg, dqt, g, sq, p.gate_delta, gq);
    }
    if (GP || GT) {
        if (GP) { run_p_lo.add(sm.hbp, -2, 0.0f, lane); run_p_hi.add(sm.hbp, -2, 0.0f, lane); }  // flush
        if (GT) {
            run_t_lo.add(&sm.hbt[0][0], -2, 0.0f, lane, 32);
            run_t_mid.add(&sm.hbt[0][0], -2, 0.0f, lane, 32);
            run_t_hi.add(&sm.hbt[0][0], -2, 0.0f, lane, 32);
        }
        __syncthreads();
        for (int b = tid; b < kNumBuckets; b += kThreads) {
            if (GP && sm.hbp[b] != 0.0f) atomicAdd(&p.drab_pos[h * kNumBuckets + b], sm.hbp[b] * p.inv_n);
            if (GT) {
                // sum the 32 columns, starting at a different column per bucket (no bank clashes)
                float v = 0.0f;
#pragma unroll 8
                for (int l = 0; l < 32; ++l) v += sm.hbt[b][(l + b) & 31];
                if (v != 0.0f) atomicAdd(&p.drab_ts[h * kNumBuckets + b], v * p.inv_n);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// pass B with stored dS: dQ = sum_j dS_ij k_j
// ---------------------------------------------------------------------------------------------
// The dK/dV pass has written dS * N for every pair it visits (AttnParams::ds, rows = keys) and
// summed the bias-table gradients, so per key tile this pass only copies the K rows and the
// 64 x 256 dS block of its rows into LDS and runs dQ^T += K^T dS^T.  With so little arithmetic
// per tile the copies set the pace: a ring of kDqStages tiles keeps kDqStages - 1 of them in
// flight.  Units of 256 query rows (the plan's dQ list), one 32-row group per wavefront (eight),
// every wavefront over all 64 keys of each tile: no partial sums to combine at the end, and each
// K tile copied serves 256 rows.
constexpr int kDqRows = 8 * kWaveRows;
constexpr int kDqStages = 3;

// Copies the 64 x 128 dS block of one key tile and 128 consecutive query rows into an LDS tile
// laid out like a 128-column operand tile (TileDma<kBlk>): its columns 0..63 are the 64-query
// chunk of the rows' first query tile and 64..127 the next chunk (two consecutive chunks of the
// tile's key block, geometry.h); the tile's 64 keys are rows 64 * (key tile & 1) .. + 63 of
// both chunks (row_bytes adds that offset).
template <int THREADS>
struct DsPairDma {
    static constexpr int C = kBlk / 8;  // 16-byte chunks per LDS row
    static constexpr int W = THREADS / 64;
    static constexpr int N = C / W;
    int off[N];
    int wave;
    __device__ __forceinline__ explicit DsPairDma(int tid) {
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int pos = (u * W + wave) * 64 + lane;
            const int row = pos / C, c = (pos % C) ^ tile_swz<kBlk>(row);
            off[u] = ((c >> 3) * kDsChunk + row * kTile + 8 * (c & 7)) * 2;
        }
    }
    __device__ __forceinline__ void issue_asm(i32x4 rs, bf16* tile, int row_bytes) const {
#pragma unroll
        for (int u = 0; u < N; ++u)
            copy16_lds_asm(rs, lds_addr(tile + (u * W + wave) * 512), off[u] + row_bytes);
    }
};

template <int D>
struct SmemC {
    alignas(16) bf16 k[kDqStages][kTile * D];      // swizzled tiles (tile_off)
    bf16 ds[kDqStages][2][kTile * kBlk];           // dS^T rows j0 .. j0 + 63, per 128-row half
};

template <int D>
__global__ __launch_bounds__(kThreadsA, 1) void bwd_dq_stored_kernel(const AttnParams p) {
    constexpr int kThreads = kThreadsA;
    __shared__ __attribute__((aligned(16))) SmemC<D> sm;
    static_assert(sizeof(SmemC<D>) <= 160 * 1024, "LDS");

    if (blockIdx.x == 0)  // the bias-table gradients the dK/dV pass summed, to the outputs
        for (int e = threadIdx.x; e < p.heads * kNumBuckets; e += kThreads) {
            if (p.drab_pos && p.gpos && p.drab_pos != p.gpos) p.drab_pos[e] = p.gpos[e];
            if (p.drab_ts && p.gts && p.drab_ts != p.gts) p.drab_ts[e] = p.gts[e];
        }
    const WorkUnit wu = p.units[blockIdx.x];
    const SeqInfo si = p.seqs[wu.seq];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lr = lane & 31;
    const int wave = uniform_i(tid >> 6), hf = wave >> 2;  // row group; 128-row half
    const int n = si.n, nc = si.nc, nh = si.nh, r0 = wu.row0, h = wu.head;
    const int64_t tok0 = si.start, ld = p.ld_in;
    const bf16* __restrict__ kg = static_cast<const bf16*>(p.k) + tok0 * ld + h * D;

    const int rhi = imin(r0 + kDqRows, n);
    const KeyTiles ktl = key_tiles_for_rows(r0, rhi, nc, nh);
    const int ntiles = ktl.count();
    const int wlo = r0 + kWaveRows * wave, whi = imin(wlo + kWaveRows, rhi);
    const int i = wlo + lr;
    const bool row_ok = i < rhi;
    int lim = -1, dg = -1;
    if (row_ok) {
        if (i < nh) lim = imax(i, nc - 1);
        else { lim = nh - 1; dg = i; }
    }
    f32x16 dqt[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqt[db] = f32x16{};

    const bf16* dss = static_cast<const bf16*>(p.ds) + p.ds_off[wu.seq];  // the sequence's chunks
    // byte size as rows_rsrc computes it (rows past the end read as zero)
    const i32x4 krs = rsrc_words(kg, n > 0 ? ((int64_t)(n - 1) * ld + D) * 2 : 0);
    const TileDma<D, kThreads> kdma(tid, ld);
    const DsPairDma<kThreads> dsdma(tid);
    const TrOperand<D> trop(lane);
    const TrBlock<kBlk> dsop(lane, wave & 3);

    // The copies of list entry t form a group (its K rows and both halves' dS); groups are issued
    // in order, every group with the same number of copies: a half whose 128 rows have no chunks
    // in the tile's key block (none of them sees the block) copies from an empty range, which
    // reads zeros, and its wavefronts skip the tile.
    constexpr int kPerTile = TileDma<D, kThreads>::N + 2 * DsPairDma<kThreads>::N;
    static_assert(kPerTile < 64, "vmcnt");
    // first chunk of the tile's key block for this head and the block's chunk count, kept while
    // the list walks the blocks in order (chunks_before(kb + 1) = chunks_before(kb) + chunks(kb))
    int kb_at = -2, nch_at = 0, q0_at = 0;
    int64_t head_at = 0, cb_at = 0;
    auto issue_group = [&](int t) {
        const int kt = ktl.tile(t), j0 = kt * kTile, kb = kt >> 1;
        if (kb != kb_at) {
            cb_at = kb == kb_at + 1 ? cb_at + nch_at : ds_chunks_before(kb, n, nc, nh);
            kb_at = kb;
            nch_at = ds_chunks(kb, n, nc, nh);
            q0_at = ds_first_qtile(kb, nc);
            head_at = (int64_t)kDsChunk * ((int64_t)p.heads * cb_at + (int64_t)h * nch_at);
        }
        kdma.issue_asm(krs, sm.k[t % kDqStages], (int)((int64_t)j0 * ld * 2));
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int c = (r0 + kBlk * half) / kTile - q0_at;  // the half's first chunk
            const bool has = c >= 0 && c + 2 <= nch_at;
            dsdma.issue_asm(rsrc_words(dss + (has ? head_at + (int64_t)kDsChunk * c : 0), has ? 2 * kDsChunk * 2 : 0),
                            sm.ds[t % kDqStages][half], (kt & 1) * kTile * kTile * 2);
        }
    };
    // waits for this thread's copies of group t, with group t + 1 still in flight
    auto wait_group = [&](int t) {
        if (t + 1 < ntiles) wait_vmcnt<kPerTile>();
        else wait_vmcnt<0>();
    };
    static_assert(kDqStages == 3, "wait_group covers one later group");

    for (int t = 0; t < kDqStages - 1 && t < ntiles; ++t) issue_group(t);

    for (int t = 0; t < ntiles; ++t) {
        const int st = t % kDqStages, jk0 = ktl.tile(t) * kTile;
        wait_group(t);  // this thread's copies of entry t have landed
        lds_barrier();  // everyone's; entry t - 1 is done with
        if (t + kDqStages - 1 < ntiles) issue_group(t + kDqStages - 1);
        const int kind = wlo < rhi && jk0 < n ? classify_row_tile(wlo, whi, jk0, n, nc, nh, kTile) : kEmpty;
        if (kind == kEmpty) continue;
        bf16x8 b8[4];  // dS (times N) of keys jk0 + 16sl + key(k) for this lane's row
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) b8[sl] = dsop.read(sm.ds[st][hf], sl);
        if (kind == kPartial) {  // entries the dK/dV pass did not write for this row
#pragma unroll
            for (int x2 = 0; x2 < 2; ++x2) {
                f32x16 dp;
#pragma unroll
                for (int x = 0; x < 16; ++x) dp[x] = (float)b8[2 * x2 + (x >> 3)][x & 7];
                mask_keys_b(dp, g, jk0 + 32 * x2, lim, dg);
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    float td[8];
#pragma unroll
                    for (int x = 0; x < 8; ++x) td[x] = dp[8 * sl + x];
                    b8[2 * x2 + sl] = pack8(td);
                }
            }
        }
#pragma unroll
        for (int sl = 0; sl < 4; ++sl)
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                dqt[db] = mfma32(trop.read(sm.k[st], sl, db), b8[sl], dqt[db]);
    }

    if (row_ok) {
        bf16* dqg = static_cast<bf16*>(p.dq) + (tok0 + i) * p.ld_grad + h * D;
        GateRow<D> gq;
        if (p.gate_delta != 0) gq.load(dqg, g, p.gate_delta);
        store_grad_row<D>(dqg, dqt, g, p.alpha * p.inv_n, p.gate_delta, gq);
    }
}

// ---------------------------------------------------------------------------------------------
// fp32 path: one thread per row (dQ) or per key (dK, dV)
// ---------------------------------------------------------------------------------------------

constexpr int kF32 = 64;

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = imax(v, __shfl_xor(v, m));
    return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = imin(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float bias_f32(const float* wp, const float* wt, bool rp, bool rt,
                                          int i, int j, int64_t ti, int64_t tj) {
    float b = 0.0f;
    if (rp) b += wp[bucket_of((uint32_t)(i > j ? i - j : j - i))];
    if (rt) b += wt[bucket_class(absdiff_sat(ti, tj))];
    return b;
}

template <int D>
__global__ __launch_bounds__(kF32) void bwd_dq_f32_kernel(const AttnParams p) {
    __shared__ float wp[kNumBuckets], wt[kNumClasses], hp[kNumClasses], ht[kNumClasses];
    const WorkUnit wu = p.units[blockIdx.x];
    const SeqInfo si = p.seqs[wu.seq];
    const int n = si.n, nc = si.nc, nh = si.nh, h = wu.head;
    const int64_t tok0 = si.start, ld = p.ld_in;
    const bool rp = p.rab_pos != nullptr, rt = p.rab_ts != nullptr;
    const bool gp = rp && p.drab_pos, gt = rt && p.drab_ts;
    for (int e = threadIdx.x; e < kNumClasses; e += kF32) {
        hp[e] = 0.0f;
        ht[e] = 0.0f;
        if (rt) wt[e] = p.rab_ts[h * kNumBuckets + bucket_of_class(e)];
        if (rp && e < kNumBuckets) wp[e] = p.rab_pos[h * kNumBuckets + e];
    }
    __syncthreads();
    const int i = wu.row0 + threadIdx.x;
    const bool row_ok = i < n;
    int lim = -1, dg = -1;
    if (row_ok) {
        if (i < nh) lim = imax(i, nc - 1);
        else { lim = nh - 1; dg = i; }
    }
    const float* qg = static_cast<const float*>(p.q) + tok0 * ld + h * D;
    const float* kg = static_cast<const float*>(p.k) + tok0 * ld + h * D;
    const float* vg = static_cast<const float*>(p.v) + tok0 * ld + h * D;
    const float* dog = static_cast<const float*>(p.dout) + tok0 * p.ld_out + h * D;
    float q[D], dO[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        q[c] = row_ok ? qg[(int64_t)i * ld + c] : 0.0f;
        dO[c] = row_ok ? dog[(int64_t)i * p.ld_out + c] : 0.0f;
        acc[c] = 0.0f;
    }
    const int64_t ti = (rt && row_ok) ? p.ts[tok0 + i] : 0;
    const int jend = wave_max(imax(lim, dg)) + 1;
    for (int j = 0; j < jend; ++j) {
        const bool vis = j <= lim || j == dg;
        if (!__any(vis)) continue;
        float dot = 0.0f, dpv = 0.0f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            dot = fmaf(q[c], kg[(int64_t)j * ld + c], dot);
            dpv = fmaf(dO[c], vg[(int64_t)j * ld + c], dpv);
        }
        const int64_t tj = (rt && vis) ? p.ts[tok0 + j] : 0;
        const float x = fmaf(p.alpha, dot, vis ? bias_f32(wp, wt, rp, rt, i, j, ti, tj) : 0.0f);
        const float sg = 1.0f / (1.0f + expf(-x));
        const float ds = vis ? dpv * sg * (1.0f + x * (1.0f - sg)) : 0.0f;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] = fmaf(ds, kg[(int64_t)j * ld + c], acc[c]);
        if (vis && gp) atomicAdd(&hp[bucket_class((uint32_t)(i > j ? i - j : j - i))], ds);
        if (vis && gt) atomicAdd(&ht[bucket_class(absdiff_sat(ti, tj))], ds);
    }
    if (row_ok) {
        float* dqg = static_cast<float*>(p.dq) + (tok0 + i) * p.ld_grad + h * D;
#pragma unroll
        for (int c = 0; c < D; ++c) dqg[c] = acc[c] * p.alpha * p.inv_n;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kNumClasses; e += kF32) {
        const int b = bucket_of_class(e);
        if (gp && hp[e] != 0.0f) atomicAdd(&p.drab_pos[h * kNumBuckets + b], hp[e] * p.inv_n);
        if (gt && ht[e] != 0.0f) atomicAdd(&p.drab_ts[h * kNumBuckets + b], ht[e] * p.inv_n);
    }
}

template <int D>
__global__ __launch_bounds__(kF32) void bwd_dkdv_f32_kernel(const AttnParams p) {
    __shared__ float wp[kNumBuckets], wt[kNumClasses];
    const WorkUnit wu = p.units[blockIdx.x];
    const SeqInfo si = p.seqs[wu.seq];
    const int n = si.n, nc = si.nc, nh = si.nh, h = wu.head;
    const int64_t tok0 = si.start, ld = p.ld_in;
    const bool rp = p.rab_pos != nullptr, rt = p.rab_ts != nullptr;
    for (int e = threadIdx.x; e < kNumClasses; e += kF32) {
        if (rt) wt[e] = p.rab_ts[h * kNumBuckets + bucket_of_class(e)];
        if (rp && e < kNumBuckets) wp[e] = p.rab_pos[h * kNumBuckets + e];
    }
    __syncthreads();
    const int j = wu.row0 + threadIdx.x;
    const bool key_ok = j < n;
    int lo = 1, hi = 0;
    if (key_ok) {
        if (j < nc) { lo = 0; hi = n - 1; }
        else if (j < nh) { lo = j; hi = n - 1; }
        else { lo = j; hi = j; }
    }
    const float* qg = static_cast<const float*>(p.q) + tok0 * ld + h * D;
    const float* kg = static_cast<const float*>(p.k) + tok0 * ld + h * D;
    const float* vg = static_cast<const float*>(p.v) + tok0 * ld + h * D;
    const float* dog = static_cast<const float*>(p.dout) + tok0 * p.ld_out + h * D;
    float kk[D], vv[D], gk[D], gv[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        kk[c] = key_ok ? kg[(int64_t)j * ld + c] : 0.0f;
        vv[c] = key_ok ? vg[(int64_t)j * ld + c] : 0.0f;
        gk[c] = 0.0f;
        gv[c] = 0.0f;
    }
    const int64_t tj = (rt && key_ok) ? p.ts[tok0 + j] : 0;
    const int ibeg = wave_min(key_ok ? lo : 0x7fffffff);
    const int iend = wave_max(key_ok ? hi : -1) + 1;
    for (int i = ibeg; i < iend; ++i) {
        const bool vis = key_ok && i >= lo && i <= hi;
        if (!__any(vis)) continue;
        float dot = 0.0f, dpv = 0.0f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            dot = fmaf(qg[(int64_t)i * ld + c], kk[c], dot);
            dpv = fmaf(dog[(int64_t)i * p.ld_out + c], vv[c], dpv);
        }
        const int64_t ti = (rt && vis) ? p.ts[tok0 + i] : 0;
        const float x = fmaf(p.alpha, dot, vis ? bias_f32(wp, wt, rp, rt, i, j, ti, tj) : 0.0f);
        const float sg = 1.0f / (1.0f + expf(-x));
        const float pw = vis ? x * sg : 0.0f;
        const float ds = vis ? dpv * sg * (1.0f + x * (1.0f - sg)) : 0.0f;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            gv[c] = fmaf(pw, dog[(int64_t)i * p.ld_out + c], gv[c]);
            gk[c] = fmaf(ds, qg[(int64_t)i * ld + c], gk[c]);
        }
    }
    if (key_ok) {
        float* dkg = static_cast<float*>(p.dk) + (tok0 + j) * p.ld_grad + h * D;
        float* dvg = static_cast<float*>(p.dv) + (tok0 + j) * p.ld_grad + h * D;
#pragma unroll
        for (int c = 0; c < D; ++c) {
            dkg[c] = gk[c] * p.alpha * p.inv_n;
            dvg[c] = gv[c] * p.inv_n;
        }
    }
}

__global__ void zero_f32_kernel(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// Up to four buffers cleared by one launch: blockIdx.y picks the buffer, each block-thread
// strides over it.
struct ZeroList {
    float* p[4];
    int64_t n[4];
};
__global__ void zero_f32_list_kernel(const ZeroList z) {
    float* p = z.p[blockIdx.y];
    const int64_t n = z.n[blockIdx.y];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
}

// The modes pass of the stored-dS backward: for each (sequence, 128-key block) -- the head-0
// units of the dK/dV unit list, every heads-th entry (the plan lists a block's heads one after
// another, in head order); the records do not depend on the head -- the mode record of every
// (query tile, wavefront) the dK/dV pass visits, and the times of the block's own rows relative to
// the sequence's first time.  Eight wavefronts take the tiles round robin; each loads the
// timestamps of up to eight of its tiles at once (one load latency per batch), takes their time
// ranges (DPP, one tile after another), and then all 64 lanes write the batch's records (lane
// 8 b + r: tile b, record r).
constexpr int kModesThreads = 512;
template <bool RP, bool RT>
__global__ __launch_bounds__(kModesThreads) void bwd_modes_kernel(const AttnParams p) {
    __shared__ int64_t kmin[4], kmax[4];
    __shared__ uint32_t kmaxr[4];
    __shared__ int kfit[4];
    constexpr int kBatch = 8;
    __shared__ int64_t qlo_s[kModesThreads / 64][kBatch][2], qhi_s[kModesThreads / 64][kBatch][2];
    __shared__ int qfit_s[kModesThreads / 64][kBatch];
    if (blockIdx.x == 0) {  // the bias-table gradient sums of the dK/dV pass start from zero
        for (int e = threadIdx.x; e < p.heads * kNumBuckets; e += kModesThreads) {
            if (p.gpos) p.gpos[e] = 0.0f;
            if (p.gts) p.gts[e] = 0.0f;
        }
    }
    const WorkUnit wu = p.units[(int64_t)blockIdx.x * p.heads];
    if (wu.head != 0) return;  // not a block's first entry: nothing to do (uniform)
    const SeqInfo si = p.seqs[wu.seq];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kWaves = kModesThreads / 64;
    const int n = si.n, nc = si.nc, nh = si.nh, k0 = wu.row0;
    const int64_t tok0 = si.start;
    const int khi = imin(k0 + kBlk, n);
    int qlo, qhi;
    rows_for_keys(k0, khi, n, nc, nh, &qlo, &qhi);
    const int tfirst = qlo / kTile, ntiles = cdiv(qhi, kTile) - tfirst;
    const int64_t tbase = RT ? p.ts[tok0] : 0;
    if (RT && wave < 4) {
        // key group `wave`: keys k0 + 32 wave + (lane % 32), as the dK/dV pass reads them
        const int j = k0 + kWaveRows * wave + (lane & 31);
        const bool key_ok = j < khi;
        const int64_t t = key_ok ? p.ts[tok0 + j] : tbase;
        const bool fit = __all(rel_time_fits(t, tbase));
        int64_t lo, hi;
        wave_time_minmax(t, key_ok, tbase, lo, hi);
        if (lane == 0) {
            kmin[wave] = lo;
            kmax[wave] = hi;
            kmaxr[wave] = rel_time_u32(hi, tbase);
            kfit[wave] = fit ? 1 : 0;
        }
    }
    if (RT)  // every row lies in exactly one key block
        for (int r = tid; r < kBlk; r += kModesThreads)
            if (k0 + r < n) p.tq_rel[tok0 + k0 + r] = rel_time_u32(p.ts[tok0 + k0 + r], tbase);
    __syncthreads();
    ModeRec* out = static_cast<ModeRec*>(p.modes) +
                   8 * (p.ds_off[wu.seq] / ((int64_t)kDsChunk * p.heads) +
                        ds_chunks_before(k0 / kBlk, n, nc, nh));
    for (int tb = wave; tb < ntiles; tb += kWaves * kBatch) {  // tiles tb + kWaves * b
        if (RT) {
            int64_t tq[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int i = (tfirst + tb + kWaves * b) * kTile + lane;
                tq[b] = tb + kWaves * b < ntiles && i < n ? p.ts[tok0 + i] : tbase;
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int t = tb + kWaves * b;
                if (t >= ntiles) break;  // wavefront-uniform
                const TimeRange tr = wave_time_range(tq[b], (tfirst + t) * kTile + lane < n, tbase);
                if (lane == 0) {
                    qlo_s[wave][b][0] = tr.lo[0];
                    qlo_s[wave][b][1] = tr.lo[1];
                    qhi_s[wave][b][0] = tr.hi[0];
                    qhi_s[wave][b][1] = tr.hi[1];
                    qfit_s[wave][b] = tr.fit ? 1 : 0;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wavefront's LDS writes
            __builtin_amdgcn_wave_barrier();
        }
        const int b = lane >> 3, r = lane & 7, t = tb + kWaves * b;
        if (t < ntiles) {  // record r (4 hq + w: key group w, query half hq) of tile t
            const int w = r & 3, hq = r >> 2, i0 = (tfirst + t) * kTile;
            const int mk0 = k0 + kWaveRows * w, mk1 = imin(mk0 + kWaveRows, khi);
            const int mq0 = i0 + kWaveRows * hq, mq1 = imin(mq0 + kWaveRows, n) - 1;
            out[8 * t + r] = make_mode_rec(
                RP, RT, mk0, mk1, mq0, mq1, n, nc, nh, kmin[w], kmax[w], kfit[w] != 0, kmaxr[w],
                RT ? qlo_s[wave][b][hq] : 0, RT ? qhi_s[wave][b][hq] : 0, RT && qfit_s[wave][b] != 0);
        }
        __builtin_amdgcn_wave_barrier();  // the batch's ranges are read before the next batch
    }
}

template <int D, bool RP, bool RT>
hipError_t launch_dkdv_t(const AttnParams& p, hipStream_t s) {
    if constexpr (D >= 64)
        if (p.ds) {
            if (!p.modes || (RT && !p.tq_rel)) return hipErrorInvalidValue;
            hipLaunchKernelGGL((bwd_modes_kernel<RP, RT>), dim3(p.num_units / p.heads), dim3(kModesThreads), 0, s, p);
            hipLaunchKernelGGL((bwd_dkdv_kernel<D, RP, RT, true>), dim3(p.num_units), dim3(kThreadsA), 0, s, p);
            return hipGetLastError();
        }
    if (p.ds) return hipErrorInvalidValue;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, RP, RT, false>), dim3(p.num_units), dim3(kThreadsA), 0, s, p);
    return hipGetLastError();
}

template <int D, bool RP, bool RT>
hipError_t launch_dq_t(const AttnParams& p, hipStream_t s) {
    const bool gp = RP && p.drab_pos, gt = RT && p.drab_ts;
    const dim3 grid(p.num_units), block(kThreadsA);
    if (p.ds) {  // stored dS: the dK/dV pass has summed the bias-table gradients
        if constexpr (D >= 64) {
            hipLaunchKernelGGL((bwd_dq_stored_kernel<D>), grid, block, 0, s, p);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    if (gp && gt) hipLaunchKernelGGL((bwd_dq_kernel<D, RP, RT, RP, RT>), grid, block, 0, s, p);
    else if (gp) hipLaunchKernelGGL((bwd_dq_kernel<D, RP, RT, RP, false>), grid, block, 0, s, p);
    else if (gt) hipLaunchKernelGGL((bwd_dq_kernel<D, RP, RT, false, RT>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((bwd_dq_kernel<D, RP, RT, false, false>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <int D, bool DQ>
hipError_t launch_bwd_d(const AttnParams& p, hipStream_t s) {
    const bool rp = p.rab_pos != nullptr, rt = p.rab_ts != nullptr;
    if (rp && rt) return DQ ? launch_dq_t<D, true, true>(p, s) : launch_dkdv_t<D, true, true>(p, s);
    if (rp) return DQ ? launch_dq_t<D, true, false>(p, s) : launch_dkdv_t<D, true, false>(p, s);
    if (rt) return DQ ? launch_dq_t<D, false, true>(p, s) : launch_dkdv_t<D, false, true>(p, s);
    return DQ ? launch_dq_t<D, false, false>(p, s) : launch_dkdv_t<D, false, false>(p, s);
}

template <bool DQ>
hipError_t launch_bwd_bf16(const AttnParams& p, hipStream_t s) {
    if (p.num_units == 0) return hipSuccess;
    switch (p.head_dim) {
        case 32: return launch_bwd_d<32, DQ>(p, s);
        case 64: return launch_bwd_d<64, DQ>(p, s);
        case 128: return launch_bwd_d<128, DQ>(p, s);
    }
    return hipErrorInvalidValue;
}

template <bool DQ>
hipError_t launch_bwd_f32(const AttnParams& p, hipStream_t s) {
    if (p.num_units == 0) return hipSuccess;
    const dim3 grid(p.num_units), block(kF32);
    switch (p.head_dim) {
        case 32:
            if (DQ) hipLaunchKernelGGL(bwd_dq_f32_kernel<32>, grid, block, 0, s, p);
            else hipLaunchKernelGGL(bwd_dkdv_f32_kernel<32>, grid, block, 0, s, p);
            break;
        case 64:
            if (DQ) hipLaunchKernelGGL(bwd_dq_f32_kernel<64>, grid, block, 0, s, p);
            else hipLaunchKernelGGL(bwd_dkdv_f32_kernel<64>, grid, block, 0, s, p);
            break;
        case 128:
            if (DQ) hipLaunchKernelGGL(bwd_dq_f32_kernel<128>, grid, block, 0, s, p);
            else hipLaunchKernelGGL(bwd_dkdv_f32_kernel<128>, grid, block, 0, s, p);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_dkdv_bf16(const AttnParams& p, hipStream_t s) { return launch_bwd_bf16<false>(p, s); }
hipError_t launch_attn_bwd_dq_bf16(const AttnParams& p, hipStream_t s) { return launch_bwd_bf16<true>(p, s); }
hipError_t launch_attn_bwd_dkdv_f32(const AttnParams& p, hipStream_t s) { return launch_bwd_f32<false>(p, s); }
hipError_t launch_attn_bwd_dq_f32(const AttnParams& p, hipStream_t s) { return launch_bwd_f32<true>(p, s); }

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int threads = 256;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((n + threads - 1) / threads)), dim3(threads), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_zero_f32_list(float* const* ptrs, const int64_t* counts, int k, hipStream_t s) {
    ZeroList z{};
    int m = 0;
    int64_t most = 0;
    for (int i = 0; i < k && i < 4; ++i)
        if (ptrs[i] && counts[i] > 0) {
            z.p[m] = ptrs[i];
            z.n[m] = counts[i];
            most = std::max(most, counts[i]);
            ++m;
        }
    if (m == 0) return hipSuccess;
    const int threads = 256;
    const int64_t blocks = std::min<int64_t>((most + threads - 1) / threads, 1024);
    hipLaunchKernelGGL(zero_f32_list_kernel, dim3((unsigned)blocks, (unsigned)m), dim3(threads), 0, s, z);
    return hipGetLastError();
}

}  // namespace hstu
