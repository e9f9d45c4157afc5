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
//   pass A (key-stationary): unit = (sequence, head, 128 keys), 4 wavefronts x 32 keys; visits
//     64-query tiles.  S = Q K^T and dP = dO V^T put one key per lane, which is the B-operand
//     layout for dV^T += dO^T P and dK^T += Q^T dS; Q and dO are staged both row-major (A operands
//     of the first two products) and transposed with renumbered rows (A operands of the last two).
//   pass B (query-stationary): unit = (sequence, head, 128 rows) exactly like the forward;
//     S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T, and the bias-table gradients.
// Bias-gradient sums: along a lane (one query row, keys increasing) the bucket of |i - j| and of
// |t_i - t_j| changes rarely, so each lane keeps a running (class, sum) pair and adds it to a
// per-unit LDS histogram only when the class changes; the histogram is flushed to the global
// table with one atomic add per non-zero class at the end of the unit.
#include "device_common.h"
#include "kernels.h"

namespace hstu {
namespace {

constexpr int kThreads = 256;
constexpr int kBlk = 4 * kWaveRows;      // 128 keys (pass A) or rows (pass B) per unit
constexpr int kTile = 64;                // queries (pass A) or keys (pass B) per tile
constexpr int kToep = kBlk + kTile - 1;  // 191 distinct i - j per (unit, tile)
constexpr int kHist = kNumClasses + 1;   // + one slot that absorbs the initial empty run

struct ToepEntry {
    float bias;
    uint32_t cls;
};

__device__ __forceinline__ void tile_store_rowmajor_and_t(bf16* rowm, int rp_pitch, bf16* trans,
                                                          int tp_pitch, const bf16x8 (&r)[4],
                                                          int grp, int ch) {
    // r[kk] = row 4*grp + kk, channels 8*ch .. 8*ch+7
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        *reinterpret_cast<bf16x8*>(&rowm[(4 * grp + kk) * rp_pitch + 8 * ch]) = r[kk];
    const int col = perm_key(4 * grp);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        bf16x4 w = {r[0][e], r[1][e], r[2][e], r[3][e]};
        *reinterpret_cast<bf16x4*>(&trans[(8 * ch + e) * tp_pitch + col]) = w;
    }
}

// ---------------------------------------------------------------------------------------------
// pass A: dK, dV
// ---------------------------------------------------------------------------------------------

template <int D>
struct SmemA {
    static constexpr int RP = D + 8;     // row-major pitch
    static constexpr int TP = kTile + 8; // transposed pitch
    bf16 q[2][kTile * RP];
    bf16 dout[2][kTile * RP];
    bf16 qt[2][D * TP];
    bf16 doutt[2][D * TP];
    float rp[2][kToep + 1];
    uint32_t tq[2][kTile];
    int64_t tq64[2][kTile];
    int fits[2];
    float wt[kNumClasses];
    float wp[kNumBuckets];
};

template <int D, bool RP, bool RT>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(const AttnParams p) {
    constexpr int RPt = SmemA<D>::RP, TP = SmemA<D>::TP;
    constexpr int KCH = D / 8;
    constexpr int ITEMS = (kTile / 4) * KCH;  // (4 rows x 8 channels) items per tensor
    __shared__ __attribute__((aligned(16))) SmemA<D> sm;

    const WorkUnit wu = p.units[blockIdx.x];
    const SeqInfo si = p.seqs[wu.seq];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, lr = lane & 31;
    const int n = si.n, nc = si.nc, nh = si.nh, k0 = wu.row0, h = wu.head;
    const int64_t tok0 = si.start, ld = p.ld_in;
    const bf16* __restrict__ qg = static_cast<const bf16*>(p.q) + tok0 * ld + h * D;
    const bf16* __restrict__ kg = static_cast<const bf16*>(p.k) + tok0 * ld + h * D;
    const bf16* __restrict__ vg = static_cast<const bf16*>(p.v) + tok0 * ld + h * D;
    const bf16* __restrict__ dog = static_cast<const bf16*>(p.dout) + tok0 * p.ld_out + h * D;

    if (RP)
        for (int e = tid; e < kNumBuckets; e += kThreads) sm.wp[e] = p.rab_pos[h * kNumBuckets + e];
    if (RT)
        for (int e = tid; e < kNumClasses; e += kThreads)
            sm.wt[e] = p.rab_ts[h * kNumBuckets + bucket_of_class(e)];
    const int64_t tbase = RT ? p.ts[tok0] : 0;

    const int khi = imin(k0 + kBlk, n);
    int qlo, qhi;
    rows_for_keys(k0, khi, n, nc, nh, &qlo, &qhi);
    const int tfirst = qlo / kTile, ntiles = cdiv(qhi, kTile) - tfirst;

    const int wk0 = k0 + kWaveRows * wave, wk1 = imin(wk0 + kWaveRows, khi);
    const int j = wk0 + lr;
    const bool key_ok = j < khi;
    int lo = 1, hi = 0;  // rows that see key j: lo <= i <= hi
    if (key_ok) {
        if (j < nc) { lo = 0; hi = n - 1; }
        else if (j < nh) { lo = j; hi = n - 1; }
        else { lo = j; hi = j; }
    }
    bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        kf[ks] = key_ok ? load_bf16x8(kg + (int64_t)j * ld + 16 * ks + 8 * g) : bf16x8{};
        vf[ks] = key_ok ? load_bf16x8(vg + (int64_t)j * ld + 16 * ks + 8 * g) : bf16x8{};
    }
    uint32_t tj = 0;
    int64_t tj64 = 0;
    bool wave_kfit = true;
    if (RT) {
        tj64 = key_ok ? p.ts[tok0 + j] : tbase;
        wave_kfit = __all(rel_time_fits(tj64, tbase));
        tj = rel_time_u32(tj64, tbase);
    }

    f32x16 dvt[D / 32], dkt[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) { dvt[db] = f32x16{}; dkt[db] = f32x16{}; }

    bf16x8 qr[4], dr[4];
    int64_t tqr = 0;
    auto load_tile = [&](int tile) {
        const int i0 = tile * kTile;
        if (tid < ITEMS) {
            const int grp = tid % (kTile / 4), ch = tid / (kTile / 4);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int i = i0 + 4 * grp + kk;
                qr[kk] = i < n ? load_bf16x8(qg + (int64_t)i * ld + 8 * ch) : bf16x8{};
                dr[kk] = i < n ? load_bf16x8(dog + (int64_t)i * p.ld_out + 8 * ch) : bf16x8{};
            }
        }
        if (RT && tid < kTile) {
            const int i = i0 + tid;
            tqr = i < n ? p.ts[tok0 + i] : tbase;
        }
    };
    auto store_tile = [&](int buf, int tile) {
        const int i0 = tile * kTile;
        if (tid < ITEMS) {
            const int grp = tid % (kTile / 4), ch = tid / (kTile / 4);
            tile_store_rowmajor_and_t(sm.q[buf], RPt, sm.qt[buf], TP, qr, grp, ch);
            tile_store_rowmajor_and_t(sm.dout[buf], RPt, sm.doutt[buf], TP, dr, grp, ch);
        }
        if (RT && tid < kTile) {
            sm.tq64[buf][tid] = tqr;
            sm.tq[buf][tid] = rel_time_u32(tqr, tbase);
            const bool all_fit = __all(rel_time_fits(tqr, tbase));
            if (tid == 0) sm.fits[buf] = all_fit ? 1 : 0;
        }
        if (RP)
            for (int u = tid; u < kToep; u += kThreads) {
                const int delta = (i0 - k0) - (kBlk - 1) + u;  // i - j for slot u
                sm.rp[buf][u] = sm.wp[bucket_of((uint32_t)(delta < 0 ? -delta : delta))];
            }
    };

    __syncthreads();
    load_tile(tfirst);
    store_tile(0, tfirst);
    if (ntiles > 1) load_tile(tfirst + 1);
    __syncthreads();

    // slot of (query i0 + ii, key j) is u0 + ii - 4g with u0 below
    const int u0 = 4 * g - (kWaveRows * wave + lr) + (kBlk - 1);
    const float alpha = p.alpha;

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1, i0 = (tfirst + t) * kTile;
        const int kind = wk0 < khi ? classify_key_tile(wk0, wk1, i0, n, nc, nh) : kEmpty;
        if (kind != kEmpty) {
            f32x16 s[2], dp[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                s[qb] = f32x16{};
                dp[qb] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    const int off = (32 * qb + lr) * RPt + 16 * ks + 8 * g;
                    bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sm.q[buf][off]);
                    bf16x8 ad = *reinterpret_cast<const bf16x8*>(&sm.dout[buf][off]);
                    s[qb] = mfma32(aq, kf[ks], s[qb]);
                    dp[qb] = mfma32(ad, vf[ks], dp[qb]);
                }
            }
            const bool fit = !RT || (wave_kfit && sm.fits[buf]);
            const bool masked = kind == kPartial;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ii = 32 * qb + 8 * r + 4 * g;
                    u32x4 tq4;
                    if (RT) tq4 = *reinterpret_cast<const u32x4*>(&sm.tq[buf][ii]);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int e = 4 * r + c;
                        float bias = 0.0f;
                        if (RP) bias += sm.rp[buf][u0 + 32 * qb + 8 * r + c];
                        if (RT) {
                            uint32_t dt = fit ? absdiff_u32(tj, tq4[c])
                                              : absdiff_sat(tj64, sm.tq64[buf][ii + c]);
                            bias += sm.wt[bucket_class(dt)];
                        }
                        const float x = fmaf(alpha, s[qb][e], bias);
                        const float sg = fast_sigmoid(x);
                        float pv = x * sg;
                        float dsv = dp[qb][e] * sg * fmaf(x, 1.0f - sg, 1.0f);
                        if (masked) {
                            const int i = i0 + ii + c;
                            const bool vis = i >= lo && i <= hi;
                            pv = vis ? pv : 0.0f;
                            dsv = vis ? dsv : 0.0f;
                        }
                        s[qb][e] = pv;
                        dp[qb][e] = dsv;
                    }
                }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                float tp[8], td[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    tp[x] = s[st >> 1][8 * (st & 1) + x];
                    td[x] = dp[st >> 1][8 * (st & 1) + x];
                }
                const bf16x8 pb = pack8(tp), db8 = pack8(td);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const int off = (32 * db + lr) * TP + 16 * st + 8 * g;
                    bf16x8 ado = *reinterpret_cast<const bf16x8*>(&sm.doutt[buf][off]);
                    bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sm.qt[buf][off]);
                    dvt[db] = mfma32(ado, pb, dvt[db]);
                    dkt[db] = mfma32(aq, db8, dkt[db]);
                }
            }
        }
        if (t + 1 < ntiles) store_tile(buf ^ 1, tfirst + t + 1);
        if (t + 2 < ntiles) load_tile(tfirst + t + 2);
        __syncthreads();
    }

    if (key_ok) {
        bf16* dvg = static_cast<bf16*>(p.dv) + (tok0 + j) * p.ld_out + h * D;
        bf16* dkg = static_cast<bf16*>(p.dk) + (tok0 + j) * p.ld_out + h * D;
        const float sk = alpha * p.inv_n;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bf16x4 wv, wk;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    wv[c] = (bf16)(dvt[db][4 * r + c] * p.inv_n);
                    wk[c] = (bf16)(dkt[db][4 * r + c] * sk);
                }
                *reinterpret_cast<bf16x4*>(dvg + 32 * db + 8 * r + 4 * g) = wv;
                *reinterpret_cast<bf16x4*>(dkg + 32 * db + 8 * r + 4 * g) = wk;
            }
    }
}

// ---------------------------------------------------------------------------------------------
// pass B: dQ and the bias-table gradients
// ---------------------------------------------------------------------------------------------

template <int D>
struct SmemB {
    static constexpr int RP = D + 8;
    static constexpr int TP = kTile + 8;
    bf16 k[2][kTile * RP];
    bf16 v[2][kTile * RP];
    bf16 kt[2][D * TP];
    ToepEntry rp[2][kToep + 1];
    uint32_t tk[2][kTile];
    int64_t tk64[2][kTile];
    int fits[2];
    float wt[kNumClasses];
    float wp[kNumBuckets];
    float hp[kHist];
    float ht[kHist];
};

// Adds v to the lane's running (class, sum); on a class change the finished run goes to hist.
__device__ __forceinline__ void run_add(float* hist, uint32_t& cur, float& sum, uint32_t cls,
                                        float v) {
    if (cls != cur) {
        atomicAdd(&hist[cur], sum);
        cur = cls;
        sum = v;
    } else {
        sum += v;
    }
}

template <int D, bool RP, bool RT>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(const AttnParams p) {
    constexpr int RPt = SmemB<D>::RP, TP = SmemB<D>::TP;
    constexpr int KCH = D / 8;
    constexpr int ITEMS = (kTile / 4) * KCH;
    __shared__ __attribute__((aligned(16))) SmemB<D> sm;

    const WorkUnit wu = p.units[blockIdx.x];
    const SeqInfo si = p.seqs[wu.seq];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, lr = lane & 31;
    const int n = si.n, nc = si.nc, nh = si.nh, r0 = wu.row0, h = wu.head;
    const int64_t tok0 = si.start, ld = p.ld_in;
    const bf16* __restrict__ qg = static_cast<const bf16*>(p.q) + tok0 * ld + h * D;
    const bf16* __restrict__ kg = static_cast<const bf16*>(p.k) + tok0 * ld + h * D;
    const bf16* __restrict__ vg = static_cast<const bf16*>(p.v) + tok0 * ld + h * D;
    const bf16* __restrict__ dog = static_cast<const bf16*>(p.dout) + tok0 * p.ld_out + h * D;
    const bool grad_p = RP && p.drab_pos != nullptr, grad_t = RT && p.drab_ts != nullptr;

    if (RP)
        for (int e = tid; e < kNumBuckets; e += kThreads) sm.wp[e] = p.rab_pos[h * kNumBuckets + e];
    if (RT)
        for (int e = tid; e < kNumClasses; e += kThreads)
            sm.wt[e] = p.rab_ts[h * kNumBuckets + bucket_of_class(e)];
    for (int e = tid; e < kHist; e += kThreads) { sm.hp[e] = 0.0f; sm.ht[e] = 0.0f; }
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
    bf16x8 qf[D / 16], dof[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
        qf[ks] = row_ok ? load_bf16x8(qg + (int64_t)i * ld + 16 * ks + 8 * g) : bf16x8{};
        dof[ks] = row_ok ? load_bf16x8(dog + (int64_t)i * p.ld_out + 16 * ks + 8 * g) : bf16x8{};
    }
    uint32_t ti = 0;
    int64_t ti64 = 0;
    bool wave_qfit = true;
    if (RT) {
        ti64 = row_ok ? p.ts[tok0 + i] : tbase;
        wave_qfit = __all(rel_time_fits(ti64, tbase));
        ti = rel_time_u32(ti64, tbase);
    }
    f32x16 dqt[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqt[db] = f32x16{};
    uint32_t cur_p = kNumClasses, cur_t = kNumClasses;
    float sum_p = 0.0f, sum_t = 0.0f;

    bf16x8 kr[4], vr[4];
    int64_t tkr = 0;
    auto load_tile = [&](int tile) {
        const int j0 = tile * kTile;
        if (tid < ITEMS) {
            const int grp = tid % (kTile / 4), ch = tid / (kTile / 4);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int jj = j0 + 4 * grp + kk;
                kr[kk] = jj < n ? load_bf16x8(kg + (int64_t)jj * ld + 8 * ch) : bf16x8{};
                vr[kk] = jj < n ? load_bf16x8(vg + (int64_t)jj * ld + 8 * ch) : bf16x8{};
            }
        }
        if (RT && tid < kTile) {
            const int jj = j0 + tid;
            tkr = jj < n ? p.ts[tok0 + jj] : tbase;
        }
    };
    auto store_tile = [&](int buf, int tile) {
        const int j0 = tile * kTile;
        if (tid < ITEMS) {
            const int grp = tid % (kTile / 4), ch = tid / (kTile / 4);
            tile_store_rowmajor_and_t(sm.k[buf], RPt, sm.kt[buf], TP, kr, grp, ch);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                *reinterpret_cast<bf16x8*>(&sm.v[buf][(4 * grp + kk) * RPt + 8 * ch]) = vr[kk];
        }
        if (RT && tid < kTile) {
            sm.tk64[buf][tid] = tkr;
            sm.tk[buf][tid] = rel_time_u32(tkr, tbase);
            const bool all_fit = __all(rel_time_fits(tkr, tbase));
            if (tid == 0) sm.fits[buf] = all_fit ? 1 : 0;
        }
        if (RP)
            for (int u = tid; u < kToep; u += kThreads) {
                const int delta = (r0 - j0) + (kBlk - 1) - u;
                const uint32_t ad = (uint32_t)(delta < 0 ? -delta : delta);
                sm.rp[buf][u] = ToepEntry{sm.wp[bucket_of(ad)], bucket_class(ad)};
            }
    };

    __syncthreads();
    load_tile(ktl.tile(0));
    store_tile(0, ktl.tile(0));
    if (ntiles > 1) load_tile(ktl.tile(1));
    __syncthreads();

    const int u0 = 4 * g - (kWaveRows * wave + lr) + (kBlk - 1);
    const float alpha = p.alpha;

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1, j0 = ktl.tile(t) * kTile;
        const int kind = wlo < rhi ? classify_row_tile(wlo, whi, j0, n, nc, nh) : kEmpty;
        if (kind != kEmpty) {
            f32x16 s[2], dp[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x16{};
                dp[kb] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks) {
                    const int off = (32 * kb + lr) * RPt + 16 * ks + 8 * g;
                    bf16x8 ak = *reinterpret_cast<const bf16x8*>(&sm.k[buf][off]);
                    bf16x8 av = *reinterpret_cast<const bf16x8*>(&sm.v[buf][off]);
                    s[kb] = mfma32(ak, qf[ks], s[kb]);
                    dp[kb] = mfma32(av, dof[ks], dp[kb]);
                }
            }
            const bool fit = !RT || (wave_qfit && sm.fits[buf]);
            const bool masked = kind == kPartial;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jj = 32 * kb + 8 * r + 4 * g;
                    u32x4 tk4;
                    if (RT) tk4 = *reinterpret_cast<const u32x4*>(&sm.tk[buf][jj]);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int e = 4 * r + c;
                        float bias = 0.0f;
                        uint32_t cls_p = 0, cls_t = 0;
                        if (RP) {
                            const ToepEntry te = sm.rp[buf][u0 + 32 * kb + 8 * r + c];
                            bias += te.bias;
                            cls_p = te.cls;
                        }
                        if (RT) {
                            uint32_t dt = fit ? absdiff_u32(ti, tk4[c])
                                              : absdiff_sat(ti64, sm.tk64[buf][jj + c]);
                            cls_t = bucket_class(dt);
                            bias += sm.wt[cls_t];
                        }
                        const float x = fmaf(alpha, s[kb][e], bias);
                        const float sg = fast_sigmoid(x);
                        float dsv = dp[kb][e] * sg * fmaf(x, 1.0f - sg, 1.0f);
                        bool vis = true;
                        if (masked) {
                            const int jk = j0 + jj + c;
                            vis = jk <= lim || jk == dg;
                            dsv = vis ? dsv : 0.0f;
                        }
                        dp[kb][e] = dsv;
                        if (grad_p) run_add(sm.hp, cur_p, sum_p, vis ? cls_p : cur_p, dsv);
                        if (grad_t) run_add(sm.ht, cur_t, sum_t, vis ? cls_t : cur_t, dsv);
                    }
                }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                float td[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) td[x] = dp[st >> 1][8 * (st & 1) + x];
                const bf16x8 db8 = pack8(td);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    bf16x8 ak = *reinterpret_cast<const bf16x8*>(
                        &sm.kt[buf][(32 * db + lr) * TP + 16 * st + 8 * g]);
                    dqt[db] = mfma32(ak, db8, dqt[db]);
                }
            }
        }
        if (t + 1 < ntiles) store_tile(buf ^ 1, ktl.tile(t + 1));
        if (t + 2 < ntiles) load_tile(ktl.tile(t + 2));
        __syncthreads();
    }

    if (row_ok) {
        bf16* dqg = static_cast<bf16*>(p.dq) + (tok0 + i) * p.ld_out + h * D;
        const float sq = alpha * p.inv_n;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bf16x4 w;
#pragma unroll
                for (int c = 0; c < 4; ++c) w[c] = (bf16)(dqt[db][4 * r + c] * sq);
                *reinterpret_cast<bf16x4*>(dqg + 32 * db + 8 * r + 4 * g) = w;
            }
    }
    if (grad_p || grad_t) {
        if (grad_p) atomicAdd(&sm.hp[cur_p], sum_p);
        if (grad_t) atomicAdd(&sm.ht[cur_t], sum_t);
        __syncthreads();
        for (int e = tid; e < kNumClasses; e += kThreads) {
            const int b = bucket_of_class(e);
            if (grad_p && sm.hp[e] != 0.0f) atomicAdd(&p.drab_pos[h * kNumBuckets + b], sm.hp[e] * p.inv_n);
            if (grad_t && sm.ht[e] != 0.0f) atomicAdd(&p.drab_ts[h * kNumBuckets + b], sm.ht[e] * p.inv_n);
        }
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
        float* dqg = static_cast<float*>(p.dq) + (tok0 + i) * p.ld_out + h * D;
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
        float* dkg = static_cast<float*>(p.dk) + (tok0 + j) * p.ld_out + h * D;
        float* dvg = static_cast<float*>(p.dv) + (tok0 + j) * p.ld_out + h * D;
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

template <int D, bool RP, bool RT>
hipError_t launch_dkdv_t(const AttnParams& p, hipStream_t s) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, RP, RT>), dim3(p.num_units), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int D, bool RP, bool RT>
hipError_t launch_dq_t(const AttnParams& p, hipStream_t s) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, RP, RT>), dim3(p.num_units), dim3(kThreads), 0, s, p);
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

}  // namespace hstu
