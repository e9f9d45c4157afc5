// hstu_api.hip -- host side of the C ABI declared in include/hstu.h: argument validation, the
// cost-balanced work lists (plans), and kernel dispatch.  No device memory is allocated outside
// hstu_plan_create.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <utility>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <new>
#include <vector>

#include "hstu.h"
#include "kernels.h"

using hstu::SeqInfo;
using hstu::WorkUnit;
using hstu::FwdItem;
using hstu::FixItem;
using hstu::CacheSeq;

struct hstu_plan {
    int device = -1;
    bool on_device = false;
    hstu_attn_args_t shape{};  // sizes only; pointer fields are cleared
    int32_t fwd_rows = 0;      // query rows per forward / dQ work unit
    int32_t bwd_keys = 0;      // keys per dK/dV work unit
    int64_t pairs = 0;
    int64_t fwd_tiles = -1;    // computed on first hstu_plan_info (-1: not yet)
    std::vector<SeqInfo> seqs;
    std::vector<WorkUnit> fwd, bwd;
    std::vector<WorkUnit> dqs;   // bf16: 256-row blocks of the stored-dS dQ pass
    std::vector<FwdItem> items;  // bf16 forward launch (row blocks, the longest split by key tiles)
    std::vector<FixItem> fix;
    int32_t item_rows = 128;     // rows per forward item: 128, or 64 (key-half layout)
    int32_t parts = 0;           // partial slots the split items write
    int32_t compute_units = 256;
    bool cached = false;         // candidate scoring against cached history
    std::vector<CacheSeq> cache;
    // stored-dS backward (bf16, head_dim 64 / 128): per-sequence element offsets of the chunked
    // layout (geometry.h), and their total
    std::vector<int64_t> ds_off;
    int64_t ds_elems = 0;
    void* dbuf = nullptr;
    bool pooled = false;  // dbuf from the device's stream-ordered pool (else hipMalloc)
    const SeqInfo* d_seqs = nullptr;
    const WorkUnit* d_fwd = nullptr;
    const WorkUnit* d_bwd = nullptr;
    const WorkUnit* d_dqs = nullptr;
    const FwdItem* d_items = nullptr;
    const FixItem* d_fix = nullptr;
    const CacheSeq* d_cache = nullptr;
    const int64_t* d_ds_off = nullptr;
};

namespace {

size_t elem_size(int32_t dtype) { return dtype == HSTU_BF16 ? 2 : 4; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The bf16 kernels address one sequence's rows of a tensor with 32-bit byte offsets (tiles of 64
// rows may run past the last row).
bool rows_addressable(int32_t max_seqlen, int64_t token_stride) {
    return (int64_t(max_seqlen) + 64) * token_stride * 2 < (int64_t(1) << 31);
}

hstu_status_t check_args(const hstu_attn_args_t* a) {
    if (!a) return HSTU_ERR_NULL_ARG;
    if (a->dtype != HSTU_F32 && a->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
    if (a->head_dim != 32 && a->head_dim != 64 && a->head_dim != 128) return HSTU_ERR_UNSUPPORTED;
    if (a->batch < 0 || a->num_heads < 1 || a->total_tokens < 0 ||
        a->total_tokens >= (int64_t(1) << 31) || a->max_seqlen < 1 || a->num_contexts < 0 ||
        a->reserved != 0 || !std::isfinite(a->alpha))
        return HSTU_ERR_BAD_SHAPE;
    int64_t hd = int64_t(a->num_heads) * a->head_dim;
    if (a->qkv_token_stride != 0 && a->qkv_token_stride < hd) return HSTU_ERR_BAD_SHAPE;
    if (a->qkv_token_stride % 8 != 0) return HSTU_ERR_MISALIGNED;
    if (a->rab_ts && !a->timestamps && a->total_tokens > 0) return HSTU_ERR_NULL_ARG;
    if (a->dtype == HSTU_BF16 && !rows_addressable(a->max_seqlen, a->qkv_token_stride > hd ? a->qkv_token_stride : hd))
        return HSTU_ERR_UNSUPPORTED;
    return HSTU_OK;
}

// The call's sizes must be the plan's.
hstu_status_t check_call(const hstu_plan_t* plan, const hstu_attn_args_t* a) {
    if (!plan) return HSTU_ERR_NULL_ARG;
    hstu_status_t s = check_args(a);
    if (s != HSTU_OK) return s;
    const hstu_attn_args_t& p = plan->shape;
    if (a->dtype != p.dtype || a->batch != p.batch || a->num_heads != p.num_heads ||
        a->head_dim != p.head_dim || a->total_tokens != p.total_tokens ||
        a->max_seqlen != p.max_seqlen || a->num_contexts != p.num_contexts)
        return HSTU_ERR_BAD_SHAPE;
    if (!plan->on_device) return HSTU_ERR_NO_DEVICE_PLAN;
    if (plan->cached) return HSTU_ERR_BAD_SHAPE;
    if ((a->timestamps && !aligned16(a->timestamps)) || (a->rab_pos && !aligned16(a->rab_pos)) ||
        (a->rab_ts && !aligned16(a->rab_ts)))
        return HSTU_ERR_MISALIGNED;
    return HSTU_OK;
}

int64_t visible_pairs(int64_t n, int64_t nc, int64_t nh) {
    // history rows: the first nc see nc keys, row i in [nc, nh) sees i + 1; candidates see nh + 1
    return nc * nc + (nh * (nh + 1) - nc * (nc + 1)) / 2 + (n - nh) * (nh + 1);
}

void sort_longest_first(std::vector<WorkUnit>& u) {
    std::stable_sort(u.begin(), u.end(),
                     [](const WorkUnit& a, const WorkUnit& b) { return a.cost > b.cost; });
}

// Forward work items.  The forward's time is at least that of its longest row block, whose key
// tiles run one after another in one workgroup; when a row block costs more than twice the
// average load of a workgroup slot (two per compute unit), its key-tile list is cut into
// near-equal pieces of at most that size (but no fewer than kMinSplit tiles) that run as separate
// items.  (Below twice the average, the fix-up pass and the pieces' extra prologues cost more
// than the shorter critical path saves.)
// Because the output is a plain sum over keys (no softmax normalisation), the pieces' fp32
// partial outputs just add up; a fix-up pass sums them.
//
// Launch order.  Workgroups are dispatched to the 8 XCDs round robin (workgroup i to XCD i % 8),
// and each XCD has its own L2.  All items of one (sequence, head) read the same K and V, so they
// are given indices of one residue mod 8, consecutively within it: they run on one XCD at about
// the same time and all but the first find K and V in that XCD's L2.  Groups are taken longest
// item first and each goes to the residue with the fewest items so far (greedy list scheduling
// by group); within a group, longest first.
constexpr int kMinSplit = 4;
constexpr int kXcds = 8;

template <class Item>
void order_for_xcds(std::vector<Item>& items) {
    std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) {
        return a.cost > b.cost;
    });
    // groups: runs of a stable sort by (sequence, head) of the positions in cost order, so each
    // group keeps its members longest first and starts at its longest item's position
    const size_t n = items.size();
    std::vector<size_t> pos(n);
    for (size_t i = 0; i < n; ++i) pos[i] = i;
    std::stable_sort(pos.begin(), pos.end(), [&](size_t a, size_t b) {
        const Item& x = items[a];
        const Item& y = items[b];
        return x.seq != y.seq ? x.seq < y.seq : x.head < y.head;
    });
    std::vector<std::pair<size_t, size_t>> runs;  // [begin, end) in pos
    for (size_t i = 0; i < n;) {
        size_t e = i + 1;
        while (e < n && items[pos[e]].seq == items[pos[i]].seq && items[pos[e]].head == items[pos[i]].head)
            ++e;
        runs.emplace_back(i, e);
        i = e;
    }
    // groups in order of their longest item
    std::sort(runs.begin(), runs.end(), [&](const std::pair<size_t, size_t>& a,
                                            const std::pair<size_t, size_t>& b) {
        return pos[a.first] < pos[b.first];
    });
    std::vector<std::vector<Item>> queues(kXcds);
    for (const auto& run : runs) {
        int best = 0;
        for (int r = 1; r < kXcds; ++r)
            if (queues[r].size() < queues[best].size()) best = r;
        for (size_t i = run.first; i < run.second; ++i) queues[best].push_back(items[pos[i]]);
    }
    items.clear();
    for (size_t k = 0;; ++k) {
        bool any = false;
        for (int r = 0; r < kXcds; ++r)
            if (k < queues[r].size()) {
                items.push_back(queues[r][k]);
                any = true;
            }
        if (!any) break;
    }
}

// Rows per item: the forward's items are the plan's 128-row blocks, unless those blocks fill at
// most half of the workgroup slots (small batches) or the plan scores candidates: then 64-row
// blocks, run in the key-half layout (two row groups x two key halves per workgroup), which
// halves the work per wavefront and tile where the GPU would otherwise idle.
void build_fwd_items(hstu_plan_t* plan, int compute_units) {
    const int64_t slots = 2 * int64_t(compute_units);
    std::vector<WorkUnit> half;  // 64-row blocks of the regular plan, when used
    const std::vector<WorkUnit>* units = &plan->fwd;
    plan->item_rows = plan->cached ? 2 * hstu::kWaveRows : 4 * hstu::kWaveRows;
    if (!plan->cached && 2 * int64_t(plan->fwd.size()) <= slots) {
        plan->item_rows = 2 * hstu::kWaveRows;
        for (const WorkUnit& u : plan->fwd) {
            const SeqInfo& si = plan->seqs[u.seq];
            for (int r0 = u.row0; r0 < std::min(u.row0 + 4 * hstu::kWaveRows, si.n); r0 += 2 * hstu::kWaveRows) {
                const hstu::KeyTiles kt =
                    hstu::key_tiles_for_rows(r0, std::min(r0 + 2 * hstu::kWaveRows, si.n), si.nc, si.nh);
                half.push_back(WorkUnit{u.seq, u.head, r0, kt.count()});
            }
        }
        units = &half;
    }
    int64_t total = 0;
    for (const WorkUnit& u : *units) total += u.cost;
    const int cap = (int)std::max<int64_t>(kMinSplit, 2 * ((total + slots - 1) / slots));
    plan->items.clear();
    plan->fix.clear();
    plan->parts = 0;
    auto item = [&](const WorkUnit& u, int cost, int t0, int t1, int part) {
        const SeqInfo& si = plan->seqs[u.seq];
        const CacheSeq cs = plan->cache.empty() ? CacheSeq{0, 0} : plan->cache[u.seq];
        return FwdItem{u.seq, u.head, u.row0, cost, t0, t1, part, 0,
                       si.start, si.n, si.nc, si.nh, cs.start, cs.n, 0, 0};
    };
    for (const WorkUnit& u : *units) {
        if (u.cost <= cap) {
            plan->items.push_back(item(u, u.cost, 0, u.cost, -1));
            continue;
        }
        const int k = (u.cost + cap - 1) / cap;
        plan->fix.push_back(FixItem{u.seq, u.head, u.row0, plan->parts, k, 0, 0, 0});
        for (int c = 0; c < k; ++c) {
            const int t0 = (int)((int64_t)c * u.cost / k), t1 = (int)((int64_t)(c + 1) * u.cost / k);
            plan->items.push_back(item(u, t1 - t0, t0, t1, plan->parts++));
        }
    }
    order_for_xcds(plan->items);
}

// The stream plan uploads go through, one per device, created on first use: non-blocking, so an
// upload neither waits for nor is ordered after the caller's queued kernels (the plan's buffer is
// new, nothing queued can touch it).
hipStream_t upload_stream(int device) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static hipStream_t streams[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!streams[device] &&
        hipStreamCreateWithFlags(&streams[device], hipStreamNonBlocking) != hipSuccess)
        streams[device] = nullptr;
    return streams[device];
}

// Returns the plan's device buffer: pool memory in the order of `stream` (after the work queued
// there), hipMalloc memory with hipFree, which waits for the device.
void release_device_lists(hstu_plan_t* plan, hipStream_t stream) {
    if (!plan->dbuf) return;
    if (plan->pooled) (void)hipFreeAsync(plan->dbuf, stream);
    else (void)hipFree(plan->dbuf);
    plan->dbuf = nullptr;
}

// HSTU_DEBUG_SYNC=1 in the environment: every kernel launch of the entry points is followed by a
// synchronisation of its stream and an error check, so a fault is reported by the call that
// caused it (as HSTU_ERR_HIP) instead of at a later synchronisation.
bool debug_sync() {
    static const bool on = [] {
        const char* v = std::getenv("HSTU_DEBUG_SYNC");
        return v && v[0] && !(v[0] == '0' && v[1] == 0);
    }();
    return on;
}

hipError_t checked(hipError_t e, hipStream_t s) {
    if (e != hipSuccess || !debug_sync()) return e;
    e = hipStreamSynchronize(s);
    const hipError_t last = hipGetLastError();
    return e != hipSuccess ? e : last;
}

size_t part_bytes(const hstu_plan_t* plan) {
    return align_up(size_t(plan->parts) * plan->item_rows * plan->shape.head_dim * 4, 256);
}

// Stored dS of the bf16 backward (0 when the plan does not use it).
size_t ds_bytes(const hstu_plan_t* plan) { return align_up(size_t(plan->ds_elems) * 2, 256); }

// The stored-dS dK/dV pass's bias-mode records (256 bytes per chunk of one head: one 32-byte
// record per wavefront of the 128-key x 64-query block) and the query times relative to each
// sequence's first (4 bytes per token), after the dS (and in op 2 after the gradient tables).
size_t rec_bytes(const hstu_plan_t* plan) {
    if (plan->ds_elems <= 0) return 0;
    const int64_t chunks = plan->ds_elems / (int64_t(hstu::kDsChunk) * plan->shape.num_heads);
    return align_up(size_t(chunks) * 256, 256);
}
size_t modes_bytes(const hstu_plan_t* plan) {
    if (plan->ds_elems <= 0) return 0;
    return rec_bytes(plan) + align_up(size_t(plan->shape.total_tokens) * 4, 256);
}
// Points p's mode records and relative times at `at` (the layout of modes_bytes).
void set_modes(const hstu_plan_t* plan, char* at, hstu::AttnParams* p) {
    p->modes = at;
    p->tq_rel = reinterpret_cast<uint32_t*>(at + rec_bytes(plan));
}

// The bias-table gradients the stored-dS dK/dV pass sums for the dQ pass to hand out: two
// [H][128] fp32 tables after the stored dS.
size_t grad_bytes(const hstu_plan_t* plan) {
    return plan->ds_elems > 0 ? align_up(size_t(2) * plan->shape.num_heads * hstu::kNumBuckets * 4, 256) : 0;
}

// The stored-dS layout (geometry.h): per sequence, its 128-key blocks in order, each holding one
// 128 x 64 bf16 chunk per 64-query tile its visible queries span, heads one after another; the
// sequence's first element offset goes to the device.  Head dims 64 and 128 only (the dQ kernel
// keeps its dS tiles where the query rows of the recomputing kernel go).
void plan_ds_layout(hstu_plan_t* plan) {
    plan->ds_off.clear();
    plan->ds_elems = 0;
    const hstu_attn_args_t& a = plan->shape;
    if (plan->cached || a.dtype != HSTU_BF16 || a.head_dim < 64) return;
    int64_t total = 0;
    std::vector<int64_t> off(plan->seqs.size());
    for (size_t b = 0; b < plan->seqs.size(); ++b) {
        const SeqInfo& si = plan->seqs[b];
        // a key block's chunks are addressed with 32-bit byte offsets (sequences up to ~8M tokens)
        if (int64_t(2) * hstu::cdiv(si.n, 128) * hstu::kDsChunk * 2 >= (int64_t(1) << 31)) return;
        off[b] = total;
        total += int64_t(hstu::kDsChunk) * a.num_heads *
                 hstu::ds_chunks_before(hstu::cdiv(si.n, 128), si.n, si.nc, si.nh);
    }
    plan->ds_off = std::move(off);
    plan->ds_elems = total;
}

hstu::AttnParams base_params(const hstu_plan_t* plan, const hstu_attn_args_t* a) {
    hstu::AttnParams p{};
    p.seqs = plan->d_seqs;
    p.units = plan->d_fwd;
    p.num_units = (int32_t)plan->fwd.size();
    p.items = plan->d_items;
    p.num_items = (int32_t)plan->items.size();
    p.fix = plan->d_fix;
    p.num_fix = (int32_t)plan->fix.size();
    p.item_rows = plan->item_rows;
    p.heads = a->num_heads;
    p.head_dim = a->head_dim;
    int64_t hd = int64_t(a->num_heads) * a->head_dim;
    p.ld_in = a->qkv_token_stride ? a->qkv_token_stride : hd;
    p.ld_out = hd;
    p.ld_grad = hd;
    p.alpha = a->alpha;
    p.inv_n = 1.0f / (float)a->max_seqlen;
    p.ts = a->timestamps;
    p.rab_pos = a->rab_pos;
    p.rab_ts = a->rab_ts;
    return p;
}

hstu_status_t hip_status(hipError_t e) { return e == hipSuccess ? HSTU_OK : HSTU_ERR_HIP; }

// Builds the bf16 forward items and, unless HSTU_PLAN_HOST_ONLY, copies every list into one
// device buffer.  Takes ownership of plan (deleted on failure).
hstu_status_t finish_plan(hstu_plan_t* plan, uint32_t flags, hstu_plan_t** out) {
    const bool host_only = (flags & HSTU_PLAN_HOST_ONLY) != 0;
    int compute_units = 256;
    if (!host_only) {
        if (hipGetDevice(&plan->device) != hipSuccess ||
            hipDeviceGetAttribute(&compute_units, hipDeviceAttributeMultiprocessorCount,
                                  plan->device) != hipSuccess) {
            delete plan;
            return HSTU_ERR_HIP;
        }
    }
    plan->compute_units = compute_units;
    if (plan->shape.dtype == HSTU_BF16) build_fwd_items(plan, compute_units);
    plan_ds_layout(plan);

    if (!host_only) {
        constexpr int kArrays = 8;
        const size_t sizes[kArrays] = {sizeof(SeqInfo) * plan->seqs.size(),
                                       sizeof(WorkUnit) * plan->fwd.size(),
                                       sizeof(WorkUnit) * plan->bwd.size(),
                                       sizeof(FwdItem) * plan->items.size(),
                                       sizeof(FixItem) * plan->fix.size(),
                                       sizeof(CacheSeq) * plan->cache.size(),
                                       sizeof(int64_t) * plan->ds_off.size(),
                                       sizeof(WorkUnit) * plan->dqs.size()};
        const void* srcs[kArrays] = {plan->seqs.data(), plan->fwd.data(), plan->bwd.data(),
                                     plan->items.data(), plan->fix.data(), plan->cache.data(),
                                     plan->ds_off.data(), plan->dqs.data()};
        size_t offs[kArrays], total = 0;
        for (int i = 0; i < kArrays; ++i) {
            offs[i] = total;
            total += align_up(sizes[i], 16);
        }
        total = std::max<size_t>(total, 16);
        std::vector<char> host(total);
        for (int i = 0; i < kArrays; ++i)
            if (sizes[i]) std::memcpy(host.data() + offs[i], srcs[i], sizes[i]);
        hipStream_t up = upload_stream(plan->device);
        if (!up) {
            delete plan;
            return HSTU_ERR_HIP;
        }
        // stream-ordered allocation where the device supports it, so that freeing a plan need
        // not synchronize the device
        plan->pooled = hipMallocAsync(&plan->dbuf, total, up) == hipSuccess;
        if (!plan->pooled) {
            (void)hipGetLastError();
            plan->dbuf = nullptr;
            if (hipMalloc(&plan->dbuf, total) != hipSuccess) {
                delete plan;
                return HSTU_ERR_HIP;
            }
        }
        if (hipMemcpyAsync(plan->dbuf, host.data(), total, hipMemcpyHostToDevice, up) != hipSuccess ||
            hipStreamSynchronize(up) != hipSuccess) {
            release_device_lists(plan, up);
            delete plan;
            return HSTU_ERR_HIP;
        }
        char* base = static_cast<char*>(plan->dbuf);
        plan->d_seqs = reinterpret_cast<const SeqInfo*>(base + offs[0]);
        plan->d_fwd = reinterpret_cast<const WorkUnit*>(base + offs[1]);
        plan->d_bwd = reinterpret_cast<const WorkUnit*>(base + offs[2]);
        plan->d_items = reinterpret_cast<const FwdItem*>(base + offs[3]);
        plan->d_fix = reinterpret_cast<const FixItem*>(base + offs[4]);
        plan->d_cache = reinterpret_cast<const CacheSeq*>(base + offs[5]);
        plan->d_ds_off = reinterpret_cast<const int64_t*>(base + offs[6]);
        plan->d_dqs = reinterpret_cast<const WorkUnit*>(base + offs[7]);
        plan->on_device = true;
    }
    *out = plan;
    return HSTU_OK;
}

// Scratch memory of hstu_attn_fwd_noalloc: a static device array, so that the call needs no
// allocation.  Each device holds its own copy (from the first call on it until the process ends);
// host code reaches a device's copy only through the address hipGetSymbolAddress returns for it,
// kept per device.  Calls that overlap on one device share the array and race.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The scratch array's address on the current device (looked up once per device).
hstu_status_t scratch_address(void** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HSTU_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return HSTU_ERR_HIP;
        }
        addr[dev] = p;
    }
    *out = addr[dev];
    return HSTU_OK;
}

}  // namespace

extern "C" {

const char* hstu_status_str(hstu_status_t s) {
    switch (s) {
        case HSTU_OK: return "ok";
        case HSTU_ERR_NULL_ARG: return "a required pointer is NULL";
        case HSTU_ERR_BAD_SHAPE: return "sizes invalid or inconsistent with the plan";
        case HSTU_ERR_BAD_OFFSETS: return "seq_offsets must run from 0 to T without decreasing, "
                                          "and no length may exceed max_seqlen";
        case HSTU_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or model width";
        case HSTU_ERR_MISALIGNED: return "pointers must be 16-byte aligned and token strides a "
                                         "multiple of 8 elements";
        case HSTU_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than hstu_workspace_bytes()";
        case HSTU_ERR_HIP: return "a HIP runtime call failed";
        case HSTU_ERR_NO_DEVICE_PLAN: return "plan was created host-only";
        case HSTU_ERR_SCRATCH_LIMIT: return "the call needs more scratch than the library's static "
                                           "buffer holds (hstu_attn_fwd_noalloc: 64 MiB)";
    }
    return "unknown status";
}

hstu_status_t hstu_plan_create(const hstu_attn_args_t* args, const int64_t* off,
                               const int32_t* num_targets, uint32_t flags, hstu_plan_t** out) {
    if (!out) return HSTU_ERR_NULL_ARG;
    *out = nullptr;
    hstu_status_t st = check_args(args);
    if (st != HSTU_OK) return st;
    if (!off) return HSTU_ERR_NULL_ARG;
    const int B = args->batch;
    if (off[0] != 0 || off[B] != args->total_tokens) return HSTU_ERR_BAD_OFFSETS;
    for (int b = 0; b < B; ++b) {
        int64_t n = off[b + 1] - off[b];
        if (n < 0 || n > args->max_seqlen) return HSTU_ERR_BAD_OFFSETS;
        if (num_targets && num_targets[b] < 0) return HSTU_ERR_BAD_SHAPE;
    }

    hstu_plan_t* plan = new (std::nothrow) hstu_plan_t();
    if (!plan) return HSTU_ERR_HIP;
    plan->shape = *args;
    plan->shape.timestamps = nullptr;
    plan->shape.rab_pos = nullptr;
    plan->shape.rab_ts = nullptr;
    const bool bf16 = args->dtype == HSTU_BF16;
    plan->fwd_rows = bf16 ? 4 * hstu::kWaveRows : 64;
    plan->bwd_keys = bf16 ? 4 * hstu::kWaveRows : 64;
    const int H = args->num_heads;

    plan->seqs.resize(B);
    for (int b = 0; b < B; ++b) {
        int n = (int)(off[b + 1] - off[b]);
        int nc, nh;
        hstu::split_sequence(n, args->num_contexts, num_targets ? num_targets[b] : 0, &nc, &nh);
        plan->seqs[b] = SeqInfo{(int32_t)off[b], n, nc, nh};
        plan->pairs += visible_pairs(n, nc, nh) * H;
    }
    for (int b = 0; b < B; ++b) {
        const SeqInfo& s = plan->seqs[b];
        // forward / dQ: row blocks
        for (int r0 = 0; r0 < s.n; r0 += plan->fwd_rows) {
            int rhi = std::min(r0 + plan->fwd_rows, s.n);
            hstu::KeyTiles kt = hstu::key_tiles_for_rows(r0, rhi, s.nc, s.nh);
            for (int h = 0; h < H; ++h) plan->fwd.push_back(WorkUnit{b, h, r0, kt.count()});
        }
        // stored-dS dQ (bf16): 256-row blocks
        if (bf16)
            for (int r0 = 0; r0 < s.n; r0 += 2 * plan->fwd_rows) {
                hstu::KeyTiles kt = hstu::key_tiles_for_rows(r0, std::min(r0 + 2 * plan->fwd_rows, s.n), s.nc, s.nh);
                for (int h = 0; h < H; ++h) plan->dqs.push_back(WorkUnit{b, h, r0, kt.count()});
            }
        // dK/dV: key blocks
        for (int k0 = 0; k0 < s.n; k0 += plan->bwd_keys) {
            int qlo, qhi;
            hstu::rows_for_keys(k0, std::min(k0 + plan->bwd_keys, s.n), s.n, s.nc, s.nh, &qlo,
                                &qhi);
            int cost = hstu::cdiv(qhi, hstu::kQueryTile) - qlo / hstu::kQueryTile;
            for (int h = 0; h < H; ++h) plan->bwd.push_back(WorkUnit{b, h, k0, cost});
        }
    }
    // row blocks in the XCD launch order (the dQ pass reads each (sequence, head)'s K rows from
    // one L2); key blocks longest first (their costs differ widely and the longest bound the pass),
    // a stable sort, so each block's heads stay together in head order (the stored-dS modes pass
    // takes every heads-th entry)
    order_for_xcds(plan->fwd);
    order_for_xcds(plan->dqs);
    sort_longest_first(plan->bwd);
    return finish_plan(plan, flags, out);
}

void hstu_plan_destroy(hstu_plan_t* plan) {
    if (!plan) return;
    if (plan->dbuf) {
        // wait for every stream of the plan's device, then free
        int cur = -1;
        const bool other = hipGetDevice(&cur) == hipSuccess && cur != plan->device;
        if (other) (void)hipSetDevice(plan->device);
        (void)hipDeviceSynchronize();
        release_device_lists(plan, nullptr);
        if (other) (void)hipSetDevice(cur);
    }
    delete plan;
}

void hstu_plan_destroy_on(hstu_plan_t* plan, void* stream) {
    if (!plan) return;
    release_device_lists(plan, static_cast<hipStream_t>(stream));
    delete plan;
}

// (32-row, 64-key) tiles the forward computes: every wavefront's non-empty tiles of every row
// block, all heads.  Only reported, so counted on request rather than while planning.
int64_t count_fwd_tiles(const hstu_plan_t* plan) {
    int64_t total = 0;
    for (const SeqInfo& s : plan->seqs)
        for (int r0 = 0; r0 < s.n; r0 += plan->fwd_rows) {
            const int rhi = std::min(r0 + plan->fwd_rows, s.n);
            const hstu::KeyTiles kt = hstu::key_tiles_for_rows(r0, rhi, s.nc, s.nh);
            for (int t = 0; t < kt.count(); ++t) {
                const int j0 = kt.tile(t) * hstu::kKeyTile;
                for (int w0 = r0; w0 < rhi; w0 += hstu::kWaveRows)
                    total += hstu::classify_row_tile(w0, std::min(w0 + hstu::kWaveRows, rhi), j0,
                                                     s.n, s.nc, s.nh) != hstu::kEmpty;
            }
        }
    return total * plan->shape.num_heads;
}

hstu_status_t hstu_plan_info(const hstu_plan_t* plan, hstu_plan_info_t* info) {
    if (!plan || !info) return HSTU_ERR_NULL_ARG;
    info->visible_pairs = plan->pairs;
    info->fwd_units = (int64_t)plan->fwd.size();
    info->bwd_units = (int64_t)plan->bwd.size();
    info->fwd_tiles = plan->fwd_tiles >= 0 ? plan->fwd_tiles : count_fwd_tiles(plan);
    info->fwd_row_block = plan->fwd_rows;
    info->bwd_key_block = plan->bwd_keys;
    info->fwd_items = plan->shape.dtype == HSTU_BF16 ? (int64_t)plan->items.size()
                                                     : (int64_t)plan->fwd.size();
    info->fwd_split_blocks = (int64_t)plan->fix.size();
    info->fwd_item_rows = plan->shape.dtype == HSTU_BF16 ? plan->item_rows : plan->fwd_rows;
    info->bwd_stored_ds = plan->ds_elems > 0 ? 1 : 0;
    info->bwd_ds_bytes = (int64_t)ds_bytes(plan);
    return HSTU_OK;
}

hstu_status_t hstu_plan_units(const hstu_plan_t* plan, int32_t op, int32_t* units, int64_t cap,
                              int64_t* count) {
    if (!plan || !count) return HSTU_ERR_NULL_ARG;
    if (op < 0 || op > 3) return HSTU_ERR_BAD_SHAPE;
    if (op == 2) {
        *count = (int64_t)plan->items.size();
        if (cap > 0 && !units) return HSTU_ERR_NULL_ARG;
        int64_t m = std::min<int64_t>(cap, (int64_t)plan->items.size());
        for (int64_t i = 0; i < m; ++i) {
            const FwdItem& it = plan->items[i];
            const int32_t rec[8] = {it.seq, it.head, it.row0, it.cost, it.t0, it.t1, it.part, 0};
            std::memcpy(units + 8 * i, rec, sizeof(rec));
        }
        return HSTU_OK;
    }
    const std::vector<WorkUnit>& u = op == 0 ? plan->fwd : op == 1 ? plan->bwd : plan->dqs;
    *count = (int64_t)u.size();
    if (cap > 0 && !units) return HSTU_ERR_NULL_ARG;
    int64_t m = std::min<int64_t>(cap, (int64_t)u.size());
    for (int64_t i = 0; i < m; ++i) {
        units[4 * i + 0] = u[i].seq;
        units[4 * i + 1] = u[i].head;
        units[4 * i + 2] = u[i].row0;
        units[4 * i + 3] = u[i].cost;
    }
    return HSTU_OK;
}

size_t hstu_workspace_bytes(const hstu_plan_t* plan, int32_t op, int32_t d_model) {
    if (!plan) return 0;
    const hstu_attn_args_t& a = plan->shape;
    size_t thd = size_t(a.total_tokens) * a.num_heads * a.head_dim;
    switch (op) {
        case 0: return part_bytes(plan);
        case 1: return align_up(thd * elem_size(a.dtype), 256) + part_bytes(plan);
        case 2: return ds_bytes(plan) + grad_bytes(plan) + modes_bytes(plan);
        case 3: {
            (void)d_model;  // Z and A depend on H*d only
            return align_up(4 * thd * 2, 256) + align_up(thd * 2, 256) + part_bytes(plan);
        }
        case 5: return plan->cached ? part_bytes(plan) : 0;
        case 4: {
            (void)d_model;
            // Z, H (pre-activation), dH: T x 4Hd bf16; A, G, dA: T x Hd bf16; dG: T x Hd fp32
            return 3 * align_up(4 * thd * 2, 256) + 3 * align_up(thd * 2, 256) +
                   align_up(thd * 4, 256) + std::max(part_bytes(plan), ds_bytes(plan) + modes_bytes(plan));
        }
        default: return 0;
    }
}

hstu_status_t hstu_attn_fwd(const hstu_plan_t* plan, const hstu_attn_args_t* args, const void* q,
                            const void* k, const void* v, const void* u, float ln_eps, void* out,
                            void* ws, size_t ws_bytes, void* stream) {
    hstu_status_t st = check_call(plan, args);
    if (st != HSTU_OK) return st;
    if (args->total_tokens == 0) return HSTU_OK;  // nothing to read or write; pointers may be NULL
    if (!q || !k || !v || !out) return HSTU_ERR_NULL_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (u && !aligned16(u)))
        return HSTU_ERR_MISALIGNED;
    const size_t need = hstu_workspace_bytes(plan, u ? 1 : 0, 0);
    if (need > 0) {
        if (!ws) return HSTU_ERR_NULL_ARG;
        if (ws_bytes < need) return HSTU_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned16(ws)) return HSTU_ERR_MISALIGNED;
    }
    if (u && (!(ln_eps >= 0.0f) || !std::isfinite(ln_eps))) return HSTU_ERR_BAD_SHAPE;
    if (plan->fwd.empty()) return HSTU_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hstu::AttnParams p = base_params(plan, args);
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = u ? ws : out;
    // partial slots follow the gated path's attention buffer in ws
    const size_t gated_bytes = u ? align_up(size_t(args->total_tokens) * p.ld_out * elem_size(args->dtype), 256) : 0;
    p.part = plan->parts ? reinterpret_cast<float*>(static_cast<char*>(ws) + gated_bytes) : nullptr;
    hipError_t e = args->dtype == HSTU_BF16 ? checked(hstu::launch_attn_fwd_bf16(p, s), s)
                                            : checked(hstu::launch_attn_fwd_f32(p, s), s);
    if (e != hipSuccess) return HSTU_ERR_HIP;
    if (u) {
        int64_t ldu = args->qkv_token_stride ? args->qkv_token_stride : p.ld_out;
        int32_t width = (int32_t)p.ld_out;
        e = args->dtype == HSTU_BF16
                ? checked(hstu::launch_ln_gate_bf16(ws, u, ldu, out, args->total_tokens, width, ln_eps, s), s)
                : checked(hstu::launch_ln_gate_f32(ws, u, ldu, out, args->total_tokens, width, ln_eps, s), s);
    }
    return hip_status(e);
}

hstu_status_t hstu_attn_fwd_noalloc(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                                    const void* q, const void* k, const void* v, const void* u,
                                    float ln_eps, void* out, void* stream) {
    hstu_status_t st = check_call(plan, args);
    if (st != HSTU_OK) return st;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return HSTU_ERR_HIP;
    if (dev != plan->device) return HSTU_ERR_BAD_SHAPE;
    const size_t need = hstu_workspace_bytes(plan, u ? 1 : 0, 0);
    if (need > kScratchBytes) return HSTU_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0 && args->total_tokens > 0) {
        st = scratch_address(&ws);
        if (st != HSTU_OK) return st;
    }
    // the same launches as hstu_attn_fwd, with the workspace in the static array: the partial
    // slots and the gated path's attention buffer are written in full before they are read, so
    // nothing left there by an earlier call is seen
    return hstu_attn_fwd(plan, args, q, k, v, u, ln_eps, out, ws, ws ? kScratchBytes : 0, stream);
}

}  // extern "C"

namespace {

// Validation and parameters shared by the backward entry points.  Pointers that a pass does not
// use are passed as NULL and not checked.
hstu_status_t bwd_params(const hstu_plan_t* plan, const hstu_attn_args_t* args, const void* q,
                         const void* k, const void* v, const void* dout,
                         std::initializer_list<const void*> outs, hstu::AttnParams* p) {
    hstu_status_t st = check_call(plan, args);
    if (st != HSTU_OK) return st;
    if (args->total_tokens != 0) {
        if (!q || !k || !v || !dout) return HSTU_ERR_NULL_ARG;
        for (const void* o : outs)
            if (!o) return HSTU_ERR_NULL_ARG;
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout)) return HSTU_ERR_MISALIGNED;
    for (const void* o : outs)
        if (!aligned16(o)) return HSTU_ERR_MISALIGNED;
    *p = base_params(plan, args);
    p->q = q;
    p->k = k;
    p->v = v;
    p->dout = dout;
    return HSTU_OK;
}

// The stored-dS workspace of a backward call: NULL when the plan has none or the caller passed
// none (the dQ pass then recomputes S and dP).
hstu_status_t ds_workspace(const hstu_plan_t* plan, void* ws, size_t ws_bytes, void** ds) {
    *ds = nullptr;
    const size_t need = hstu_workspace_bytes(plan, 2, 0);
    if (need == 0 || !ws) return HSTU_OK;
    if (ws_bytes < need) return HSTU_ERR_WORKSPACE_TOO_SMALL;
    if (!aligned16(ws)) return HSTU_ERR_MISALIGNED;
    *ds = ws;
    return HSTU_OK;
}

}  // namespace

extern "C" {

hstu_status_t hstu_attn_bwd_dkdv(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                                 const void* q, const void* k, const void* v, const void* dout,
                                 void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
    hstu::AttnParams p;
    hstu_status_t st = bwd_params(plan, args, q, k, v, dout, {dk, dv}, &p);
    if (st != HSTU_OK) return st;
    if (args->total_tokens == 0) return HSTU_OK;
    st = ds_workspace(plan, ws, ws_bytes, &p.ds);
    if (st != HSTU_OK) return st;
    p.ds_off = p.ds ? plan->d_ds_off : nullptr;
    p.units = plan->d_bwd;
    p.num_units = (int32_t)plan->bwd.size();
    p.dk = dk;
    p.dv = dv;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.ds) {  // this pass sums the bias-table gradients into the workspace (the modes pass,
                 // which runs first, clears them)
        set_modes(plan, static_cast<char*>(ws) + ds_bytes(plan) + grad_bytes(plan), &p);
        float* grads = reinterpret_cast<float*>(static_cast<char*>(ws) + ds_bytes(plan));
        const int64_t nb = int64_t(args->num_heads) * hstu::kNumBuckets;
        p.gpos = args->rab_pos ? grads : nullptr;
        p.gts = args->rab_ts ? grads + nb : nullptr;
    }
    return hip_status(args->dtype == HSTU_BF16 ? checked(hstu::launch_attn_bwd_dkdv_bf16(p, s), s)
                                               : checked(hstu::launch_attn_bwd_dkdv_f32(p, s), s));
}

hstu_status_t hstu_attn_bwd_dq(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                               const void* q, const void* k, const void* v, const void* dout,
                               void* dq, float* drab_pos, float* drab_ts, void* ws,
                               size_t ws_bytes, void* stream) {
    hstu::AttnParams p;
    hstu_status_t st = bwd_params(plan, args, q, k, v, dout, {dq}, &p);
    if (st != HSTU_OK) return st;
    if ((drab_pos && !aligned16(drab_pos)) || (drab_ts && !aligned16(drab_ts)))
        return HSTU_ERR_MISALIGNED;
    if (args->total_tokens != 0) {
        st = ds_workspace(plan, ws, ws_bytes, &p.ds);
        if (st != HSTU_OK) return st;
        p.ds_off = p.ds ? plan->d_ds_off : nullptr;
        if (p.ds) {  // the stored-dS pass runs over 256-row blocks
            p.units = plan->d_dqs;
            p.num_units = (int32_t)plan->dqs.size();
        }
    }
    p.dq = dq;
    p.drab_pos = args->rab_pos ? drab_pos : nullptr;
    p.drab_ts = args->rab_ts ? drab_ts : nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t nb = int64_t(args->num_heads) * hstu::kNumBuckets;
    hipError_t e = hipSuccess;
    if (p.ds) {  // the dK/dV pass summed the bias-table gradients into the workspace; the dQ
                 // pass's first workgroup copies them to the outputs
        float* grads = reinterpret_cast<float*>(static_cast<char*>(ws) + ds_bytes(plan));
        p.gpos = p.drab_pos ? grads : nullptr;
        p.gts = p.drab_ts ? grads + nb : nullptr;
    } else {
        if (p.drab_pos) e = checked(hstu::launch_zero_f32(p.drab_pos, nb, s), s);
        if (e == hipSuccess && p.drab_ts) e = checked(hstu::launch_zero_f32(p.drab_ts, nb, s), s);
    }
    if (e != hipSuccess) return HSTU_ERR_HIP;
    if (args->total_tokens == 0) return HSTU_OK;
    return hip_status(args->dtype == HSTU_BF16 ? checked(hstu::launch_attn_bwd_dq_bf16(p, s), s)
                                               : checked(hstu::launch_attn_bwd_dq_f32(p, s), s));
}

hstu_status_t hstu_attn_bwd(const hstu_plan_t* plan, const hstu_attn_args_t* args, const void* q,
                            const void* k, const void* v, const void* dout, void* dq, void* dk,
                            void* dv, float* drab_pos, float* drab_ts, void* ws, size_t ws_bytes,
                            void* stream) {
    hstu::AttnParams p;
    hstu_status_t st = bwd_params(plan, args, q, k, v, dout, {dq, dk, dv}, &p);
    if (st != HSTU_OK) return st;
    if (args->total_tokens != 0 && hstu_workspace_bytes(plan, 2, 0) > 0 && !ws)
        return HSTU_ERR_NULL_ARG;
    st = hstu_attn_bwd_dkdv(plan, args, q, k, v, dout, dk, dv, ws, ws_bytes, stream);
    if (st != HSTU_OK) return st;
    return hstu_attn_bwd_dq(plan, args, q, k, v, dout, dq, drab_pos, drab_ts, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

hstu_status_t layer_checks(const hstu_plan_t* plan, const hstu_attn_args_t* args, int32_t d_model,
                           std::initializer_list<const void*> ptrs, float ln_eps) {
    hstu_status_t st = check_call(plan, args);
    if (st != HSTU_OK) return st;
    if (args->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
    for (const void* q : ptrs)
        if (!q) return HSTU_ERR_NULL_ARG;
    if (d_model < 128 || d_model % 128 != 0) return HSTU_ERR_UNSUPPORTED;
    if (!rows_addressable(args->max_seqlen, 4 * int64_t(args->num_heads) * args->head_dim))
        return HSTU_ERR_UNSUPPORTED;
    if ((args->num_heads * args->head_dim) % 64 != 0 || args->num_heads * args->head_dim > 4096)
        return HSTU_ERR_UNSUPPORTED;
    for (const void* q : ptrs)
        if (!aligned16(q)) return HSTU_ERR_MISALIGNED;
    if (!(ln_eps >= 0.0f) || !std::isfinite(ln_eps)) return HSTU_ERR_BAD_SHAPE;
    return HSTU_OK;
}

hstu::GemmArgs gemm_args(const hstu_plan_t* plan, const void* a, int64_t lda, bool at,
                         const void* b, int64_t ldb, bool bt, int64_t M, int32_t N, int64_t K,
                         void* c, int64_t ldc, int32_t epi) {
    hstu::GemmArgs g{};
    g.a = a;
    g.lda = lda;
    g.at = at;
    g.b = b;
    g.ldb = ldb;
    g.bt = bt;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = c;
    g.ldc = ldc;
    g.epilogue = epi;
    g.compute_units = plan->compute_units;
    return g;
}

// Tokens per workgroup for a weight gradient (M x N outputs summed over T tokens): enough
// splits for about one tile per compute unit, at least 256 tokens each.  More splits add more
// fp32 partial tiles atomically (four per compute unit took twice as long on the layer shapes).
int64_t token_chunk(const hstu_plan_t* plan, int64_t T, int64_t M, int64_t N) {
    const int64_t tiles = (M / 128) * (N / 128);
    const int64_t want = std::max<int64_t>(1, (int64_t(plan->compute_units) + tiles - 1) / tiles);
    int64_t chunk = (T + want - 1) / want;
    chunk = std::max<int64_t>(256, (chunk + 63) / 64 * 64);
    while ((T + chunk - 1) / chunk > 65535) chunk *= 2;
    return chunk;
}

}  // namespace

extern "C" {

hstu_status_t hstu_layer_fwd(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                             int32_t d_model, const void* x, const void* w1, const void* w2,
                             float ln_eps, void* y, void* ws, size_t ws_bytes, void* stream) {
    hstu_status_t st = layer_checks(plan, args, d_model, {x, w1, w2, y, ws}, ln_eps);
    if (st != HSTU_OK) return st;
    if (ws_bytes < hstu_workspace_bytes(plan, 3, d_model)) return HSTU_ERR_WORKSPACE_TOO_SMALL;
    const int64_t T = args->total_tokens;
    const int32_t hd = args->num_heads * args->head_dim;
    if (T == 0) return HSTU_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* z = static_cast<char*>(ws);
    char* a = z + align_up(size_t(T) * 4 * hd * 2, 256);
    // Z = SiLU(X W1): columns [U | V | Q | K]
    hipError_t e = checked(hstu::launch_gemm(
        gemm_args(plan, x, d_model, false, w1, 4 * hd, false, T, 4 * hd, d_model, z, 4 * hd, hstu::kEpiSilu), s), s);
    if (e != hipSuccess) return HSTU_ERR_HIP;
    hstu::AttnParams p = base_params(plan, args);
    const int64_t ldz = 4 * int64_t(hd);
    p.ld_in = ldz;
    p.part = plan->parts ? reinterpret_cast<float*>(a + align_up(size_t(T) * hd * 2, 256)) : nullptr;
    p.v = z + size_t(hd) * 2;
    p.q = z + size_t(2 * hd) * 2;
    p.k = z + size_t(3 * hd) * 2;
    p.out = a;
    e = checked(hstu::launch_attn_fwd_bf16(p, s), s);
    if (e != hipSuccess) return HSTU_ERR_HIP;
    // G = LayerNorm(A) * U, in place over A
    e = checked(hstu::launch_ln_gate_bf16(a, z, ldz, a, T, hd, ln_eps, s), s);
    if (e != hipSuccess) return HSTU_ERR_HIP;
    // Y = G W2 + X
    hstu::GemmArgs g = gemm_args(plan, a, hd, false, w2, d_model, false, T, d_model, hd, y, d_model,
                                 hstu::kEpiResidual);
    g.r = x;
    g.ldr = d_model;
    return hip_status(checked(hstu::launch_gemm(g, s), s));
}

hstu_status_t hstu_layer_bwd(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                             int32_t d_model, const void* x, const void* w1, const void* w2,
                             const void* dy, float ln_eps, void* dx, float* dw1, float* dw2,
                             float* drab_pos, float* drab_ts, void* ws, size_t ws_bytes,
                             void* stream) {
    // with no tokens only the gradients that are cleared need to exist
    hstu_status_t st = args && args->total_tokens == 0
                           ? layer_checks(plan, args, d_model, {dw1, dw2}, ln_eps)
                           : layer_checks(plan, args, d_model, {x, w1, w2, dy, dx, dw1, dw2, ws}, ln_eps);
    if (st != HSTU_OK) return st;
    const int64_t T = args->total_tokens;
    const int32_t hd = args->num_heads * args->head_dim;
    if (hd % 128 != 0) return HSTU_ERR_UNSUPPORTED;
    if ((drab_pos && !aligned16(drab_pos)) || (drab_ts && !aligned16(drab_ts)))
        return HSTU_ERR_MISALIGNED;
    if (T > 0 && ws_bytes < hstu_workspace_bytes(plan, 4, d_model))
        return HSTU_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // weight and bias-table gradients are sums over tokens: clear them (also when T == 0)
    drab_pos = args->rab_pos ? drab_pos : nullptr;
    drab_ts = args->rab_ts ? drab_ts : nullptr;
    const int64_t nb = int64_t(args->num_heads) * hstu::kNumBuckets;
    float* const outs[4] = {dw1, dw2, drab_pos, drab_ts};
    const int64_t counts[4] = {int64_t(d_model) * 4 * hd, int64_t(hd) * d_model, nb, nb};
    hipError_t e = checked(hstu::launch_zero_f32_list(outs, counts, 4, s), s);
    if (e != hipSuccess) return HSTU_ERR_HIP;
    if (T == 0) return HSTU_OK;
    const size_t wide = align_up(size_t(T) * 4 * hd * 2, 256), narrow = align_up(size_t(T) * hd * 2, 256);
    char* z = static_cast<char*>(ws);
    char* hpre = z + wide;
    char* dh = hpre + wide;
    char* a = dh + wide;
    char* g = a + narrow;
    char* da = g + narrow;
    float* dg = reinterpret_cast<float*>(da + narrow);
    // the forward's partial slots, later the backward's stored dS
    char* tail = reinterpret_cast<char*>(dg) + align_up(size_t(T) * hd * 4, 256);
    float* part = reinterpret_cast<float*>(tail);
    const int64_t ldz = 4 * int64_t(hd);

    // recompute H = X W1 and Z = SiLU(H), columns [U | V | Q | K]
    hstu::GemmArgs ga = gemm_args(plan, x, d_model, false, w1, 4 * hd, false, T, 4 * hd, d_model, z,
                                  ldz, hstu::kEpiSilu);
    ga.c2 = hpre;
    e = checked(hstu::launch_gemm(ga, s), s);
    // recompute A = attention(Q, K, V)
    hstu::AttnParams p = base_params(plan, args);
    p.ld_in = ldz;
    p.ld_out = hd;
    p.ld_grad = ldz;
    p.v = z + size_t(hd) * 2;
    p.q = z + size_t(2 * hd) * 2;
    p.k = z + size_t(3 * hd) * 2;
    p.out = a;
    p.part = plan->parts ? part : nullptr;
    if (e == hipSuccess) e = checked(hstu::launch_attn_fwd_bf16(p, s), s);
    // dG = dY W2^T (fp32)
    if (e == hipSuccess)
        e = checked(hstu::launch_gemm(gemm_args(plan, dy, d_model, false, w2, d_model, true, T, hd, d_model, dg,
                                        hd, hstu::kEpiStoreF32), s), s);
    // G, dA and the U-slot gradient of H
    if (e == hipSuccess)
        e = checked(hstu::launch_ln_gate_bwd_bf16(a, z, hpre, ldz, dg, g, da, dh, ldz, T, hd, ln_eps, s), s);
    // dW2 = G^T dY, split over tokens
    if (e == hipSuccess) {
        hstu::GemmArgs gw = gemm_args(plan, g, hd, true, dy, d_model, false, hd, d_model, T, dw2,
                                      d_model, hstu::kEpiAtomicF32);
        gw.kchunk = token_chunk(plan, T, hd, d_model);
        e = checked(hstu::launch_gemm(gw, s), s);
    }
    // attention backward with dout = dA: dV, dQ, dK into their slots of dH, already multiplied
    // by SiLU'(H) (the projection's SiLU; the U slot is done by the LayerNorm backward)
    if (e == hipSuccess) {
        p.gate_delta = hpre - dh;
        p.dout = da;
        p.dv = dh + size_t(hd) * 2;
        p.dq = dh + size_t(2 * hd) * 2;
        p.dk = dh + size_t(3 * hd) * 2;
        p.units = plan->d_bwd;
        p.num_units = (int32_t)plan->bwd.size();
        if (plan->ds_elems > 0) {  // the dK/dV pass then sums the bias-table gradients
            p.ds = tail;
            p.ds_off = plan->d_ds_off;
            set_modes(plan, tail + ds_bytes(plan), &p);
            p.gpos = drab_pos;
            p.gts = drab_ts;
        }
        e = checked(hstu::launch_attn_bwd_dkdv_bf16(p, s), s);
    }
    if (e == hipSuccess) {
        p.units = p.ds ? plan->d_dqs : plan->d_fwd;  // the stored-dS pass runs over 256-row blocks
        p.num_units = (int32_t)(p.ds ? plan->dqs.size() : plan->fwd.size());
        p.drab_pos = drab_pos;
        p.drab_ts = drab_ts;
        e = checked(hstu::launch_attn_bwd_dq_bf16(p, s), s);
    }
    // dW1 = X^T dH, split over tokens
    if (e == hipSuccess) {
        hstu::GemmArgs gw = gemm_args(plan, x, d_model, true, dh, ldz, false, d_model, 4 * hd, T, dw1,
                                      ldz, hstu::kEpiAtomicF32);
        gw.kchunk = token_chunk(plan, T, d_model, 4 * hd);
        e = checked(hstu::launch_gemm(gw, s), s);
    }
    // dX = dH W1^T + dY
    if (e == hipSuccess) {
        hstu::GemmArgs gx = gemm_args(plan, dh, ldz, false, w1, ldz, true, T, d_model, ldz, dx, d_model,
                                      hstu::kEpiResidual);
        gx.r = dy;
        gx.ldr = d_model;
        e = checked(hstu::launch_gemm(gx, s), s);
    }
    return hip_status(e);
}

hstu_status_t hstu_plan_create_cached(const hstu_attn_args_t* args, const int64_t* cand_off,
                                      const int64_t* cache_off, uint32_t flags,
                                      hstu_plan_t** out) {
    if (!out) return HSTU_ERR_NULL_ARG;
    *out = nullptr;
    hstu_status_t st = check_args(args);
    if (st != HSTU_OK) return st;
    if (args->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
    if (!cand_off || !cache_off) return HSTU_ERR_NULL_ARG;
    const int B = args->batch;
    if (cand_off[0] != 0 || cand_off[B] != args->total_tokens || cache_off[0] != 0)
        return HSTU_ERR_BAD_OFFSETS;
    for (int b = 0; b < B; ++b) {
        const int64_t m = cand_off[b + 1] - cand_off[b], nk = cache_off[b + 1] - cache_off[b];
        if (m < 0 || nk < 0 || m + nk > args->max_seqlen) return HSTU_ERR_BAD_OFFSETS;
    }
    if (cache_off[B] >= (int64_t(1) << 31)) return HSTU_ERR_BAD_SHAPE;
    hstu_plan_t* plan = new (std::nothrow) hstu_plan_t();
    if (!plan) return HSTU_ERR_HIP;
    plan->shape = *args;
    plan->shape.timestamps = nullptr;
    plan->shape.rab_pos = nullptr;
    plan->shape.rab_ts = nullptr;
    plan->cached = true;
    plan->fwd_rows = 2 * hstu::kWaveRows;  // 64 candidates per item (fwd_bf16_kernel)
    plan->bwd_keys = 0;
    plan->fwd_tiles = 0;  // counted here: every key tile of the cache is visible
    const int H = args->num_heads;
    plan->seqs.resize(B);
    plan->cache.resize(B);
    for (int b = 0; b < B; ++b) {
        const int m = (int)(cand_off[b + 1] - cand_off[b]), nk = (int)(cache_off[b + 1] - cache_off[b]);
        plan->seqs[b] = SeqInfo{(int32_t)cand_off[b], m, 0, m};
        plan->cache[b] = CacheSeq{(int32_t)cache_off[b], nk};
        plan->pairs += int64_t(nk + 1) * m * H;
        const int tiles = hstu::cdiv(nk, hstu::kKeyTile);
        for (int r0 = 0; r0 < m; r0 += plan->fwd_rows) {
            plan->fwd_tiles += int64_t(tiles) * hstu::cdiv(std::min(plan->fwd_rows, m - r0), hstu::kWaveRows) * H;
            for (int h = 0; h < H; ++h) plan->fwd.push_back(WorkUnit{b, h, r0, tiles});
        }
    }
    sort_longest_first(plan->fwd);
    return finish_plan(plan, flags, out);
}

hstu_status_t hstu_attn_fwd_cached(const hstu_plan_t* plan, const hstu_attn_args_t* args,
                                   const void* q, const void* k, const void* v,
                                   const void* k_cache, const void* v_cache,
                                   const int64_t* cache_timestamps, void* out, void* ws,
                                   size_t ws_bytes, void* stream) {
    if (!plan) return HSTU_ERR_NULL_ARG;
    hstu_status_t st = check_args(args);
    if (st != HSTU_OK) return st;
    const hstu_attn_args_t& ps = plan->shape;
    if (!plan->cached || args->dtype != ps.dtype || args->batch != ps.batch ||
        args->num_heads != ps.num_heads || args->head_dim != ps.head_dim ||
        args->total_tokens != ps.total_tokens || args->max_seqlen != ps.max_seqlen)
        return HSTU_ERR_BAD_SHAPE;
    if (!plan->on_device) return HSTU_ERR_NO_DEVICE_PLAN;
    if (args->total_tokens == 0) return HSTU_OK;
    if (!q || !k || !v || !out) return HSTU_ERR_NULL_ARG;
    int64_t cache_tokens = 0;
    for (const CacheSeq& c : plan->cache) cache_tokens += c.n;
    if (cache_tokens > 0 && (!k_cache || !v_cache)) return HSTU_ERR_NULL_ARG;
    if (args->rab_ts && cache_tokens > 0 && !cache_timestamps) return HSTU_ERR_NULL_ARG;
    for (const void* ptr : {q, k, v, (const void*)out, k_cache, v_cache, (const void*)cache_timestamps,
                            (const void*)args->timestamps, (const void*)args->rab_pos,
                            (const void*)args->rab_ts})
        if (ptr && !aligned16(ptr)) return HSTU_ERR_MISALIGNED;
    const size_t need = hstu_workspace_bytes(plan, 5, 0);
    if (need > 0) {
        if (!ws) return HSTU_ERR_NULL_ARG;
        if (ws_bytes < need) return HSTU_ERR_WORKSPACE_TOO_SMALL;
        if (!aligned16(ws)) return HSTU_ERR_MISALIGNED;
    }
    hstu::AttnParams p = base_params(plan, args);
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.part = plan->parts ? static_cast<float*>(ws) : nullptr;
    p.cache = plan->d_cache;
    p.kc = k_cache;
    p.vc = v_cache;
    p.ts_cache = args->rab_ts ? cache_timestamps : nullptr;
    p.ld_cache = int64_t(args->num_heads) * args->head_dim;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(checked(hstu::launch_attn_fwd_bf16(p, s), s));
}

hstu_status_t hstu_jagged_select(int32_t batch, const int64_t* src_offsets, int64_t src_rows,
                                 const int64_t* dst_offsets, int64_t dst_rows,
                                 const int64_t* keep_start, int64_t row_bytes, const void* src,
                                 void* dst, void* stream) {
    if (batch < 0 || src_rows < 0 || dst_rows < 0 || row_bytes <= 0) return HSTU_ERR_BAD_SHAPE;
    if (row_bytes % 8 != 0) return HSTU_ERR_MISALIGNED;
    if (dst_rows == 0) return HSTU_OK;
    if (batch == 0) return HSTU_ERR_BAD_SHAPE;
    if (!src_offsets || !dst_offsets || !src || !dst) return HSTU_ERR_NULL_ARG;
    for (const void* ptr : {(const void*)src_offsets, (const void*)dst_offsets,
                            (const void*)keep_start, src, (const void*)dst})
        if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 7) != 0) return HSTU_ERR_MISALIGNED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(checked(hstu::launch_jagged_select(batch, src_offsets, src_rows, dst_offsets,
                                                         dst_rows, keep_start, row_bytes, src, dst, s),
                              s));
}

}  // extern "C"
