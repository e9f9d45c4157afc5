// Host-only driver for the plan builder, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitizer.py).  It links the library's host code (hstu_api.hip, compiled for the
// host only) with stub kernel launchers, reads problems from stdin and, for each, builds host-only
// plans and reads back everything a plan reports.  No GPU call is made: host-only plans never
// touch the device, and the stubs fail if anything tries to launch.
//
// Input, one problem per line:
//   kind dtype H d nc B n_0 .. n_{B-1} t_0 .. t_{B-1}
// kind 0: a regular plan (t = candidates per sequence); kind 1: a cached plan (n = cache lengths,
// t = candidates per user).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <iostream>
#include <vector>

#include "hstu.h"
#include "kernels.h"

namespace hstu {
// Launch stubs: a host-only plan must never reach them.
#define HSTU_STUB(name, ...)                                  \
    hipError_t name(__VA_ARGS__) {                            \
        std::fprintf(stderr, "unexpected launch: %s\n", #name); \
        std::abort();                                         \
    }
HSTU_STUB(launch_attn_fwd_bf16, const AttnParams&, hipStream_t)
HSTU_STUB(launch_attn_fwd_f32, const AttnParams&, hipStream_t)
HSTU_STUB(launch_attn_bwd_dkdv_bf16, const AttnParams&, hipStream_t)
HSTU_STUB(launch_attn_bwd_dq_bf16, const AttnParams&, hipStream_t)
HSTU_STUB(launch_attn_bwd_dkdv_f32, const AttnParams&, hipStream_t)
HSTU_STUB(launch_attn_bwd_dq_f32, const AttnParams&, hipStream_t)
HSTU_STUB(launch_zero_f32, float*, int64_t, hipStream_t)
HSTU_STUB(launch_zero_f32_list, float* const*, const int64_t*, int, hipStream_t)
HSTU_STUB(launch_ln_gate_bf16, const void*, const void*, int64_t, void*, int64_t, int32_t, float,
          hipStream_t)
HSTU_STUB(launch_ln_gate_f32, const void*, const void*, int64_t, void*, int64_t, int32_t, float,
          hipStream_t)
HSTU_STUB(launch_ln_gate_bwd_bf16, const void*, const void*, const void*, int64_t, const float*,
          void*, void*, void*, int64_t, int64_t, int32_t, float, hipStream_t)
HSTU_STUB(launch_gemm, const GemmArgs&, hipStream_t)
HSTU_STUB(launch_jagged_select, int32_t, const int64_t*, int64_t, const int64_t*, int64_t,
          const int64_t*, int64_t, const void*, void*, hipStream_t)
#undef HSTU_STUB
}  // namespace hstu

namespace {

int fail(const char* what, int code) {
    std::fprintf(stderr, "%s: status %d\n", what, code);
    return 1;
}

// Reads everything the plan reports back into host memory.
int inspect(const hstu_plan_t* plan, int64_t* checksum) {
    hstu_plan_info_t info{};
    hstu_status_t st = hstu_plan_info(plan, &info);
    if (st != HSTU_OK) return fail("plan_info", st);
    *checksum += info.visible_pairs + info.fwd_units + info.bwd_units + info.fwd_tiles +
                 info.fwd_items + info.fwd_split_blocks + info.bwd_ds_bytes;
    for (int op = 0; op < 3; ++op) {
        int64_t count = 0;
        st = hstu_plan_units(plan, op, nullptr, 0, &count);
        if (st != HSTU_OK) return fail("plan_units count", st);
        const int width = op == 2 ? 8 : 4;
        std::vector<int32_t> units(static_cast<size_t>(count) * width + 1);
        st = hstu_plan_units(plan, op, units.data(), count, &count);
        if (st != HSTU_OK) return fail("plan_units", st);
        for (int64_t i = 0; i < count * width; ++i) *checksum += units[i];
    }
    for (int op = 0; op < 6; ++op) *checksum += (int64_t)hstu_workspace_bytes(plan, op, 512);
    return 0;
}

}  // namespace

int main() {
    int kind, dtype, H, d, nc, B;
    int problems = 0;
    int64_t checksum = 0;
    while (std::cin >> kind >> dtype >> H >> d >> nc >> B) {
        std::vector<int64_t> n(B), t(B);
        for (auto& x : n) std::cin >> x;
        for (auto& x : t) std::cin >> x;
        std::vector<int64_t> off(B + 1, 0), toff(B + 1, 0);
        int64_t maxn = 1;
        for (int b = 0; b < B; ++b) {
            off[b + 1] = off[b] + n[b];
            toff[b + 1] = toff[b] + t[b];
            maxn = std::max(maxn, kind == 1 ? n[b] + t[b] : n[b]);
        }
        hstu_attn_args_t a{};
        a.dtype = dtype;
        a.batch = B;
        a.num_heads = H;
        a.head_dim = d;
        a.max_seqlen = (int32_t)maxn;
        a.num_contexts = nc;
        a.alpha = 0.125f;
        hstu_plan_t* plan = nullptr;
        hstu_status_t st;
        if (kind == 0) {
            a.total_tokens = off[B];
            std::vector<int32_t> nt(t.begin(), t.end());
            st = hstu_plan_create(&a, off.data(), nt.data(), HSTU_PLAN_HOST_ONLY, &plan);
        } else {
            a.total_tokens = toff[B];
            st = hstu_plan_create_cached(&a, toff.data(), off.data(), HSTU_PLAN_HOST_ONLY, &plan);
        }
        if (st != HSTU_OK) return fail("plan_create", st);
        if (inspect(plan, &checksum)) return 1;
        hstu_plan_destroy(plan);
        ++problems;
    }
    std::printf("problems %d checksum %lld\n", problems, (long long)checksum);
    return problems > 0 ? 0 : 1;
}
