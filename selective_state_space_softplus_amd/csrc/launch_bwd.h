// launch_bwd.h -- the scan_bwd launcher (kernel form, segments along L).
// Included only by the translation units that instantiate it.
#pragma once

#include "ss_host.h"

namespace ss_host {

// Launches scan_bwd (SL: the form for n taken in several slices of states),
// cut into segments along L as the forward is (same rule: balance the
// resident workgroups); p.K and p.Lseg are set here and the number of
// segments is returned in *segments.
template <typename TIn, int SC, int NSW, bool SL>
int launch_bwd(ss::BwdParams p, bool gate, bool zoh, hipStream_t st, int* segments) {
    constexpr int threads = (SC + 4) * 64;
    constexpr int T = ss::kCkptSteps;
    using Kern = void (*)(ss::BwdParams);
    static constexpr Kern kernels[16] = {
        ss::scan_bwd<TIn, SC, NSW, SL, false, false, false, false>,
        ss::scan_bwd<TIn, SC, NSW, SL, false, true, false, false>,
        ss::scan_bwd<TIn, SC, NSW, SL, true, false, false, false>,
        ss::scan_bwd<TIn, SC, NSW, SL, true, true, false, false>,
        ss::scan_bwd<TIn, SC, NSW, SL, false, false, true, false>,
        ss::scan_bwd<TIn, SC, NSW, SL, false, true, true, false>,
        ss::scan_bwd<TIn, SC, NSW, SL, true, false, true, false>,
        ss::scan_bwd<TIn, SC, NSW, SL, true, true, true, false>,
        ss::scan_bwd<TIn, SC, NSW, SL, false, false, false, true>,
        ss::scan_bwd<TIn, SC, NSW, SL, false, true, false, true>,
        ss::scan_bwd<TIn, SC, NSW, SL, true, false, false, true>,
        ss::scan_bwd<TIn, SC, NSW, SL, true, true, false, true>,
        ss::scan_bwd<TIn, SC, NSW, SL, false, false, true, true>,
        ss::scan_bwd<TIn, SC, NSW, SL, false, true, true, true>,
        ss::scan_bwd<TIn, SC, NSW, SL, true, false, true, true>,
        ss::scan_bwd<TIn, SC, NSW, SL, true, true, true, true>};
    // Channel pairs: an element thread's two channels adjacent, so each row's
    // two elements move in one access; needs d_in even and every per-element
    // tensor aligned to two elements.
    auto pair_ok = [](const void* q) { return !q || aligned(q, 2 * sizeof(TIn)); };
    const bool pr = p.d_in % 2 == 0 && pair_ok(p.u) && pair_ok(p.delta) && (!gate || pair_ok(p.z)) &&
                    pair_ok(p.dy) && pair_ok(p.ypre) && pair_ok(p.dz) && pair_ok(p.du) && pair_ok(p.ddelta) &&
                    (!p.part_du || aligned(p.part_du, 8)) && (!p.part_dd || aligned(p.part_dd, 8));
    const Kern kern = kernels[(pr ? 8 : 0) | (zoh ? 4 : 0) | (p.softplus ? 2 : 0) | (gate ? 1 : 0)];
    const size_t lds = ss::BwdLds<SC, SC * NSW>::bytes;
    const int64_t G = p.b * p.nblk_d * p.slices;
    const int cus = device_cus();
    const int per_cu = resident_per_cu(reinterpret_cast<const void*>(kern), threads, lds);
    int K = choose_segments(G, p.L, T, int64_t(std::max(cus, 0)) * per_cu);
    while (K > 1 && G * K > kMaxWorkgroups) K--;
    int64_t Lseg = (p.L + K - 1) / K;
    Lseg = (Lseg + T - 1) / T * T;
    K = int((p.L + Lseg - 1) / Lseg);
    p.K = K;
    p.Lseg = Lseg;
    p.spin_limit = spin_limit();
    p.wait_never = test_plan().wait_never.load(std::memory_order_relaxed);
    *segments = K;
    if (K > 1) {
        // The status words were cleared by the forward pass of this call.
        const size_t words = size_t(ss::kFlagOffset) + size_t(G) * K;
        const int rb = int(std::min<size_t>(1024, (words + 255) / 256));
        hipLaunchKernelGGL(ss::scan_ctl_reset, dim3(rb), dim3(256), 0, st, p.ctl, int64_t(words), nullptr);
        if (hipGetLastError() != hipSuccess) return SS_ERR_HIP;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(G * K)), dim3(threads), lds, st, p);
    return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
}

}  // namespace ss_host
