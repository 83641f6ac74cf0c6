// launch_bwd.h -- the scan_bwd launcher (kernel form, segments along L).
// Included only by the translation units that instantiate it.
#pragma once

#include "ss_host.h"

namespace ss_host {

// Launches scan_bwd, cut into segments along L as the forward is (same rule:
// balance the resident workgroups); p.K and p.Lseg are set here and the
// number of segments is returned in *segments.
template <typename TIn, int SC, int NSW>
int launch_bwd(ss::BwdParams p, bool gate, bool zoh, hipStream_t st, int* segments) {
    constexpr int threads = (SC + 4) * 64;
    constexpr int T = ss::kCkptSteps;
    using Kern = void (*)(ss::BwdParams);
    static constexpr Kern kernels[8] = {
        ss::scan_bwd<TIn, SC, NSW, false, false, false>, ss::scan_bwd<TIn, SC, NSW, false, true, false>,
        ss::scan_bwd<TIn, SC, NSW, true, false, false>,  ss::scan_bwd<TIn, SC, NSW, true, true, false>,
        ss::scan_bwd<TIn, SC, NSW, false, false, true>,  ss::scan_bwd<TIn, SC, NSW, false, true, true>,
        ss::scan_bwd<TIn, SC, NSW, true, false, true>,   ss::scan_bwd<TIn, SC, NSW, true, true, true>};
    const Kern kern = kernels[(zoh ? 4 : 0) | (p.softplus ? 2 : 0) | (gate ? 1 : 0)];
    const size_t lds = ss::BwdLds<SC, SC * NSW>::bytes;
    const int64_t G = p.b * p.nblk_d;
    const int cus = device_cus();
    const int per_cu = resident_per_cu(reinterpret_cast<const void*>(kern), threads, lds);
    int K = choose_segments(G, p.L, T, int64_t(std::max(cus, 0)) * per_cu);
    while (K > 1 && G * K > kMaxWorkgroups) K--;
    int64_t Lseg = (p.L + K - 1) / K;
    Lseg = (Lseg + T - 1) / T * T;
    K = int((p.L + Lseg - 1) / Lseg);
    p.K = K;
    p.Lseg = Lseg;
    *segments = K;
    if (K > 1) {
        const size_t words = size_t(ss::kFlagOffset) + size_t(G) * K;
        const int rb = int(std::min<size_t>(1024, (words + 255) / 256));
        hipLaunchKernelGGL(ss::scan_ctl_reset, dim3(rb), dim3(256), 0, st, p.ctl, int64_t(words));
        if (hipGetLastError() != hipSuccess) return SS_ERR_HIP;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(G * K)), dim3(threads), lds, st, p);
    return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
}

}  // namespace ss_host
