// launch_seq.h -- the scan_seq launcher: picks the kernel form for a call
// (input type, wide or element loads, softplus, gate, discretisation, cross
// scan, dz), cuts L into segments and launches.  Included only by the
// translation units that instantiate it.
#pragma once

#include "ss_host.h"

namespace ss_host {

// scan_seq writing dz, for the state sizes the backward takes (none above).
template <typename TIn, int SC, int NSW, int T, bool WIDE, bool SP, bool ZOH = false>
constexpr void (*dz_kernel())(ss::ScanParams) {
    if constexpr (SC * NSW <= SS_MAX_BWD_STATE)
        return ss::scan_seq<TIn, SC, NSW, T, WIDE, SP, true, ZOH, false, true>;
    else
        return nullptr;
}

template <typename TIn, int SC, int NSW>
int launch_seq(ss::ScanParams p, SeqMode mode, void* ws, size_t ws_bytes, hipStream_t st) {
    constexpr int TW = ss::seq_chunk<TIn, SC, NSW, true>(), TN = ss::seq_chunk<TIn, SC, NSW, false>();
    constexpr int threads = (SC + ss::kSeqElemWaves + 1) * 64;
    const int64_t G = p.b * p.nblk_d;
    if (!ws || ws_bytes < seq_workspace(p.b, p.d_in, p.n, 1).total) return SS_ERR_WORKSPACE;

    // Wide path: whole 16-byte pieces per row and 16-byte aligned u, delta, z
    // (and dy); y (dz) aligned for V-element stores (the cross scan adds to y
    // element by element).  The cross scan has no gate.
    const bool dz = mode == SeqMode::Dz || mode == SeqMode::ZohDz;
    const void* out = dz ? p.dz : p.y;
    const bool wide = (p.d_in * int64_t(sizeof(TIn))) % 16 == 0 && aligned(p.u, 16) &&
                      aligned(p.delta, 16) && (!p.z || aligned(p.z, 16)) &&
                      (!dz || aligned(p.dy, 16)) &&
                      (!p.ypre || aligned(p.ypre, (TW / ss::kSeqElemWaves) * sizeof(TIn))) &&
                      (mode == SeqMode::Cross || aligned(out, (TW / ss::kSeqElemWaves) * sizeof(TIn)));
    const int T = wide ? TW : TN;
    const int variant = mode == SeqMode::Cross   ? 12 + (wide ? 2 : 0) + (p.softplus ? 1 : 0)
                        : mode == SeqMode::Dz    ? 16 + (wide ? 2 : 0) + (p.softplus ? 1 : 0)
                        : mode == SeqMode::ZohDz ? 20 + (wide ? 2 : 0) + (p.softplus ? 1 : 0)
                        : ((mode == SeqMode::Zoh ? (wide ? 24 : 8) : wide ? 4 : 0) | (p.softplus ? 2 : 0) | (p.z ? 1 : 0));
    using Kern = void (*)(ss::ScanParams);
    static constexpr Kern kernels[28] = {
        ss::scan_seq<TIn, SC, NSW, TN, false, false, false, false, false>,
        ss::scan_seq<TIn, SC, NSW, TN, false, false, true, false, false>,
        ss::scan_seq<TIn, SC, NSW, TN, false, true, false, false, false>,
        ss::scan_seq<TIn, SC, NSW, TN, false, true, true, false, false>,
        ss::scan_seq<TIn, SC, NSW, TW, true, false, false, false, false>,
        ss::scan_seq<TIn, SC, NSW, TW, true, false, true, false, false>,
        ss::scan_seq<TIn, SC, NSW, TW, true, true, false, false, false>,
        ss::scan_seq<TIn, SC, NSW, TW, true, true, true, false, false>,
        ss::scan_seq<TIn, SC, NSW, TN, false, false, false, true, false>,
        ss::scan_seq<TIn, SC, NSW, TN, false, false, true, true, false>,
        ss::scan_seq<TIn, SC, NSW, TN, false, true, false, true, false>,
        ss::scan_seq<TIn, SC, NSW, TN, false, true, true, true, false>,
        ss::scan_seq<TIn, SC, NSW, TN, false, false, false, false, true>,
        ss::scan_seq<TIn, SC, NSW, TN, false, true, false, false, true>,
        ss::scan_seq<TIn, SC, NSW, TW, true, false, false, false, true>,
        ss::scan_seq<TIn, SC, NSW, TW, true, true, false, false, true>,
        dz_kernel<TIn, SC, NSW, TN, false, false>(),
        dz_kernel<TIn, SC, NSW, TN, false, true>(),
        dz_kernel<TIn, SC, NSW, TW, true, false>(),
        dz_kernel<TIn, SC, NSW, TW, true, true>(),
        dz_kernel<TIn, SC, NSW, TN, false, false, true>(),
        dz_kernel<TIn, SC, NSW, TN, false, true, true>(),
        dz_kernel<TIn, SC, NSW, TW, true, false, true>(),
        dz_kernel<TIn, SC, NSW, TW, true, true, true>(),
        ss::scan_seq<TIn, SC, NSW, TW, true, false, false, true, false>,
        ss::scan_seq<TIn, SC, NSW, TW, true, false, true, true, false>,
        ss::scan_seq<TIn, SC, NSW, TW, true, true, false, true, false>,
        ss::scan_seq<TIn, SC, NSW, TW, true, true, true, true, false>};
    const Kern kern = kernels[variant];
    if (!kern) return SS_ERR_UNSUPPORTED;
    const size_t lds = wide ? ss::SeqLds<TW, SC, SC * NSW, sizeof(TIn), true>::bytes
                            : ss::SeqLds<TN, SC, SC * NSW, sizeof(TIn), false>::bytes;

    const int cus = device_cus();
    const int per_cu = resident_per_cu(reinterpret_cast<const void*>(kern), threads, lds);
    int K = choose_segments(G, p.L, T, int64_t(std::max(cus, 0)) * per_cu);
    while (K > 1 && G * K > kMaxWorkgroups) K--;   // a launch holds fewer than 2^32 work-items
    // Fewer segments where the workspace is smaller than the query asks:
    // results are the same, since every segment starts from the exact state
    // its predecessor ended with.
    while (K > 1 && seq_workspace(p.b, p.d_in, p.n, K).total > ws_bytes) K--;
    int64_t Lseg = (p.L + K - 1) / K;
    Lseg = (Lseg + T - 1) / T * T;
    K = int((p.L + Lseg - 1) / Lseg);
    p.K = K;
    p.Lseg = Lseg;
    const SeqWorkspace w = seq_workspace(p.b, p.d_in, p.n, K);
    char* base = static_cast<char*>(ws);
    p.ctl = reinterpret_cast<uint32_t*>(base);
    p.handoff = reinterpret_cast<float*>(base + w.ctl);
    p.spin_limit = spin_limit();
    p.wait_never = test_plan().wait_never.load(std::memory_order_relaxed);
    if (K > 1) {
        const size_t words = size_t(ss::kFlagOffset) + size_t(G) * K;
        const int rb = int(std::min<size_t>(1024, (words + 255) / 256));
        hipLaunchKernelGGL(ss::scan_ctl_reset, dim3(rb), dim3(256), 0, st, p.ctl, int64_t(words), p.err);
        if (hipGetLastError() != hipSuccess) return SS_ERR_HIP;
    }
    hipLaunchKernelGGL(kern, dim3(unsigned(G * K)), dim3(threads), lds, st, p);
    return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
}

}  // namespace ss_host
