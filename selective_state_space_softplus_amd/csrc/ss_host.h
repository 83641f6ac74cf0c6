// ss_host.h -- host-side planning shared by the library's translation units:
// size limits, launch shapes, workspace layouts, device queries, the segment
// count along L, and the scan_seq / scan_bwd launchers, which launch_seq.h
// and launch_bwd.h define and one translation unit per input type and kernel
// family instantiates (so the kernels compile in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "ss_scan.h"
#include "scan_bwd_kernels.h"
#include "scan_kernels.h"

namespace ss_host {

constexpr int kMaxSegments = 16;
constexpr int64_t kMaxElems = int64_t(1) << 46;   // keeps every index product far from int64 overflow
constexpr int kTparWaves = 8;
// Largest grid in workgroups of up to 1024 threads: a launch holds at most 2^32 - 1 work-items.
constexpr int64_t kMaxWorkgroups = (int64_t(1) << 22) - 1;
// Longest sequence: per-segment time indices of scan_seq are 32-bit.
constexpr int64_t kMaxLength = (int64_t(1) << 31) - 1024;
// LDS one workgroup may take on gfx950.
constexpr size_t kMaxLdsBytes = 160 * 1024;
// Largest b * d_in of the decode step (up to 16 threads per channel in one launch).
constexpr int64_t kMaxStepChannels = (int64_t(1) << 28) - 1;

inline bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Grid of a grid-stride kernel of 256-thread workgroups over `items` items:
// one item per thread up to 2^20 workgroups, so the launch stays far below
// the 2^32 - 1 work-items a launch may hold.
inline dim3 grid_1d(int64_t items) {
    return dim3(unsigned(std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, int64_t(1) << 20))));
}

// Overrides of the launch plan set by ss_set_test_plan (tests and tuning
// only; every field 0 = the library's own choice).  Each changes how the work
// is split, never what is computed.
struct TestPlan {
    std::atomic<int> segments{0};    // segments along L, 1..kMaxSegments
    std::atomic<int> waves{0};       // 4: 4 recurrence waves of 4 states at 9 <= n <= 16
    std::atomic<int> tpar{0};        // 1: scan_tpar for n <= 2 (zero initial state, Euler)
    std::atomic<int> spin_limit{0};  // polls before a segment wait gives up
    std::atomic<int> wait_never{0};  // 1: segment waits poll a word nothing sets (they all give up)
};

inline TestPlan& test_plan() {
    static TestPlan plan;
    return plan;
}

inline int spin_limit() {
    const int v = test_plan().spin_limit.load(std::memory_order_relaxed);
    return v > 0 ? v : ss::kSpinLimit;
}

struct SeqShape {
    int SC;    // recurrence waves per workgroup
    int NSW;   // states per recurrence wave
};

// Recurrence waves and states per wave (the test plan may take 4 waves of 4
// states at 9 <= n <= 16).
inline SeqShape seq_shape(int64_t n) {
    const int want = test_plan().waves.load(std::memory_order_relaxed);
    if (n <= 2) return {1, 2};
    if (n <= 8) return {4, 2};
    if (n <= 16) return want == 4 ? SeqShape{4, 4} : SeqShape{8, 2};
    if (n <= 32) return {8, 4};
    return {8, 8};
}

// Recurrence waves and states per wave of scan_bwd (n <= 64).
// Backward shapes: at most 16 states per workgroup; larger n is taken in
// slices of 16 states by separate workgroups (bwd_slices), so that each
// recurrence wave keeps two states' chunk of values in registers.
inline SeqShape bwd_shape(int64_t n) {
    if (n <= 2) return {1, 2};
    if (n <= 8) return {4, 2};
    return {8, 2};
}

inline int64_t bwd_slices(int64_t n) {
    const SeqShape sh = bwd_shape(n);
    const int64_t np = int64_t(sh.SC) * sh.NSW;
    return (n + np - 1) / np;
}

// Workspace of scan_seq cut into K segments, in order: control words (ticket
// counter, one flag per (segment, group)) and the states published between
// segments.  The size asked of callers is that for kMaxSegments.
struct SeqWorkspace {
    size_t ctl, handoff, total;
};

inline SeqWorkspace seq_workspace(int64_t b, int64_t d_in, int64_t n, int K = kMaxSegments) {
    const int64_t G = b * ((d_in + 63) / 64);
    SeqWorkspace w;
    w.ctl = ((size_t(ss::kFlagOffset) + (K > 1 ? size_t(G) * size_t(K) : 0)) * sizeof(uint32_t) + 255) / 256 * 256;
    w.handoff = (size_t(K - 1) * size_t(G) * size_t(n) * 64 * sizeof(float) + 255) / 256 * 256;
    w.total = w.ctl + w.handoff;
    return w;
}

inline int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < 64 && cached[dev].load(std::memory_order_relaxed) > 0) return cached[dev].load(std::memory_order_relaxed);
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Workgroups of `fn` that fit on one compute unit at once (cached per kernel
// and device; 0 when unknown).
inline int resident_per_cu(const void* fn, int threads, size_t lds) {
    static std::mutex mu;
    static std::map<std::pair<const void*, int>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const auto key = std::make_pair(fn, dev);
    {
        std::lock_guard<std::mutex> g(mu);
        const auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, threads, lds) != hipSuccess) nb = 0;
    std::lock_guard<std::mutex> g(mu);
    cache[key] = nb;
    return nb;
}

// Number of segments K along L for scan_seq.  Pieces (segment, group) are
// taken in ticket order, segment-major, by `slots` resident workgroups.  When
// the G groups fill the slots at least once, a piece's predecessor always ran
// in an earlier round, so with pieces of equal length the time is
// ceil(G K / slots) rounds of 1/K of the work each, plus a fixed cost per piece
// (pipeline fill and drain, state handoff) taken as 2% of a whole-length
// piece.  K minimises that.  With fewer groups than slots the segments of a
// group would only run one after another, so K = 1.  Every segment keeps at
// least 4 chunks.  The test plan may fix K.
inline int choose_segments(int64_t G, int64_t L, int T, int64_t slots) {
    const int64_t max_k = std::max<int64_t>(1, std::min<int64_t>(kMaxSegments, L / (4 * int64_t(T))));
    if (const int v = test_plan().segments.load(std::memory_order_relaxed); v >= 1)
        return int(std::min<int64_t>(std::min<int64_t>(v, kMaxSegments), std::max<int64_t>(1, (L + T - 1) / T)));
    if (slots <= 0 || G < slots) return 1;
    int best = 1;
    double best_t = 0.0;
    for (int64_t k = 1; k <= max_k; k++) {
        const double rounds = double((G * k + slots - 1) / slots);
        const double t = rounds * (1.0 / double(k) + 0.02);
        if (k == 1 || t < best_t * (1.0 - 1e-9)) {
            best = int(k);
            best_t = t;
        }
    }
    return best;
}

// Which family of scan_seq kernels a call needs.  Dz, ZohDz: the gated scan
// inside the backward, writing dz in place of y.
enum class SeqMode { Euler, Zoh, Cross, Dz, ZohDz };

// Launch scan_seq<TIn, SC, NSW, ...> for one call (launch_seq.h).
template <typename TIn, int SC, int NSW>
int launch_seq(ss::ScanParams p, SeqMode mode, void* ws, size_t ws_bytes, hipStream_t st);

// Launch scan_bwd<TIn, SC, NSW, SL, ...> for one call (launch_bwd.h); the
// number of segments along L is returned in *segments.
template <typename TIn, int SC, int NSW, bool SL>
int launch_bwd(ss::BwdParams p, bool gate, bool zoh, hipStream_t st, int* segments);

}  // namespace ss_host
