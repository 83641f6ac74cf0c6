// ss_scan.hip -- host side of libss_scan.so: argument validation, the choice
// of kernel and launch shape, and the C entry points declared in ss_scan.h.
//
// Nothing here allocates device memory or synchronises: every launch goes on
// the caller's stream, and the only scratch memory is the caller's workspace
// or, for ss_scan_fwd_noalloc, a static device array of fixed size.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "ss_scan.h"
#include "conv_kernels.h"
#include "cross_kernels.h"
#include "scan_bwd_kernels.h"
#include "scan_kernels.h"
#include "ss_host.h"
#include "state_update_kernels.h"

#define SS_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using namespace ss_host;
using ss::ConvParams;
using ss::ScanParams;
using ss::StepParams;


// ----------------------------------------------------------------------------- validation helpers

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range range_of(const void* p, int64_t count, size_t elem) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, p ? lo + uintptr_t(count) * elem : lo};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

size_t elem_size(int dtype) { return dtype == SS_BF16 ? 2 : 4; }

// Every scan workspace (ss_scan_fwd, ss_cross_scan_fwd, ss_scan_bwd) starts
// with the forward scan's control words; the call's status words are words
// kStatusWord and kStatusWord + 1 of it (ss_scan_status reads the first).
constexpr int kStatusWord = 1;

// a, b, c >= 1 and a * b * c <= 2^46 (checked without forming an overflowing product).
bool sizes_ok(int64_t a, int64_t b, int64_t c) {
    if (a <= 0 || b <= 0 || c <= 0) return false;
    if (a > kMaxElems / b) return false;
    return a * b <= kMaxElems / c;
}

// ----------------------------------------------------------------------------- scan planning

enum class ScanKernel { Tpar, Seq };

// scan_seq for every n; the test plan may select scan_tpar for n <= 2, which
// starts from a zero state with the delta' input weight only.
ScanKernel choose_kernel(const ScanParams& p, bool zoh) {
    if (test_plan().tpar.load(std::memory_order_relaxed) && p.n <= 2 && !p.h0 && !zoh) return ScanKernel::Tpar;
    return ScanKernel::Seq;
}

template <typename TIn>
int dispatch_seq(const ScanParams& p, SeqMode mode, void* ws, size_t ws_bytes, hipStream_t st) {
    const SeqShape sh = seq_shape(p.n);
    if (sh.SC == 1) return launch_seq<TIn, 1, 2>(p, mode, ws, ws_bytes, st);
    if (sh.SC == 4)
        return sh.NSW == 2 ? launch_seq<TIn, 4, 2>(p, mode, ws, ws_bytes, st)
                           : launch_seq<TIn, 4, 4>(p, mode, ws, ws_bytes, st);
    if (sh.NSW == 2) return launch_seq<TIn, 8, 2>(p, mode, ws, ws_bytes, st);
    if (sh.NSW == 4) return launch_seq<TIn, 8, 4>(p, mode, ws, ws_bytes, st);
    return launch_seq<TIn, 8, 8>(p, mode, ws, ws_bytes, st);
}

template <typename TIn>
int dispatch_tpar(const ScanParams& p, hipStream_t st) {
    const dim3 grid(unsigned(p.b * p.nblk_d));
    if (p.n == 1)
        hipLaunchKernelGGL((ss::scan_tpar<TIn, 1, kTparWaves>), grid, dim3(kTparWaves * 64), 0, st, p);
    else
        hipLaunchKernelGGL((ss::scan_tpar<TIn, 2, kTparWaves>), grid, dim3(kTparWaves * 64), 0, st, p);
    return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
}

template <typename TIn, int W>
void launch_conv(const ConvParams& p, bool vec, hipStream_t st) {
    const dim3 grid(unsigned((p.b * p.d_in + 255) / 256));
    constexpr int NW = sizeof(TIn) == 2 ? (W + 1) / 2 : W;
    constexpr bool can_vec = (NW == 2 || NW == 4) && W * int(sizeof(TIn)) == 4 * NW;
    if constexpr (can_vec) {
        if (vec) {
            hipLaunchKernelGGL((ss::conv_update<TIn, W, true>), grid, dim3(256), 0, st, p);
            return;
        }
    }
    hipLaunchKernelGGL((ss::conv_update<TIn, W, false>), grid, dim3(256), 0, st, p);
}

template <typename TIn>
void dispatch_conv(const ConvParams& p, int W, bool vec, hipStream_t st) {
    switch (W) {
        case 1: launch_conv<TIn, 1>(p, vec, st); break;
        case 2: launch_conv<TIn, 2>(p, vec, st); break;
        case 3: launch_conv<TIn, 3>(p, vec, st); break;
        case 4: launch_conv<TIn, 4>(p, vec, st); break;
        case 5: launch_conv<TIn, 5>(p, vec, st); break;
        case 6: launch_conv<TIn, 6>(p, vec, st); break;
        case 7: launch_conv<TIn, 7>(p, vec, st); break;
        default: launch_conv<TIn, 8>(p, vec, st); break;
    }
}

}  // namespace

// ============================================================================= C ABI

SS_EXPORT const char* ss_status_string(int status) {
    switch (status) {
        case SS_OK: return "ok";
        case SS_ERR_NULL: return "a required pointer is NULL";
        case SS_ERR_SHAPE: return "a size is <= 0 or too large";
        case SS_ERR_DTYPE: return "dtype is not SS_F32 or SS_BF16";
        case SS_ERR_UNSUPPORTED: return "state size n is above SS_MAX_STATE";
        case SS_ERR_WORKSPACE: return "workspace is missing or too small";
        case SS_ERR_HIP: return "the HIP runtime refused the launch";
        case SS_ERR_ALIAS: return "an output overlaps an input";
        case SS_ERR_ALIGN: return "a pointer is not aligned to its element size";
        case SS_ERR_MODE: return "discretization is not SS_DISC_EULER or SS_DISC_ZOH";
        case SS_ERR_TIMEOUT: return "a wait between sequence segments gave up; the outputs hold NaN";
        default: return "unknown status";
    }
}

SS_EXPORT size_t ss_scan_fwd_workspace_bytes(int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype) {
    if (dtype != SS_F32 && dtype != SS_BF16) return 0;
    if (!sizes_ok(b, L, d_in) || n <= 0 || n > SS_MAX_STATE || d_in > SS_MAX_CHANNELS) return 0;
    if (b * ((d_in + 63) / 64) > kMaxWorkgroups || L > kMaxLength) return 0;
    // Sized for scan_seq with the most segments; scan_tpar (n <= 2) needs none
    // but the same size is asked for so that either kernel can be chosen.
    return seq_workspace(b, d_in, n).total;
}

// Static scratch of ss_scan_fwd_noalloc, one copy per device, kept until the
// process ends.  Host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (in host code the
// array's own name is a host-side stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[SS_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device; null if the lookup fails.
void* scratch_address() {
    static std::mutex mu;
    static void* addr[64] = {};
    static bool done[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> g(mu);
    if (!done[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev] = ptr;
        done[dev] = true;
    }
    return addr[dev];
}

// The scan forward behind ss_scan_fwd_ex and ss_scan_fwd_noalloc.  `own_ws`:
// the workspace is the caller's, which must be as large as the query says;
// otherwise it is the library's static scratch, and the segment count is
// lowered until the scan fits in it.
// save: keep what ss_scan_bwd_saved starts from -- in ckpt the state after
// every kCkptSteps steps, (b, (L - 1) / kCkptSteps, n, d_in) fp32 (null when
// there is none, L <= kCkptSteps), and, gated, in ypre the readout before the
// gate, (b, L, d_in).
int scan_fwd_impl(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                  const float* D, const void* z, const float* delta_bias, int delta_softplus,
                  const float* initial_state, int discretization, void* y, float* last_state, float* ckpt,
                  void* ypre, int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype, void* workspace,
                  size_t workspace_bytes, bool own_ws, void* stream, bool save = false) {
    if (!u || !delta || !A_log || !B || !C || !D || !y) return SS_ERR_NULL;
    if (save && z && !ypre) return SS_ERR_NULL;
    if (!z) ypre = nullptr;
    if (!sizes_ok(b, L, d_in) || n <= 0 || d_in > SS_MAX_CHANNELS) return SS_ERR_SHAPE;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_DTYPE;
    if (n > SS_MAX_STATE) return SS_ERR_UNSUPPORTED;
    if (b * ((d_in + 63) / 64) > kMaxWorkgroups || L > kMaxLength) return SS_ERR_SHAPE;
    if (discretization != SS_DISC_EULER && discretization != SS_DISC_ZOH) return SS_ERR_MODE;
    const size_t es = elem_size(dtype);
    for (const void* p : {u, delta, B, C, z, static_cast<const void*>(y), static_cast<const void*>(ypre)})
        if (p && !aligned(p, es)) return SS_ERR_ALIGN;
    for (const void* p : {static_cast<const void*>(A_log), static_cast<const void*>(D),
                          static_cast<const void*>(delta_bias), static_cast<const void*>(initial_state),
                          static_cast<const void*>(last_state), static_cast<const void*>(ckpt)})
        if (p && !aligned(p, 4)) return SS_ERR_ALIGN;
    const int64_t nel = b * L * d_in;
    const Range ins[] = {range_of(u, nel, es), range_of(delta, nel, es), range_of(A_log, d_in * n, 4),
                         range_of(B, b * L * n, es), range_of(C, b * L * n, es), range_of(D, d_in, 4),
                         range_of(z, z ? nel : 0, es), range_of(delta_bias, delta_bias ? d_in : 0, 4)};
    const Range ry = range_of(y, nel, es);
    const Range rs = range_of(last_state, last_state ? b * d_in * n : 0, 4);
    // The initial state may be read and overwritten in place as last_state
    // (each workgroup reads its own states before it, or the last segment of
    // its channels, writes them); any other overlap with an output is refused.
    const Range rh = range_of(initial_state, initial_state ? b * d_in * n : 0, 4);
    const bool in_place = initial_state && static_cast<const void*>(initial_state) == last_state;
    for (const Range& r : ins)
        if (overlaps(r, ry) || overlaps(r, rs)) return SS_ERR_ALIAS;
    if (overlaps(ry, rs) || overlaps(rh, ry) || (!in_place && overlaps(rh, rs))) return SS_ERR_ALIAS;
    // The saved states are outputs too.
    const Range rc = range_of(ckpt, ckpt ? b * ((L - 1) / ss::kCkptSteps) * n * d_in : 0, 4);
    const Range rp = range_of(ypre, ypre ? nel : 0, es);
    for (const Range& r : ins)
        if (overlaps(r, rc) || overlaps(r, rp)) return SS_ERR_ALIAS;
    for (const Range& r : {ry, rs, rh})
        if (overlaps(r, rc) || overlaps(r, rp)) return SS_ERR_ALIAS;
    if (overlaps(rc, rp)) return SS_ERR_ALIAS;
    if (own_ws) {
        const size_t need = ss_scan_fwd_workspace_bytes(b, L, d_in, n, dtype);
        if (!workspace || workspace_bytes < need) return SS_ERR_WORKSPACE;
        // The workspace starts with 32-bit words updated by device atomics.
        if (!aligned(workspace, 256)) return SS_ERR_ALIGN;
        const Range rw = range_of(workspace, int64_t(workspace_bytes), 1);
        for (const Range& r : ins)
            if (overlaps(r, rw)) return SS_ERR_ALIAS;
        if (overlaps(ry, rw) || overlaps(rs, rw) || overlaps(rh, rw) || overlaps(rc, rw) || overlaps(rp, rw))
            return SS_ERR_ALIAS;
    } else {
        // Validation is done: only now is the device touched.
        workspace = scratch_address();
        if (!workspace) return SS_ERR_HIP;
        workspace_bytes = SS_NOALLOC_SCRATCH_BYTES;
        if (workspace_bytes < seq_workspace(b, d_in, n, 1).total) return SS_ERR_WORKSPACE;
    }

    ScanParams p{};
    p.u = u;
    p.delta = delta;
    p.A_log = A_log;
    p.B = B;
    p.C = C;
    p.D = D;
    p.z = z;
    p.bias = delta_bias;
    p.y = y;
    p.last_state = last_state;
    p.h0 = initial_state;
    p.ckpt = ckpt;
    p.nck = int((L - 1) / ss::kCkptSteps);
    p.ypre = ypre;
    p.b = b;
    p.L = L;
    p.d_in = d_in;
    p.n = n;
    p.softplus = delta_softplus ? 1 : 0;
    p.nblk_d = int((d_in + 63) / 64);
    p.K = 1;
    p.Lseg = L;
    p.err = static_cast<uint32_t*>(workspace) + kStatusWord;
    hipStream_t st = static_cast<hipStream_t>(stream);

    const bool zoh = discretization == SS_DISC_ZOH;
    if (!save && choose_kernel(p, zoh) == ScanKernel::Tpar) {
        // No segment waits: only the status words need clearing.
        hipLaunchKernelGGL(ss::scan_ctl_reset, dim3(1), dim3(64), 0, st, p.err, int64_t(0), p.err);
        if (hipGetLastError() != hipSuccess) return SS_ERR_HIP;
        return dtype == SS_BF16 ? dispatch_tpar<uint16_t>(p, st) : dispatch_tpar<float>(p, st);
    }
    const SeqMode mode = zoh ? SeqMode::Zoh : SeqMode::Euler;
    return dtype == SS_BF16 ? dispatch_seq<uint16_t>(p, mode, workspace, workspace_bytes, st)
                            : dispatch_seq<float>(p, mode, workspace, workspace_bytes, st);
}

}  // namespace

SS_EXPORT int ss_scan_fwd_ex(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int delta_softplus,
                             const float* initial_state, int discretization, void* y, float* last_state, int64_t b,
                             int64_t L, int64_t d_in, int64_t n, int dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return scan_fwd_impl(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, initial_state, discretization, y,
                         last_state, nullptr, nullptr, b, L, d_in, n, dtype, workspace, workspace_bytes, true, stream);
}

SS_EXPORT int ss_scan_fwd_save(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                               const float* D, const void* z, const float* delta_bias, int delta_softplus,
                               const float* initial_state, int discretization, void* y, float* last_state,
                               float* checkpoints, void* y_pre, int64_t b, int64_t L, int64_t d_in, int64_t n,
                               int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (!checkpoints && L > ss::kCkptSteps) return SS_ERR_NULL;   // none are kept for L <= 8
    if (n > SS_MAX_BWD_STATE) return SS_ERR_UNSUPPORTED;
    return scan_fwd_impl(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, initial_state, discretization, y,
                         last_state, L > ss::kCkptSteps ? checkpoints : nullptr, y_pre, b, L, d_in, n, dtype,
                         workspace, workspace_bytes, true, stream, true);
}

SS_EXPORT int ss_scan_fwd_noalloc(const void* u, const void* delta, const float* A_log, const void* B,
                                  const void* C, const float* D, const void* z, const float* delta_bias,
                                  int delta_softplus, const float* initial_state, int discretization, void* y,
                                  float* last_state, int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                                  void* stream) {
    return scan_fwd_impl(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, initial_state, discretization, y,
                         last_state, nullptr, nullptr, b, L, d_in, n, dtype, nullptr, 0, false, stream);
}

SS_EXPORT int ss_scan_status(const void* workspace, size_t workspace_bytes, int32_t* status, void* stream) {
    if (!status) return SS_ERR_NULL;
    if (!workspace) {
        // The static scratch of ss_scan_fwd_noalloc on the current device.
        workspace = scratch_address();
        if (!workspace) return SS_ERR_HIP;
        workspace_bytes = SS_NOALLOC_SCRATCH_BYTES;
    }
    if (workspace_bytes < 256) return SS_ERR_WORKSPACE;
    if (!aligned(workspace, 256) || !aligned(status, 4)) return SS_ERR_ALIGN;
    hipLaunchKernelGGL(ss::scan_status_copy, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint32_t*>(workspace) + kStatusWord, status);
    return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
}

SS_EXPORT int ss_set_test_plan(int segments, int waves, int time_parallel, int spin_limit, int wait_never) {
    if (segments < 0 || segments > kMaxSegments || (waves != 0 && waves != 4) || spin_limit < 0 ||
        (time_parallel != 0 && time_parallel != 1) || (wait_never != 0 && wait_never != 1))
        return SS_ERR_SHAPE;
    TestPlan& t = test_plan();
    t.segments.store(segments);
    t.waves.store(waves);
    t.tpar.store(time_parallel);
    t.spin_limit.store(spin_limit);
    t.wait_never.store(wait_never);
    return SS_OK;
}

SS_EXPORT int ss_scan_fwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, int delta_softplus, void* y,
                          float* last_state, int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return ss_scan_fwd_ex(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, nullptr, SS_DISC_EULER, y,
                          last_state, b, L, d_in, n, dtype, workspace, workspace_bytes, stream);
}

SS_EXPORT int ss_state_update_ex(float* state, const void* x, const void* dt, const float* A_log, const void* B,
                                 const void* C, const float* D, const void* z, const float* dt_bias, int dt_softplus,
                                 int discretization, void* y, int64_t b, int64_t d_in, int64_t n, int dtype,
                                 void* stream) {
    if (!state || !x || !dt || !A_log || !B || !C || !D || !y) return SS_ERR_NULL;
    if (!sizes_ok(b, d_in, 1) || n <= 0 || !sizes_ok(b, d_in, n) || b * d_in > kMaxStepChannels) return SS_ERR_SHAPE;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_DTYPE;
    if (n > SS_MAX_STATE) return SS_ERR_UNSUPPORTED;
    if (discretization != SS_DISC_EULER && discretization != SS_DISC_ZOH) return SS_ERR_MODE;
    const size_t es = elem_size(dtype);
    for (const void* p : {x, dt, B, C, z, static_cast<const void*>(y)})
        if (p && !aligned(p, es)) return SS_ERR_ALIGN;
    for (const void* p : {static_cast<const void*>(state), static_cast<const void*>(A_log),
                          static_cast<const void*>(D), static_cast<const void*>(dt_bias)})
        if (p && !aligned(p, 4)) return SS_ERR_ALIGN;
    const int64_t nch = b * d_in;
    const Range ins[] = {range_of(x, nch, es), range_of(dt, nch, es), range_of(A_log, d_in * n, 4),
                         range_of(B, b * n, es), range_of(C, b * n, es), range_of(D, d_in, 4),
                         range_of(z, z ? nch : 0, es), range_of(dt_bias, dt_bias ? d_in : 0, 4)};
    const Range ry = range_of(y, nch, es);
    const Range rs = range_of(state, nch * n, 4);
    for (const Range& r : ins)
        if (overlaps(r, ry) || overlaps(r, rs)) return SS_ERR_ALIAS;
    if (overlaps(ry, rs)) return SS_ERR_ALIAS;

    StepParams p{};
    p.state = state;
    p.x = x;
    p.dt = dt;
    p.A_log = A_log;
    p.B = B;
    p.C = C;
    p.D = D;
    p.z = z;
    p.bias = dt_bias;
    p.y = y;
    p.b = b;
    p.d_in = d_in;
    p.n = n;
    p.softplus = dt_softplus ? 1 : 0;
    p.zoh = discretization == SS_DISC_ZOH ? 1 : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);

    // The vector kernel takes n = 4 lpc, forms offsets within one batch row
    // of the state in 32 bits, and covers lpc rows of 256 / lpc channels per
    // workgroup.
    const int64_t lpc = n % 4 == 0 ? n / 4 : 0;
    const bool lpc_ok = lpc == 1 || lpc == 2 || lpc == 4 || lpc == 8 || lpc == 16;
    const int64_t tiles = lpc_ok ? (d_in * lpc + 255) / 256 : 0, groups = lpc_ok ? (b + lpc - 1) / lpc : 0;
    const bool vec = lpc_ok && d_in * n < (int64_t(1) << 31) && tiles * groups < (int64_t(1) << 31) &&
                     aligned(state, 16) && aligned(A_log, 16) && aligned(B, 4 * es) && aligned(C, 4 * es);
    if (vec) {
        const dim3 grid(unsigned(tiles * groups));
#define SS_STEP_VEC(T_, LPC_)                                                            \
    if (p.zoh)                                                                           \
        hipLaunchKernelGGL((ss::state_update_vec<T_, LPC_, true>), grid, dim3(256), 0, st, p); \
    else                                                                                 \
        hipLaunchKernelGGL((ss::state_update_vec<T_, LPC_, false>), grid, dim3(256), 0, st, p)
        if (dtype == SS_BF16) {
            switch (lpc) {
                case 1: SS_STEP_VEC(uint16_t, 1); break;
                case 2: SS_STEP_VEC(uint16_t, 2); break;
                case 4: SS_STEP_VEC(uint16_t, 4); break;
                case 8: SS_STEP_VEC(uint16_t, 8); break;
                default: SS_STEP_VEC(uint16_t, 16); break;
            }
        } else {
            switch (lpc) {
                case 1: SS_STEP_VEC(float, 1); break;
                case 2: SS_STEP_VEC(float, 2); break;
                case 4: SS_STEP_VEC(float, 4); break;
                case 8: SS_STEP_VEC(float, 8); break;
                default: SS_STEP_VEC(float, 16); break;
            }
        }
#undef SS_STEP_VEC
    } else {
        const dim3 grid(unsigned((nch + 255) / 256));
        if (dtype == SS_BF16)
            hipLaunchKernelGGL((ss::state_update_any<uint16_t>), grid, dim3(256), 0, st, p);
        else
            hipLaunchKernelGGL((ss::state_update_any<float>), grid, dim3(256), 0, st, p);
    }
    return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
}

SS_EXPORT int ss_state_update(float* state, const void* x, const void* dt, const float* A_log, const void* B,
                              const void* C, const float* D, const void* z, const float* dt_bias, int dt_softplus,
                              void* y, int64_t b, int64_t d_in, int64_t n, int dtype, void* stream) {
    return ss_state_update_ex(state, x, dt, A_log, B, C, D, z, dt_bias, dt_softplus, SS_DISC_EULER, y, b, d_in, n,
                              dtype, stream);
}

SS_EXPORT int ss_conv_update(void* conv_state, const void* x, const float* weight, const float* bias, int silu,
                             void* out, int64_t b, int64_t d_in, int64_t W, int dtype, void* stream) {
    if (!conv_state || !x || !weight || !out) return SS_ERR_NULL;
    if (!sizes_ok(b, d_in, 1) || W <= 0 || b * d_in > kMaxStepChannels) return SS_ERR_SHAPE;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_DTYPE;
    if (W > SS_MAX_CONV_WIDTH) return SS_ERR_UNSUPPORTED;
    const size_t es = elem_size(dtype);
    for (const void* p : {static_cast<const void*>(conv_state), x, static_cast<const void*>(out)})
        if (!aligned(p, es)) return SS_ERR_ALIGN;
    for (const void* p : {static_cast<const void*>(weight), static_cast<const void*>(bias)})
        if (p && !aligned(p, 4)) return SS_ERR_ALIGN;
    const int64_t nch = b * d_in;
    const Range rs = range_of(conv_state, nch * W, es);
    const Range ro = range_of(out, nch, es);
    const Range ins[] = {range_of(x, nch, es), range_of(weight, d_in * W, 4), range_of(bias, bias ? d_in : 0, 4)};
    for (const Range& r : ins)
        if (overlaps(r, rs) || overlaps(r, ro)) return SS_ERR_ALIAS;
    if (overlaps(rs, ro)) return SS_ERR_ALIAS;

    ConvParams p{};
    p.state = conv_state;
    p.x = x;
    p.weight = weight;
    p.bias = bias;
    p.out = out;
    p.b = b;
    p.d_in = d_in;
    p.silu = silu ? 1 : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // A channel's window is one 8- or 16-byte access when it is that long and so aligned.
    const bool vec = aligned(conv_state, size_t(W) * es);
    if (dtype == SS_BF16)
        dispatch_conv<uint16_t>(p, int(W), vec, st);
    else
        dispatch_conv<float>(p, int(W), vec, st);
    return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
}

// Per-direction outputs of the cross scan, (4 maps, L, d_in) fp32, placed
// before the scan's own workspace.
size_t cross_ys_bytes(int64_t maps, int64_t L, int64_t d_in) {
    return (size_t(4 * maps) * size_t(L) * size_t(d_in) * sizeof(float) + 255) / 256 * 256;
}

bool cross_sizes_ok(int64_t maps, int64_t H, int64_t W, int64_t d_in, int64_t n) {
    if (!sizes_ok(maps, H, W) || d_in <= 0 || n <= 0 || d_in > SS_MAX_CHANNELS || maps > kMaxElems / 4) return false;
    const int64_t b = 4 * maps, L = H * W;
    return sizes_ok(b, L, d_in) && b * ((d_in + 63) / 64) <= kMaxWorkgroups && L <= kMaxLength;
}

// State slots of cross_fused for state size n (0: not taken there).
int cross_fused_ns(int64_t n) { return n == 1 ? 1 : n == 2 ? 2 : n <= 4 ? 4 : 0; }

// The one-pass cross scan (cross_fused) takes n <= 4 and maps whose sum fits
// in LDS next to its staging areas, with positions below 2^16 (the exact
// 32-bit division by H and W) and a map slice whose byte offsets, the chunks
// loaded past its end included, stay below 2^31.
bool cross_one_pass_fits(int64_t L, int64_t d_in, int64_t n) {
    const int ns = cross_fused_ns(n);
    return ns > 0 && L < (int64_t(1) << 16) && ss::cross_lds_bytes(int(L), ns) <= kMaxLdsBytes &&
           (L + (ss::kCrossAhead + 2) * ss::kCrossChunk) * d_in * 4 < (int64_t(1) << 31);
}

// The form a call runs: SS_CROSS_AUTO is the two-pass form, the faster of the
// two on MI355X at every size measured (the one-pass form moves 2.3x fewer
// bytes at scan-vmamba but takes 1.24x as long: with 8 channels per
// workgroup, the most its LDS sum allows, it is bound by its memory requests
// and the per-chunk synchronisation, not by bandwidth).  0: not runnable.
int cross_form(int form, int64_t L, int64_t d_in, int64_t n) {
    if (form == SS_CROSS_AUTO || form == SS_CROSS_TWO_PASS) return SS_CROSS_TWO_PASS;
    if (form == SS_CROSS_ONE_PASS) return cross_one_pass_fits(L, d_in, n) ? SS_CROSS_ONE_PASS : 0;
    return 0;
}

SS_EXPORT size_t ss_cross_scan_fwd_ex_workspace_bytes(int64_t maps, int64_t H, int64_t W, int64_t d_in, int64_t n,
                                                      int dtype, int form) {
    if (dtype != SS_F32 && dtype != SS_BF16) return 0;
    if (!cross_sizes_ok(maps, H, W, d_in, n) || n > SS_MAX_STATE) return 0;
    const int f = cross_form(form, H * W, d_in, n);
    if (f == 0) return 0;
    if (f == SS_CROSS_ONE_PASS) return 256;   // the call's status words only
    return ss_scan_fwd_workspace_bytes(4 * maps, H * W, d_in, n, dtype) + cross_ys_bytes(maps, H * W, d_in);
}

SS_EXPORT size_t ss_cross_scan_fwd_workspace_bytes(int64_t maps, int64_t H, int64_t W, int64_t d_in, int64_t n,
                                                   int dtype) {
    return ss_cross_scan_fwd_ex_workspace_bytes(maps, H, W, d_in, n, dtype, SS_CROSS_AUTO);
}

template <typename TIn>
void launch_cross_fused(const ss::CrossParams& p, int ns, hipStream_t st) {
    const dim3 grid(unsigned(int64_t(p.maps) * p.ncb));
    const size_t lds = ss::cross_lds_bytes(p.L, ns);
    using Kern = void (*)(ss::CrossParams);
    static constexpr Kern kernels[2][3] = {
        {ss::cross_fused<TIn, 1, false>, ss::cross_fused<TIn, 2, false>, ss::cross_fused<TIn, 4, false>},
        {ss::cross_fused<TIn, 1, true>, ss::cross_fused<TIn, 2, true>, ss::cross_fused<TIn, 4, true>}};
    const Kern kern = kernels[p.softplus ? 1 : 0][ns == 1 ? 0 : ns == 2 ? 1 : 2];
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, p);
}

SS_EXPORT int ss_cross_scan_fwd_ex(const void* x, const void* delta, const float* A_log, const void* B,
                                   const void* C, const float* D, const float* delta_bias, int delta_softplus,
                                   float* y, float* last_state, int64_t maps, int64_t H, int64_t W, int64_t d_in,
                                   int64_t n, int dtype, int form, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    if (!x || !delta || !A_log || !B || !C || !D || !y) return SS_ERR_NULL;
    if (!cross_sizes_ok(maps, H, W, d_in, n)) return SS_ERR_SHAPE;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_DTYPE;
    if (form != SS_CROSS_AUTO && form != SS_CROSS_ONE_PASS && form != SS_CROSS_TWO_PASS) return SS_ERR_MODE;
    if (n > SS_MAX_STATE || cross_form(form, H * W, d_in, n) == 0) return SS_ERR_UNSUPPORTED;
    const int64_t b = 4 * maps, L = H * W;
    const size_t es = elem_size(dtype);
    for (const void* p : {x, delta, B, C})
        if (!aligned(p, es)) return SS_ERR_ALIGN;
    for (const void* p : {static_cast<const void*>(A_log), static_cast<const void*>(D),
                          static_cast<const void*>(delta_bias), static_cast<const void*>(y),
                          static_cast<const void*>(last_state)})
        if (p && !aligned(p, 4)) return SS_ERR_ALIGN;
    if (!aligned(workspace, 256)) return workspace ? SS_ERR_ALIGN : SS_ERR_WORKSPACE;
    const Range ins[] = {range_of(x, maps * L * d_in, es), range_of(delta, b * L * d_in, es),
                         range_of(A_log, 4 * d_in * n, 4), range_of(B, b * L * n, es), range_of(C, b * L * n, es),
                         range_of(D, 4 * d_in, 4), range_of(delta_bias, delta_bias ? 4 * d_in : 0, 4)};
    const Range ry = range_of(y, maps * L * d_in, 4);
    const Range rs = range_of(last_state, last_state ? b * d_in * n : 0, 4);
    for (const Range& r : ins)
        if (overlaps(r, ry) || overlaps(r, rs)) return SS_ERR_ALIAS;
    if (overlaps(ry, rs)) return SS_ERR_ALIAS;
    const size_t need = ss_cross_scan_fwd_ex_workspace_bytes(maps, H, W, d_in, n, dtype, form);
    if (!workspace || workspace_bytes < need) return SS_ERR_WORKSPACE;
    const Range rw = range_of(workspace, int64_t(workspace_bytes), 1);
    for (const Range& r : ins)
        if (overlaps(r, rw)) return SS_ERR_ALIAS;
    if (overlaps(ry, rw) || overlaps(rs, rw)) return SS_ERR_ALIAS;

    hipStream_t st = static_cast<hipStream_t>(stream);
    if (cross_form(form, L, d_in, n) == SS_CROSS_ONE_PASS) {
        ss::CrossParams c{};
        c.x = x;
        c.delta = delta;
        c.A_log = A_log;
        c.B = B;
        c.C = C;
        c.D = D;
        c.bias = delta_bias;
        c.y = y;
        c.last_state = last_state;
        c.err = static_cast<uint32_t*>(workspace) + kStatusWord;
        c.maps = int(maps);
        c.H = int(H);
        c.W = int(W);
        c.L = int(L);
        c.d_in = int(d_in);
        c.n = int(n);
        c.softplus = delta_softplus ? 1 : 0;
        c.ncb = int((d_in + ss::kCrossCh - 1) / ss::kCrossCh);
        c.vec_y = d_in % 4 == 0 && aligned(y, 16);
        c.magic_h = H > 1 ? uint32_t(((uint64_t(1) << 32) + uint64_t(H) - 1) / uint64_t(H)) : 0u;
        c.magic_w = W > 1 ? uint32_t(((uint64_t(1) << 32) + uint64_t(W) - 1) / uint64_t(W)) : 0u;
        if (dtype == SS_BF16)
            launch_cross_fused<uint16_t>(c, cross_fused_ns(n), st);
        else
            launch_cross_fused<float>(c, cross_fused_ns(n), st);
        return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
    }

    // Two passes: the scan's own workspace first (so the status words lead
    // the workspace), then the four directions' outputs.
    const size_t scan_ws_bytes = ss_scan_fwd_workspace_bytes(b, L, d_in, n, dtype);
    float* ys = reinterpret_cast<float*>(static_cast<char*>(workspace) + scan_ws_bytes);
    ScanParams p{};
    p.u = x;
    p.delta = delta;
    p.A_log = A_log;
    p.B = B;
    p.C = C;
    p.D = D;
    p.z = nullptr;
    p.bias = delta_bias;
    p.y = ys;
    p.last_state = last_state;
    p.b = b;
    p.L = L;
    p.d_in = d_in;
    p.n = n;
    p.softplus = delta_softplus ? 1 : 0;
    p.cross_h = int(H);
    p.cross_w = int(W);
    p.nblk_d = int((d_in + 63) / 64);
    p.K = 1;
    p.Lseg = L;
    p.err = static_cast<uint32_t*>(workspace) + kStatusWord;
    const int rc = dtype == SS_BF16 ? dispatch_seq<uint16_t>(p, SeqMode::Cross, workspace, scan_ws_bytes, st)
                                    : dispatch_seq<float>(p, SeqMode::Cross, workspace, scan_ws_bytes, st);
    if (rc != SS_OK) return rc;
    // CrossMerge: the four directions' outputs added back at their positions.
    const bool vec = d_in % 4 == 0 && aligned(y, 16);
    const int64_t threads = maps * L * (vec ? d_in / 4 : d_in);
    const dim3 grid = grid_1d(threads);
    if (vec)
        hipLaunchKernelGGL((ss::cross_merge<4>), grid, dim3(256), 0, st, ys, y, maps, int(H), int(W), d_in);
    else
        hipLaunchKernelGGL((ss::cross_merge<1>), grid, dim3(256), 0, st, ys, y, maps, int(H), int(W), d_in);
    return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
}

SS_EXPORT int ss_cross_scan_fwd(const void* x, const void* delta, const float* A_log, const void* B, const void* C,
                                const float* D, const float* delta_bias, int delta_softplus, float* y,
                                float* last_state, int64_t maps, int64_t H, int64_t W, int64_t d_in, int64_t n,
                                int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return ss_cross_scan_fwd_ex(x, delta, A_log, B, C, D, delta_bias, delta_softplus, y, last_state, maps, H, W,
                                d_in, n, dtype, SS_CROSS_AUTO, workspace, workspace_bytes, stream);
}

// ============================================================================= backward

namespace {

using namespace ss_host;
using ss::BwdParams;

// Workspace of ss_scan_bwd, in order: the forward scan's own workspace (whose
// control words lead with the call's status words), the forward's
// checkpoints, the dB and dC partials per channel group, the dA_log, dD and
// dbias partials per segment and batch row, then the control words and
// adjoints of the backward's segments.
struct BwdWorkspace {
    size_t fwd, ckpt, part_B, part_C, part_A, part_D, part_bias, part_du, part_dd, ctl, handoff, total;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// saved: the backward from states the forward saved (no forward pass, no
// checkpoints of its own; the first 256 bytes hold the status words).
BwdWorkspace bwd_workspace(int64_t b, int64_t L, int64_t d_in, int64_t n, bool saved = false) {
    const int64_t nck = (L - 1) / ss::kCkptSteps;
    const int64_t nblk = (d_in + 63) / 64;
    BwdWorkspace w;
    w.ckpt = saved ? 0 : round256(size_t(b) * size_t(nck) * size_t(n) * size_t(d_in) * 4);
    w.part_B = w.part_C = round256(size_t(nblk) * size_t(b) * size_t(L) * size_t(n) * 4);
    w.part_A = round256(size_t(kMaxSegments) * size_t(b) * size_t(d_in) * size_t(n) * 4);
    const int64_t slices = bwd_slices(n);
    w.part_D = round256(size_t(kMaxSegments) * size_t(b) * size_t(d_in) * 4);
    w.part_bias = round256(size_t(kMaxSegments) * size_t(slices) * size_t(b) * size_t(d_in) * 4);
    // du and ddelta in parts, one per slice of the states, when there are several.
    w.part_du = w.part_dd = slices > 1 ? round256(size_t(slices) * size_t(b) * size_t(L) * size_t(d_in) * 4) : 0;
    const int64_t G = b * nblk * slices;
    const SeqShape sh = bwd_shape(n);
    w.ctl = round256((size_t(ss::kFlagOffset) + size_t(G) * kMaxSegments) * sizeof(uint32_t));
    w.handoff = round256(size_t(kMaxSegments - 1) * size_t(G) * size_t(sh.SC * sh.NSW) * 64 * sizeof(float));
    w.fwd = saved ? 256 : seq_workspace(b, d_in, n).total;
    w.total = w.fwd + w.ckpt + w.part_B + w.part_C + w.part_A + w.part_D + w.part_bias + w.part_du + w.part_dd +
              w.ctl + w.handoff;
    return w;
}

template <typename TIn>
int dispatch_bwd(const BwdParams& p, bool gate, bool zoh, hipStream_t st, int* segments) {
    const SeqShape sh = bwd_shape(p.n);
    if (p.slices > 1) return launch_bwd<TIn, 8, 2, true>(p, gate, zoh, st, segments);
    if (sh.SC == 1) return launch_bwd<TIn, 1, 2, false>(p, gate, zoh, st, segments);
    if (sh.SC == 4) return launch_bwd<TIn, 4, 2, false>(p, gate, zoh, st, segments);
    return launch_bwd<TIn, 8, 2, false>(p, gate, zoh, st, segments);
}

template <typename TOut>
int reduce(const float* part, void* out, int64_t count, int64_t groups, hipStream_t st) {
    hipLaunchKernelGGL((ss::reduce_groups<TOut>), grid_1d(count), dim3(256), 0, st, part,
                       static_cast<TOut*>(out), count, int(groups));
    return hipGetLastError() == hipSuccess ? SS_OK : SS_ERR_HIP;
}

}  // namespace

namespace {

bool bwd_sizes_ok(int64_t b, int64_t L, int64_t d_in, int64_t n) {
    return sizes_ok(b, L, d_in) && n > 0 && n <= SS_MAX_BWD_STATE && d_in <= SS_MAX_CHANNELS &&
           b * ((d_in + 63) / 64) * bwd_slices(n) <= kMaxWorkgroups && L <= kMaxLength;
}

}  // namespace

SS_EXPORT size_t ss_scan_bwd_workspace_bytes(int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype) {
    if (dtype != SS_F32 && dtype != SS_BF16) return 0;
    return bwd_sizes_ok(b, L, d_in, n) ? bwd_workspace(b, L, d_in, n).total : 0;
}

SS_EXPORT size_t ss_scan_bwd_saved_workspace_bytes(int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype) {
    if (dtype != SS_F32 && dtype != SS_BF16) return 0;
    return bwd_sizes_ok(b, L, d_in, n) ? bwd_workspace(b, L, d_in, n, true).total : 0;
}

SS_EXPORT size_t ss_scan_checkpoint_bytes(int64_t b, int64_t L, int64_t d_in, int64_t n) {
    if (!bwd_sizes_ok(b, L, d_in, n)) return 0;
    return size_t(b) * size_t((L - 1) / ss::kCkptSteps) * size_t(n) * size_t(d_in) * 4;
}

namespace {

// The backward pass.  Without saved states (ckpt_in null) it first runs the
// forward scan again to save the state every kCkptSteps steps (and, gated,
// to write dz); with them it starts from the checkpoints and the pre-gate
// readout y_pre that ss_scan_fwd_save wrote, and forms dz itself.
int scan_bwd_impl(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                  const float* D, const void* z, const float* delta_bias, int delta_softplus,
                  const float* initial_state, int discretization, const float* ckpt_in, const void* y_pre,
                  const void* dy, const float* dlast_state, void* du, void* ddelta, float* dA_log, void* dB,
                  void* dC, float* dD, void* dz, float* ddelta_bias, float* dinitial_state, int64_t b, int64_t L,
                  int64_t d_in, int64_t n, int dtype, void* workspace, size_t workspace_bytes, bool saved,
                  void* stream) {
    if (!u || !delta || !A_log || !B || !C || !D || !dy || !du || !ddelta || !dA_log || !dB || !dC || !dD)
        return SS_ERR_NULL;
    if (z && !dz) return SS_ERR_NULL;
    if (saved && ((!ckpt_in && L > ss::kCkptSteps) || (z && !y_pre))) return SS_ERR_NULL;
    if (discretization != SS_DISC_EULER && discretization != SS_DISC_ZOH) return SS_ERR_MODE;
    const bool zoh = discretization == SS_DISC_ZOH;
    if (!sizes_ok(b, L, d_in) || n <= 0 || d_in > SS_MAX_CHANNELS) return SS_ERR_SHAPE;
    if (dtype != SS_F32 && dtype != SS_BF16) return SS_ERR_DTYPE;
    if (n > SS_MAX_BWD_STATE) return SS_ERR_UNSUPPORTED;
    if (b * ((d_in + 63) / 64) * bwd_slices(n) > kMaxWorkgroups || L > kMaxLength) return SS_ERR_SHAPE;
    if (!saved) y_pre = nullptr;
    const size_t es = elem_size(dtype);
    for (const void* p : {u, delta, B, C, z, dy, y_pre, static_cast<const void*>(du),
                          static_cast<const void*>(ddelta), static_cast<const void*>(dB), static_cast<const void*>(dC),
                          static_cast<const void*>(dz)})
        if (p && !aligned(p, es)) return SS_ERR_ALIGN;
    for (const void* p : {static_cast<const void*>(A_log), static_cast<const void*>(D),
                          static_cast<const void*>(delta_bias), static_cast<const void*>(initial_state),
                          static_cast<const void*>(dlast_state), static_cast<const void*>(dA_log),
                          static_cast<const void*>(dD), static_cast<const void*>(ddelta_bias),
                          static_cast<const void*>(dinitial_state), static_cast<const void*>(ckpt_in)})
        if (p && !aligned(p, 4)) return SS_ERR_ALIGN;
    if (!aligned(workspace, 256)) return workspace ? SS_ERR_ALIGN : SS_ERR_WORKSPACE;
    const int64_t nel = b * L * d_in, nst = b * d_in * n;
    const Range ins[] = {range_of(u, nel, es), range_of(delta, nel, es), range_of(A_log, d_in * n, 4),
                         range_of(B, b * L * n, es), range_of(C, b * L * n, es), range_of(D, d_in, 4),
                         range_of(z, z ? nel : 0, es), range_of(delta_bias, delta_bias ? d_in : 0, 4),
                         range_of(initial_state, initial_state ? nst : 0, 4), range_of(dy, nel, es),
                         range_of(dlast_state, dlast_state ? nst : 0, 4),
                         range_of(ckpt_in, saved ? int64_t(ss_scan_checkpoint_bytes(b, L, d_in, n)) : 0, 1),
                         range_of(y_pre, y_pre ? nel : 0, es)};
    const Range outs[] = {range_of(du, nel, es), range_of(ddelta, nel, es), range_of(dA_log, d_in * n, 4),
                          range_of(dB, b * L * n, es), range_of(dC, b * L * n, es), range_of(dD, d_in, 4),
                          range_of(dz, z ? nel : 0, es), range_of(ddelta_bias, ddelta_bias ? d_in : 0, 4),
                          range_of(dinitial_state, dinitial_state ? nst : 0, 4)};
    const size_t need = saved ? ss_scan_bwd_saved_workspace_bytes(b, L, d_in, n, dtype)
                              : ss_scan_bwd_workspace_bytes(b, L, d_in, n, dtype);
    if (!workspace || workspace_bytes < need) return SS_ERR_WORKSPACE;
    const Range rw = range_of(workspace, int64_t(workspace_bytes), 1);
    for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); i++) {
        for (const Range& r : ins)
            if (overlaps(r, outs[i])) return SS_ERR_ALIAS;
        for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); j++)
            if (overlaps(outs[i], outs[j])) return SS_ERR_ALIAS;
        if (overlaps(outs[i], rw)) return SS_ERR_ALIAS;
    }
    for (const Range& r : ins)
        if (overlaps(r, rw)) return SS_ERR_ALIAS;

    const BwdWorkspace w = bwd_workspace(b, L, d_in, n, saved);
    char* const base = static_cast<char*>(workspace);
    void* fwd_ws = base;
    char* at = base + w.fwd;
    float* ckpt = saved ? const_cast<float*>(ckpt_in) : reinterpret_cast<float*>(at);
    float* part_B = reinterpret_cast<float*>(at += w.ckpt);
    float* part_C = reinterpret_cast<float*>(at += w.part_B);
    float* part_A = reinterpret_cast<float*>(at += w.part_C);
    float* part_D = reinterpret_cast<float*>(at += w.part_A);
    float* part_bias = reinterpret_cast<float*>(at += w.part_D);
    float* part_du = reinterpret_cast<float*>(at += w.part_bias);
    float* part_dd = reinterpret_cast<float*>(at += w.part_du);
    uint32_t* bctl = reinterpret_cast<uint32_t*>(at += w.part_dd);
    float* handoff = reinterpret_cast<float*>(at += w.ctl);
    uint32_t* err = static_cast<uint32_t*>(workspace) + kStatusWord;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int nblk = int((d_in + 63) / 64);

    // 1. The forward scan again, saving the state every kCkptSteps steps.  No
    //    y; with a gate it writes dz, the one gradient that needs the readout
    //    sum C h + D u (so the backward pass never recomputes the readout).
    //    From saved states only the status words are cleared.
    const int nck = int((L - 1) / ss::kCkptSteps);
    int rc = SS_OK;
    if (saved) {
        hipLaunchKernelGGL(ss::scan_ctl_reset, dim3(1), dim3(64), 0, st, err, int64_t(0), err);
        if (hipGetLastError() != hipSuccess) return SS_ERR_HIP;
    } else {
        ScanParams f{};
        f.u = u;
        f.delta = delta;
        f.A_log = A_log;
        f.B = B;
        f.C = C;
        f.D = D;
        f.z = z;
        f.bias = delta_bias;
        f.y = nullptr;
        f.last_state = nullptr;
        f.h0 = initial_state;
        f.ckpt = ckpt;
        f.dy = z ? dy : nullptr;
        f.dz = z ? dz : nullptr;
        f.nck = nck;
        f.b = b;
        f.L = L;
        f.d_in = d_in;
        f.n = n;
        f.softplus = delta_softplus ? 1 : 0;
        f.nblk_d = nblk;
        f.K = 1;
        f.Lseg = L;
        f.err = err;
        const SeqMode fm = zoh ? (z ? SeqMode::ZohDz : SeqMode::Zoh) : (z ? SeqMode::Dz : SeqMode::Euler);
        rc = dtype == SS_BF16 ? dispatch_seq<uint16_t>(f, fm, fwd_ws, w.fwd, st)
                              : dispatch_seq<float>(f, fm, fwd_ws, w.fwd, st);
        if (rc != SS_OK) return rc;
    }

    // 2. Backward through every chunk.
    BwdParams p{};
    p.u = u;
    p.delta = delta;
    p.A_log = A_log;
    p.B = B;
    p.C = C;
    p.D = D;
    p.z = z;
    p.bias = delta_bias;
    p.h0 = initial_state;
    p.dy = dy;
    p.ypre = z ? y_pre : nullptr;
    p.dz = p.ypre ? dz : nullptr;
    p.dlast = dlast_state;
    p.ckpt = ckpt;
    p.du = du;
    p.ddelta = ddelta;
    p.dh0 = dinitial_state;
    p.part_B = part_B;
    p.part_C = part_C;
    p.part_A = part_A;
    p.part_D = part_D;
    p.part_bias = part_bias;
    p.slices = int(bwd_slices(n));
    p.part_du = p.slices > 1 ? part_du : nullptr;
    p.part_dd = p.slices > 1 ? part_dd : nullptr;
    p.b = b;
    p.L = L;
    p.d_in = d_in;
    p.n = n;
    p.nck = nck;
    p.nblk_d = nblk;
    p.softplus = delta_softplus ? 1 : 0;
    p.ctl = bctl;
    p.handoff = handoff;
    p.err = err;
    int K = 1;
    rc = dtype == SS_BF16 ? dispatch_bwd<uint16_t>(p, z != nullptr, zoh, st, &K)
                          : dispatch_bwd<float>(p, z != nullptr, zoh, st, &K);
    if (rc != SS_OK) return rc;

    // 3. Sums over state slices (du, ddelta), channel groups (dB, dC) and
    //    segments, slices and batch rows (dA_log, dD, dbias), in a fixed order.
    const int64_t nbc = b * L * n;
    if (p.slices > 1) {
        rc = dtype == SS_BF16 ? reduce<uint16_t>(part_du, du, nel, p.slices, st)
                              : reduce<float>(part_du, du, nel, p.slices, st);
        if (rc == SS_OK)
            rc = dtype == SS_BF16 ? reduce<uint16_t>(part_dd, ddelta, nel, p.slices, st)
                                  : reduce<float>(part_dd, ddelta, nel, p.slices, st);
        if (rc != SS_OK) return rc;
    }
    rc = dtype == SS_BF16 ? reduce<uint16_t>(part_B, dB, nbc, nblk, st) : reduce<float>(part_B, dB, nbc, nblk, st);
    if (rc == SS_OK)
        rc = dtype == SS_BF16 ? reduce<uint16_t>(part_C, dC, nbc, nblk, st) : reduce<float>(part_C, dC, nbc, nblk, st);
    if (rc == SS_OK) rc = reduce<float>(part_A, dA_log, d_in * n, int64_t(K) * b, st);
    if (rc == SS_OK) rc = reduce<float>(part_D, dD, d_in, int64_t(K) * b, st);
    if (rc == SS_OK && ddelta_bias && delta_bias)
        rc = reduce<float>(part_bias, ddelta_bias, d_in, int64_t(K) * p.slices * b, st);
    return rc;
}

}  // namespace

SS_EXPORT int ss_scan_bwd_ex(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                             const float* D, const void* z, const float* delta_bias, int delta_softplus,
                             const float* initial_state, int discretization, const void* dy,
                             const float* dlast_state, void* du, void* ddelta, float* dA_log, void* dB, void* dC,
                             float* dD, void* dz, float* ddelta_bias, float* dinitial_state, int64_t b, int64_t L,
                             int64_t d_in, int64_t n, int dtype, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return scan_bwd_impl(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, initial_state, discretization,
                         nullptr, nullptr, dy, dlast_state, du, ddelta, dA_log, dB, dC, dD, dz, ddelta_bias,
                         dinitial_state, b, L, d_in, n, dtype, workspace, workspace_bytes, false, stream);
}

SS_EXPORT int ss_scan_bwd_saved(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                                const float* D, const void* z, const float* delta_bias, int delta_softplus,
                                const float* initial_state, int discretization, const float* checkpoints,
                                const void* y_pre, const void* dy, const float* dlast_state, void* du, void* ddelta,
                                float* dA_log, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                                float* dinitial_state, int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return scan_bwd_impl(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, initial_state, discretization,
                         checkpoints, y_pre, dy, dlast_state, du, ddelta, dA_log, dB, dC, dD, dz, ddelta_bias,
                         dinitial_state, b, L, d_in, n, dtype, workspace, workspace_bytes, true, stream);
}

SS_EXPORT int ss_scan_bwd(const void* u, const void* delta, const float* A_log, const void* B, const void* C,
                          const float* D, const void* z, const float* delta_bias, int delta_softplus,
                          const float* initial_state, const void* dy, const float* dlast_state, void* du,
                          void* ddelta, float* dA_log, void* dB, void* dC, float* dD, void* dz, float* ddelta_bias,
                          float* dinitial_state, int64_t b, int64_t L, int64_t d_in, int64_t n, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return ss_scan_bwd_ex(u, delta, A_log, B, C, D, z, delta_bias, delta_softplus, initial_state, SS_DISC_EULER, dy,
                          dlast_state, du, ddelta, dA_log, dB, dC, dD, dz, ddelta_bias, dinitial_state, b, L, d_in, n,
                          dtype, workspace, workspace_bytes, stream);
}
