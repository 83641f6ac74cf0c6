// ss_device.h -- device helpers shared by the selective-scan kernels (gfx950).
//
// Element access for the two input types (fp32 and bf16 kept as raw 16-bit
// words), the hardware transcendental instructions, and the two pointwise
// functions of the method: softplus for the step size (mhpn.cn selective_scan
// walk-through, section 7; jiafeimiao.top Mamba.step: softplus(dt + dt_bias))
// and silu for the output gate (Mamba.step: y * act(z)).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v_exp_f32 / v_log_f32 / v_rcp_f32: base-2 exponential and logarithm and the
// reciprocal, each about 1 ulp.  On gfx950 they issue at half the fp32 FMA rate.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// bf16 <-> fp32.  Widening is exact (the bf16 word is the high half of the
// fp32 word).  Narrowing rounds to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}
// Two values narrowed at once (one v_cvt_pk_bf16_f32): lo in bits 0-15.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// fences global memory, which makes every wave wait for all its outstanding
// global loads at the barrier; a software pipeline that keeps loads in flight
// across barriers needs this narrower form.  Global memory shared between
// waves must be ordered with explicit fences instead.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// An LDS-space pointer (the direct-to-LDS loads take their destination so).
using lds_ptr = __attribute__((address_space(3))) char*;

// LDS-space pointer to the start of a kernel's dynamic LDS (extern __shared__
// __align__(16)), which begins at the end of the static allocation rounded up
// to that alignment; the kernels here declare no static LDS, so it is 0.
// Formed from the LDS address itself: converting a generic pointer to LDS
// space adds a null check of it (which the compiler has also been seen to
// emit as an invalid instruction).
__device__ __forceinline__ lds_ptr dynamic_lds_base() {
    return (lds_ptr)(uintptr_t)((__builtin_amdgcn_groupstaticsize() + 15u) & ~15u);
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, unrolled at compile time.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// `v` unchanged, but opaque to the optimiser: a constant passed through here
// is formed where it is used (one scalar instruction) instead of being
// hoisted into a register of its own for a whole loop.
__device__ __forceinline__ uint32_t opaque_scalar(uint32_t v) {
    asm volatile("" : "+s"(v));
    return v;
}

// Direct-to-LDS load: every lane reads BYTES bytes at `src` and the wave's data
// lands in LDS at `lds_dst` + lane * max(BYTES, 4), without passing through
// registers.  Completion is tracked by the vector-memory counter.
template <int BYTES>
__device__ __forceinline__ void load_to_lds(const void* src, lds_ptr lds_dst) {
    static_assert(BYTES == 2 || BYTES == 4 || BYTES == 16, "direct-to-LDS load size");
    auto* dst = (__attribute__((address_space(3))) void*)lds_dst;
    if constexpr (BYTES == 16) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    else if constexpr (BYTES == 4) __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
    else __builtin_amdgcn_global_load_lds(src, dst, 2, 0, 0);
}

// The same through a buffer descriptor: every lane reads BYTES bytes at byte
// offset voff + soff of the descriptor's base.  `soff` is wave-uniform (a
// scalar register), so a stream of such loads whose per-lane offsets are
// fixed costs no vector instruction.  Lanes whose voff is at or beyond the
// descriptor's byte count read zeros instead of memory.
template <int BYTES>
__device__ __forceinline__ void buffer_load_to_lds(__amdgpu_buffer_rsrc_t rsrc, lds_ptr lds_dst, uint32_t voff,
                                                   uint32_t soff) {
    static_assert(BYTES == 2 || BYTES == 4 || BYTES == 16, "direct-to-LDS load size");
    auto* dst = (__attribute__((address_space(3))) void*)lds_dst;
    if constexpr (BYTES == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, voff, soff, 0, 0);
    else if constexpr (BYTES == 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 4, voff, soff, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 2, voff, soff, 0, 0);
}

// Buffer descriptor of `bytes` bytes at `base` (wave-uniform): untyped, no
// stride, the data-format word that raw buffer accesses take on gfx9 parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
struct VmemWait {
    static constexpr int n = N > 63 ? 63 : N;
    enum : int { code = (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8) };
};
template <int N>
__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt(VmemWait<N>::code);
}

// Integer min/max with both operands of one type.  HIP's own min/max also
// accept mixed argument types, and those overloads compute in double.
__device__ __forceinline__ int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }

template <typename T> struct Elem;

template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};

template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Raw input element as loaded (bf16 kept as its 16-bit word until used).
template <typename T> struct Raw;
template <> struct Raw<uint16_t> {
    using type = uint32_t;
    static __device__ __forceinline__ type load(const uint16_t* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ float f(type v) { return __uint_as_float(v << 16); }
};
template <> struct Raw<float> {
    using type = float;
    static __device__ __forceinline__ type load(const float* p, int64_t i) { return p[i]; }
    static __device__ __forceinline__ float f(type v) { return v; }
};

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e) with e = exp(-|x|) in (0, 1].
// log1p(e) is log2(u) * ln 2 for u = 1 + e rounded to fp32, corrected by the
// rounding error of u: log(1 + e) = log(u) - log(u / (1 + e)) and
// log(u / (1 + e)) = ((u - 1) - e) / u to first order, where (u - 1) - e is
// exact (Sterbenz) and dropping the division by u in [1, 2] changes the
// result by less than 2^-24 relative.  This keeps small step sizes
// (x << 0, e.g. softplus(-12) ~ 6e-6) accurate to a few ulp, which a plain
// log(1 + exp(x)) would not; it costs one exp2 and one log2.
__device__ __forceinline__ float softplus(float x) {
    const float e = exp2_hw(-fabsf(x) * kLog2e);
    const float uu = 1.0f + e;
    const float c = (uu - 1.0f) - e;
    return fmaxf(x, 0.0f) + fmaf(log2_hw(uu), kLn2, -c);
}

// silu(z) = z / (1 + e^-z); for z -> -inf the reciprocal of +inf is 0.
__device__ __forceinline__ float silu(float z) {
    return z * rcp_hw(1.0f + exp2_hw(-z * kLog2e));
}

// Step size of one (b, t, d) element: delta plus the optional bias, then the
// optional softplus.
__device__ __forceinline__ float step_size(float delta, float bias, int use_softplus) {
    const float v = delta + bias;
    return use_softplus ? softplus(v) : v;
}

// A2 = A * log2(e) with A = -exp(A_log), so that exp(delta * A) = exp2(delta * A2).
__device__ __forceinline__ float a2_from_alog(float a_log) {
    return -exp2_hw(a_log * kLog2e) * kLog2e;
}

// 1 / A = -exp(-A_log).
__device__ __forceinline__ float inv_a_from_alog(float a_log) {
    return -exp2_hw(-a_log * kLog2e);
}

// Zero-order-hold input weight (exp(delta' A) - 1) / A of one state (mhpn.cn
// selective_scan walk-through, section 6: the exact discretisation of the B
// term, which for a diagonal A acts state by state), given x2 = delta' A2,
// a = exp2(x2) and invA = 1 / A.
//   |x2| >= 1/2: |a - 1| > 0.29, so (a - 1) / A loses less than 2^-22 to the
//     cancellation and is used as it stands.
//   |x2| <  1/2: the weight is delta' E(x) with E(x) = expm1(x) / x and
//     x = x2 ln 2, |x| < 0.35, from its Taylor series sum_k x^k / (k+1)! cut
//     after x^6 (the first dropped term is below 1.6e-8 relative), written in
//     powers of x2 and evaluated by Horner's rule; in fp32 the result is
//     within 8e-8 relative of E.
__device__ __forceinline__ float zoh_weight(float dl, float x2, float a, float invA) {
    constexpr double l = 0.6931471805599453;   // ln 2; c_k = ln2^k / (k+1)!
    constexpr float c6 = float(l * l * l * l * l * l / 5040.0), c5 = float(l * l * l * l * l / 720.0),
                    c4 = float(l * l * l * l / 120.0), c3 = float(l * l * l / 24.0), c2 = float(l * l / 6.0),
                    c1 = float(l / 2.0);
    float e = fmaf(c6, x2, c5);
    e = fmaf(e, x2, c4);
    e = fmaf(e, x2, c3);
    e = fmaf(e, x2, c2);
    e = fmaf(e, x2, c1);
    e = fmaf(e, x2, 1.0f);
    return fabsf(x2) < 0.5f ? dl * e : (a - 1.0f) * invA;
}

}  // namespace ss
