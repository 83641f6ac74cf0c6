// state_update_kernels.h -- the single-token decode step on a persistent state
// (jiafeimiao.top, Mamba.step and its selective_state_update call):
//     delta' = softplus(dt + dt_bias)
//     state[k] = exp(delta' A[d,k]) state[k] + delta' B[b,k] x      (in place)
//     y = sum_k C[b,k] state[k] + D[d] x,   then y *= silu(z) if z is given.
// With the zero-order hold (mhpn.cn selective_scan walk-through, section 6)
// the input term is (exp(delta' A[d,k]) - 1) / A[d,k] * B[b,k] x instead.
// The step reads and writes the whole fp32 state once, so it is bound by HBM
// bandwidth; everything else is small.
//
// state_update_vec: n a multiple of 4 with n/4 in {1, 2, 4, 8, 16}.  LPC = n/4
//   consecutive lanes share one (b, d) channel; each lane moves 4 states with
//   one 16-byte load and one 16-byte store, so a wave reads and writes
//   contiguous 1 KiB spans of the state.  The partial readouts are summed
//   across the LPC lanes with butterfly shuffles; the first lane of the group
//   finishes y.
// state_update_any: any n.  One thread per channel, states walked in a loop.
#pragma once

#include "ss_device.h"

namespace ss {

struct StepParams {
    float* state;
    const void* x;
    const void* dt;
    const float* A_log;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* bias;
    void* y;
    int64_t b, d_in, n;
    int softplus;
    int zoh;             // zero-order-hold input weight instead of delta'
};

// New value of one state: exp(delta' A) s + w B x, where w is delta' or the
// zero-order-hold weight (exp(delta' A) - 1) / A.
__device__ __forceinline__ float step_state(float s, float dl, float xv, float a_log, float Bk, int zoh) {
    const float x2 = dl * a2_from_alog(a_log);
    const float a = exp2_hw(x2);
    const float w = zoh ? zoh_weight(dl, x2, a, inv_a_from_alog(a_log)) : dl;
    return fmaf(a, s, (w * xv) * Bk);
}

template <typename TIn>
__device__ __forceinline__ float4 load4(const TIn* p, int64_t i);

template <>
__device__ __forceinline__ float4 load4<float>(const float* p, int64_t i) {
    return *reinterpret_cast<const float4*>(p + i);
}

template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t* p, int64_t i) {
    const uint2 v = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
}

template <typename TIn, int LPC>
__global__ __launch_bounds__(256) void state_update_vec(const StepParams p) {
    const TIn* __restrict__ xp = static_cast<const TIn*>(p.x);
    const TIn* __restrict__ dtp = static_cast<const TIn*>(p.dt);
    const TIn* __restrict__ Bm = static_cast<const TIn*>(p.B);
    const TIn* __restrict__ Cm = static_cast<const TIn*>(p.C);
    const TIn* __restrict__ zp = static_cast<const TIn*>(p.z);
    TIn* __restrict__ yp = static_cast<TIn*>(p.y);

    const int64_t tid = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    const int64_t ch = tid / LPC;                 // (b, d) channel
    const int q = int(tid % LPC);                 // which group of 4 states
    const int64_t nch = p.b * p.d_in;
    // Whole LPC groups sit inside one wave and leave together, so the
    // shuffles below only ever read lanes of live groups.
    if (ch >= nch) return;
    const int64_t bi = ch / p.d_in;
    const int64_t d = ch - bi * p.d_in;
    const int64_t n = p.n;

    // The state is read once and written once per step: non-temporal
    // accesses (the state is the bulk of the traffic and no other access of
    // this step reuses it), issued first, as the longest wait.
    typedef float f4v __attribute__((ext_vector_type(4)));
    f4v* sp = reinterpret_cast<f4v*>(p.state) + ch * LPC + q;
    f4v s = __builtin_nontemporal_load(sp);
    const float xv = Elem<TIn>::load(xp, ch);
    const float dl = step_size(Elem<TIn>::load(dtp, ch), p.bias ? p.bias[d] : 0.0f, p.softplus);
    const float4 al = reinterpret_cast<const float4*>(p.A_log)[d * LPC + q];
    const float4 Bv = load4<TIn>(Bm, bi * n + 4 * q);
    const float4 Cv = load4<TIn>(Cm, bi * n + 4 * q);

    s.x = step_state(s.x, dl, xv, al.x, Bv.x, p.zoh);
    s.y = step_state(s.y, dl, xv, al.y, Bv.y, p.zoh);
    s.z = step_state(s.z, dl, xv, al.z, Bv.z, p.zoh);
    s.w = step_state(s.w, dl, xv, al.w, Bv.w, p.zoh);
    __builtin_nontemporal_store(s, sp);

    float acc = fmaf(Cv.x, s.x, fmaf(Cv.y, s.y, fmaf(Cv.z, s.z, Cv.w * s.w)));
#pragma unroll
    for (int m = 1; m < LPC; m <<= 1) acc += __shfl_xor(acc, m, LPC);
    if (q == 0) {
        acc = fmaf(p.D[d], xv, acc);
        if (zp) acc *= silu(Elem<TIn>::load(zp, ch));
        Elem<TIn>::store(yp, ch, acc);
    }
}

template <typename TIn>
__global__ __launch_bounds__(256) void state_update_any(const StepParams p) {
    const TIn* __restrict__ xp = static_cast<const TIn*>(p.x);
    const TIn* __restrict__ dtp = static_cast<const TIn*>(p.dt);
    const TIn* __restrict__ Bm = static_cast<const TIn*>(p.B);
    const TIn* __restrict__ Cm = static_cast<const TIn*>(p.C);
    const TIn* __restrict__ zp = static_cast<const TIn*>(p.z);
    TIn* __restrict__ yp = static_cast<TIn*>(p.y);

    const int64_t ch = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (ch >= p.b * p.d_in) return;
    const int64_t bi = ch / p.d_in;
    const int64_t d = ch - bi * p.d_in;
    const int64_t n = p.n;

    const float xv = Elem<TIn>::load(xp, ch);
    const float dl = step_size(Elem<TIn>::load(dtp, ch), p.bias ? p.bias[d] : 0.0f, p.softplus);
    float acc = 0.0f;
    for (int64_t k = 0; k < n; k++) {
        const float s = step_state(p.state[ch * n + k], dl, xv, p.A_log[d * n + k], Elem<TIn>::load(Bm, bi * n + k),
                                   p.zoh);
        p.state[ch * n + k] = s;
        acc = fmaf(Elem<TIn>::load(Cm, bi * n + k), s, acc);
    }
    acc = fmaf(p.D[d], xv, acc);
    if (zp) acc *= silu(Elem<TIn>::load(zp, ch));
    Elem<TIn>::store(yp, ch, acc);
}

}  // namespace ss
