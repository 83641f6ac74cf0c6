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
// state_update_vec: n a multiple of 4 with n/4 in {1, 2, 4, 8, 16}; see the
//   kernel.  state_update_any: any n.  One thread per channel, states walked
//   in a loop.
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

// Value of lane (group base + j) in every lane of a group of G lanes, G a
// power of two up to 16: a DPP quad permute for G <= 4, a lane shuffle above.
template <int G, int J>
__device__ __forceinline__ float group_bcast(float v) {
    if constexpr (G == 1) {
        return v;
    } else if constexpr (G <= 4) {
        // quad_perm: quad position p reads position (p & ~(G - 1)) + J.
        constexpr int ctrl = (((0 & ~(G - 1)) + J) << 0) | (((1 & ~(G - 1)) + J) << 2) |
                             (((2 & ~(G - 1)) + J) << 4) | (((3 & ~(G - 1)) + J) << 6);
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xf, 0xf, false));
    } else {
        return __shfl(v, J, G);
    }
}

// Value of lane (lane ^ M) in every lane, M in {1, 2, 4, 8}: DPP quad
// permutes for 1 and 2, a row rotation by 8 for 8 (within a row of 16 lanes
// that is the xor), a lane shuffle for 4.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    if constexpr (M == 1) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));
    } else if constexpr (M == 2) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));
    } else if constexpr (M == 8) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
    } else {
        return __shfl_xor(v, M, 16);
    }
}

// Sums over a group of G lanes for G rows at once: lane q of the group
// starts with v[r] for every row r and ends holding the group's total of row
// q.  Each step halves the rows a lane carries: of a pair of rows the lane
// keeps the one its lane bit selects, adds its partner's copy of that row,
// and hands the other row to the partner.  Every total is the same sum tree
// as a butterfly of xor shuffles over the group, so the result is bitwise
// the same.
template <int G, int M = 1>
__device__ __forceinline__ float group_transpose_sum(float (&v)[G], int q) {
    if constexpr (M >= G) {
        return v[0];
    } else {
        const bool hi = (q & M) != 0;
#pragma unroll
        for (int i = 0; i < G / (2 * M); i++) {
            const float keep = hi ? v[2 * i + 1] : v[2 * i];
            const float send = hi ? v[2 * i] : v[2 * i + 1];
            v[i] = keep + lane_xor<M>(send);
        }
        return group_transpose_sum<G, 2 * M>(v, q);
    }
}

// state_update_vec: n = 4 LPC with LPC in {1, 2, 4, 8, 16}.  A group of LPC
// consecutive lanes holds one channel d, 4 states per lane (one 16-byte
// access, so a wave reads and writes contiguous spans of the state), and does
// so for LPC consecutive batch rows b0 .. b0 + LPC - 1: the LPC state loads
// of a lane are in flight together, and A = -exp(A_log) is formed once for
// all of them.  The per-(row, channel) scalars are spread over the group:
// lane q loads x, dt and z of row b0 + q, forms that row's step size (the
// softplus) and its gate, and hands the step size on to the group; after the
// readout each lane holds the total of its own row (group_transpose_sum) and
// writes that row's y.  Lanes past d_in stay active for the cross-lane steps
// but touch no memory.
template <typename TIn, int LPC, bool ZOH>
__global__ __launch_bounds__(256) void state_update_vec(const StepParams p) {
    constexpr int CPB = 256 / LPC;   // channels per workgroup
    const TIn* __restrict__ xp = static_cast<const TIn*>(p.x);
    const TIn* __restrict__ dtp = static_cast<const TIn*>(p.dt);
    const TIn* __restrict__ Bm = static_cast<const TIn*>(p.B);
    const TIn* __restrict__ Cm = static_cast<const TIn*>(p.C);
    const TIn* __restrict__ zp = static_cast<const TIn*>(p.z);
    TIn* __restrict__ yp = static_cast<TIn*>(p.y);

    // Workgroup -> (group of LPC rows, tile of CPB channels), tiles fastest.
    const int d_in = int(p.d_in), n = int(p.n), nb = int(p.b);
    const int ntiles = (d_in + CPB - 1) / CPB;
    const int rg = int(blockIdx.x) / ntiles;
    const int b0 = rg * LPC;
    const int q = int(threadIdx.x) & (LPC - 1);
    const int d = (int(blockIdx.x) - rg * ntiles) * CPB + int(threadIdx.x) / LPC;
    const bool dv = d < d_in;
    // Lanes past d_in and rows past b read the last valid channel and row
    // (in bounds, results dropped) and write nothing.
    const int dc = dv ? d : d_in - 1;
    const uint32_t so = uint32_t(dc) * uint32_t(n) + 4u * uint32_t(q);   // within a state row
    const int nrows = min(LPC, nb - b0);

    typedef float f4v __attribute__((ext_vector_type(4)));
    f4v s[LPC];
    float4 Bv[LPC], Cv[LPC];
    static_for<0, LPC>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if (j < nrows) {
            const f4v* row = reinterpret_cast<const f4v*>(p.state + int64_t(b0 + j) * d_in * n);
            s[j] = __builtin_nontemporal_load(row + so / 4);
        }
    });
    const float4 al = *reinterpret_cast<const float4*>(p.A_log + so);
    static_for<0, LPC>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if (j < nrows) {
            Bv[j] = load4<TIn>(Bm + int64_t(b0 + j) * n, 4 * q);
            Cv[j] = load4<TIn>(Cm + int64_t(b0 + j) * n, 4 * q);
        }
    });
    // This lane's own row, b0 + q.
    const bool rv = dv && q < nrows;
    const uint32_t xo = uint32_t(b0 + min(q, nrows - 1)) * uint32_t(d_in) + uint32_t(dc);
    const float xq = Elem<TIn>::load(xp, xo);
    const float dlq = step_size(Elem<TIn>::load(dtp, xo), p.bias ? p.bias[dc] : 0.0f, p.softplus);
    const float gate = zp ? silu(Elem<TIn>::load(zp, xo)) : 1.0f;
    const float Dd = p.D[dc];
    const float a2[4] = {a2_from_alog(al.x), a2_from_alog(al.y), a2_from_alog(al.z), a2_from_alog(al.w)};
    float ia[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (ZOH) {
        ia[0] = inv_a_from_alog(al.x);
        ia[1] = inv_a_from_alog(al.y);
        ia[2] = inv_a_from_alog(al.z);
        ia[3] = inv_a_from_alog(al.w);
    }
    const float bxq = dlq * xq;

    float acc[LPC];
    static_for<0, LPC>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        acc[j] = 0.0f;
        if (j >= nrows) return;
        const float dl = group_bcast<LPC, j>(dlq);
        // Input term w B x with w = delta' (Euler) or the hold weight.
        const float xj = ZOH ? group_bcast<LPC, j>(xq) : 0.0f;
        const float bx = ZOH ? 0.0f : group_bcast<LPC, j>(bxq);
        const float Bk[4] = {Bv[j].x, Bv[j].y, Bv[j].z, Bv[j].w};
        float sv[4] = {s[j].x, s[j].y, s[j].z, s[j].w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float x2 = dl * a2[k];
            const float a = exp2_hw(x2);
            const float wx = ZOH ? zoh_weight(dl, x2, a, ia[k]) * xj : bx;
            sv[k] = fmaf(a, sv[k], wx * Bk[k]);
        }
        if (dv) {
            f4v* row = reinterpret_cast<f4v*>(p.state + int64_t(b0 + j) * d_in * n);
            const f4v o = {sv[0], sv[1], sv[2], sv[3]};
            __builtin_nontemporal_store(o, row + so / 4);
        }
        acc[j] = fmaf(Cv[j].x, sv[0], fmaf(Cv[j].y, sv[1], fmaf(Cv[j].z, sv[2], Cv[j].w * sv[3])));
    });
    const float total = group_transpose_sum<LPC>(acc, q);
    if (rv) Elem<TIn>::store(yp, xo, fmaf(Dd, xq, total) * gate);
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
