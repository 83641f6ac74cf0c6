// scan_kernels.h -- forward selective-scan kernels for gfx950.
//
// Both kernels compute, for every batch b, channel d and time t, with h = 0
// at t = 0 (mhpn.cn selective_scan walk-through, sections 3-5 and 7;
// jiafeimiao.top Mamba.step for the bias and the gate):
//     delta' = softplus(delta + bias[d])
//     h[k]   = exp(delta' A[d,k]) h[k] + delta' B[b,t,k] u      (A = -exp(A_log))
//     y      = sum_k C[b,t,k] h[k] + D[d] u,   then y *= silu(z) if z is given.
// exp(delta' A) and delta' B u are formed in registers and never stored.
//
// scan_seq  (state sizes n >= 3).  One lane per channel d, 64 channels per
//   workgroup; the n states of a channel are split across the S waves of the
//   workgroup, NSW states per wave (4, or 8 above n = 32), so the B and C values a wave needs at
//   step t are the same for all its lanes and come through scalar loads.
//   The per-(b,t,d) work -- softplus, delta' u, the D skip, the gate and the
//   sum of the S partial readouts -- is done once per element by the whole
//   workgroup through LDS, not once per wave.  Time is walked in chunks of T
//   steps.  L may be cut into K segments ("pieces"); workgroups take pieces in
//   ticket order (an atomic counter), segment-major, and a piece starts from
//   the state its predecessor segment published.  A piece therefore waits
//   only on a piece that an already running workgroup holds, so the wait
//   cannot deadlock; it lets the GPU balance 64-channel groups whose count is
//   not a multiple of the compute-unit count without any extra arithmetic.
//
// scan_tpar (n = 1 or 2).  One lane per channel; the W waves of a workgroup
//   take W consecutive sub-chunks of TS steps each.  Every wave scans its
//   sub-chunk from a zero state, keeping the running decay product P_t and
//   the partial outputs; the waves then combine their (P, h) aggregates
//   through LDS, (P1, h1) then (P2, h2) -> (P1 P2, P2 h1 + h2), and each wave
//   adds C_t P_t h_in to its outputs.  At n <= 2 this fix-up costs about
//   three extra operations per element, far less than the parallelism it
//   buys when b * d_in is small.
#pragma once

#include "ss_device.h"

namespace ss {

struct ScanParams {
    const void* u;
    const void* delta;
    const float* A_log;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* bias;
    void* y;
    float* last_state;
    int64_t b, L, d_in, n;
    int softplus;
    // plan
    int nblk_d;          // ceil(d_in / 64)
    int K;               // segments along L (scan_seq)
    int64_t Lseg;        // steps per segment (a multiple of the chunk length)
    uint32_t* ctl;       // [0] ticket counter, [1] error word, [kFlagOffset + i] segment-done flags
    float* handoff;      // (K - 1) * G * n * 64 states published between segments
};

constexpr int kFlagOffset = 64;
constexpr int kSpinLimit = 1 << 25;   // ~2 s of s_sleep before a wait gives up and flags an error

// Chunk length of scan_seq: every wave walks T steps between barriers.
constexpr int kSeqChunk = 32;

// Steps of B/C and (delta', delta' u) a wave reads ahead of the step it computes.
constexpr int kSeqAhead = 4;

// LDS of scan_seq: (delta', delta' u) per (t, d); the S partial readouts per
// (t, d); B and C of the chunk as fp32, grouped per wave; 16 bytes for the
// ticket.  Everything is one dynamic block starting 16-byte aligned: a static
// __shared__ variable would shift the dynamic block by its size and leave the
// 8- and 16-byte LDS accesses misaligned, which the LDS serialises.
template <int S, int NSW>
constexpr size_t seq_lds_bytes() {
    return size_t(kSeqChunk) * (64 * (sizeof(float2) + S * sizeof(float)) + 2 * S * NSW * sizeof(float)) + 16;
}

// V consecutive input elements of one row: one wide load when VEC, else V
// bounds-checked scalar loads (past-the-end elements read as 0).
template <typename TIn, int V, bool VEC>
struct Span {
    using R = Raw<TIn>;
    typename R::type v[V];
    __device__ __forceinline__ void load(const TIn* p, int64_t e, int valid) {
        if constexpr (VEC) {
            constexpr int BYTES = V * sizeof(TIn);
            static_assert(BYTES % 16 == 0 || BYTES == 8, "wide loads of 8 or 16k bytes");
            if constexpr (BYTES == 8) {
                const uint2 w = *reinterpret_cast<const uint2*>(p + e);
                const uint32_t ww[2] = {w.x, w.y};
                unpack(ww);
            } else {
                uint32_t ww[BYTES / 4];
#pragma unroll
                for (int c = 0; c < BYTES / 16; c++) {
                    const uint4 w = reinterpret_cast<const uint4*>(p + e)[c];
                    ww[4 * c] = w.x;
                    ww[4 * c + 1] = w.y;
                    ww[4 * c + 2] = w.z;
                    ww[4 * c + 3] = w.w;
                }
                unpack(ww);
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; i++) v[i] = i < valid ? R::load(p, e + i) : typename R::type(0);
        }
    }
    template <int W>
    __device__ __forceinline__ void unpack(const uint32_t (&ww)[W]) {
        if constexpr (sizeof(TIn) == 2) {
#pragma unroll
            for (int i = 0; i < W; i++) {
                v[2 * i] = ww[i] & 0xffffu;
                v[2 * i + 1] = ww[i] >> 16;
            }
        } else {
#pragma unroll
            for (int i = 0; i < W; i++) v[i] = __uint_as_float(ww[i]);
        }
    }
    __device__ __forceinline__ float f(int i) const { return R::f(v[i]); }
};

template <typename TIn, int V, bool VEC>
__device__ __forceinline__ void store_span(TIn* p, int64_t e, const float* y, int valid) {
    if constexpr (VEC && sizeof(TIn) == 2) {
        uint32_t ww[V / 2];
#pragma unroll
        for (int i = 0; i < V / 2; i++)
            ww[i] = uint32_t(f32_to_bf16(y[2 * i])) | (uint32_t(f32_to_bf16(y[2 * i + 1])) << 16);
        if constexpr (V == 4) {
            *reinterpret_cast<uint2*>(p + e) = make_uint2(ww[0], ww[1]);
        } else {
#pragma unroll
            for (int c = 0; c < V / 8; c++)
                reinterpret_cast<uint4*>(p + e)[c] = make_uint4(ww[4 * c], ww[4 * c + 1], ww[4 * c + 2], ww[4 * c + 3]);
        }
    } else if constexpr (VEC) {
#pragma unroll
        for (int c = 0; c < V / 4; c++)
            reinterpret_cast<float4*>(p + e)[c] = make_float4(y[4 * c], y[4 * c + 1], y[4 * c + 2], y[4 * c + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < V; i++)
            if (i < valid) Elem<TIn>::store(p, e + i, y[i]);
    }
}

// VEC: d_in is a multiple of the per-thread span V and the tensors are
// aligned for it, so the per-element phases use wide loads and stores.
template <typename TIn, int S, int NSW, bool VEC>
__global__ __launch_bounds__(S * 64) void scan_seq(const ScanParams p) {
    constexpr int T = kSeqChunk;
    constexpr int NT = S * 64;                     // threads
    constexpr int V = T / S;                       // consecutive channels per thread in the per-element phases
    constexpr int TPR = 64 / V;                    // threads per step row
    constexpr int NP = S * NSW;                    // states per channel, padded
    constexpr int EBC = T * NP / NT;               // B (and C) values each thread stages per chunk
    static_assert(T % S == 0 && 64 % V == 0 && NT / TPR == T, "thread tiling of a chunk");
    static_assert((T * NP) % NT == 0 && NSW % 4 == 0, "B/C tile splits evenly; states come in quads");
    using R = Raw<TIn>;
    extern __shared__ __align__(16) float smem[];
    float2* s_dw = reinterpret_cast<float2*>(smem);               // [T][64]  (delta', delta' u)
    float* s_yp = smem + 2 * T * 64;                              // [S][T][64] partial readouts
    float* s_bc = s_yp + S * T * 64;                              // [T][S][2][NSW]  B, C per wave
    int& s_ticket = *reinterpret_cast<int*>(s_bc + T * 2 * NP);

    const TIn* __restrict__ Bm = static_cast<const TIn*>(p.B);
    const TIn* __restrict__ Cm = static_cast<const TIn*>(p.C);

    const TIn* __restrict__ u = static_cast<const TIn*>(p.u);
    const TIn* __restrict__ dlt = static_cast<const TIn*>(p.delta);
    const TIn* __restrict__ zp = static_cast<const TIn*>(p.z);
    TIn* __restrict__ yp = static_cast<TIn*>(p.y);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t L = p.L, d_in = p.d_in, n = p.n;
    const int64_t G = p.b * p.nblk_d;

    int ticket;
    if (p.K == 1) {
        ticket = blockIdx.x;
    } else {
        if (tid == 0) s_ticket = atomicAdd(p.ctl, 1u);
        __syncthreads();
        ticket = __builtin_amdgcn_readfirstlane(s_ticket);
    }
    const int64_t seg = ticket / G;
    const int64_t g = ticket - seg * G;
    const int64_t bi = g / p.nblk_d;
    const int64_t dbase = (g - bi * p.nblk_d) * 64;
    const int64_t d = dbase + lane;               // channel of this lane in the recurrence
    const bool dv = d < d_in;
    const int64_t t_begin = seg * p.Lseg;
    const int64_t t_end = min(L, t_begin + p.Lseg);
    const int n0 = wave * NSW;

    // Per-element phases: thread owns step row er of the chunk, channels ec .. ec+V.
    const int er = tid / TPR;
    const int ec = (tid - er * TPR) * V;
    const int64_t ech = dbase + ec;               // first channel of the span
    const int evalid = int(max<int64_t>(0, min<int64_t>(V, d_in - ech)));
    const int64_t ech_c = evalid > 0 ? ech : 0;   // loads of an empty span stay in bounds

    float A2[NSW], h[NSW];
#pragma unroll
    for (int q = 0; q < NSW; q++) {
        A2[q] = (dv && n0 + q < n) ? a2_from_alog(p.A_log[d * n + n0 + q]) : 0.0f;
        h[q] = 0.0f;
    }
    float Dv[V], bias_v[V];
#pragma unroll
    for (int i = 0; i < V; i++) {
        Dv[i] = i < evalid ? p.D[ech + i] : 0.0f;
        bias_v[i] = (i < evalid && p.bias) ? p.bias[ech + i] : 0.0f;
    }
    const bool gated = zp != nullptr;

    if (seg > 0) {
        // Wait for the previous segment of this channel group, then take its state.
        if (tid == 0) {
            uint32_t* flag = p.ctl + kFlagOffset + (seg - 1) * G + g;
            int spins = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > kSpinLimit) {
                    atomicOr(p.ctl + 1, 1u);
                    break;
                }
            }
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        const float* src = p.handoff + ((seg - 1) * G + g) * n * 64;
#pragma unroll
        for (int q = 0; q < NSW; q++)
            if (n0 + q < n) h[q] = src[(n0 + q) * 64 + lane];
    }

    // B/C staging: thread owns tile slots f = m*NT + tid, step f / NP, state f % NP.
    Span<TIn, V, VEC> su, sd, sz;
    typename R::type rb[EBC], rc[EBC];
    auto load_ud = [&](int64_t tc) {
        const int64_t t = min(tc + er, L - 1);
        const int64_t e = (bi * L + t) * d_in + ech_c;
        su.load(u, e, evalid);
        sd.load(dlt, e, evalid);
#pragma unroll
        for (int m = 0; m < EBC; m++) {
            const int f = m * NT + tid;
            const int64_t tb = min(tc + f / NP, L - 1);
            const int64_t k = min<int64_t>(f % NP, n - 1);
            rb[m] = R::load(Bm, (bi * L + tb) * n + k);
            rc[m] = R::load(Cm, (bi * L + tb) * n + k);
        }
    };
    load_ud(t_begin);

    for (int64_t tc = t_begin; tc < t_end; tc += T) {
        const int nt = int(min<int64_t>(T, t_end - tc));
        const bool rv = er < nt;

        // Per-element phase 1: step size and delta' u, once per (t, d).
        float uv[V];
        {
            float2 dwv[V];
#pragma unroll
            for (int i = 0; i < V; i++) {
                const bool ok = rv && i < evalid;
                const float dl = ok ? step_size(sd.f(i), bias_v[i], p.softplus) : 0.0f;
                uv[i] = ok ? su.f(i) : 0.0f;
                dwv[i] = make_float2(dl, dl * uv[i]);
            }
            float4* dst = reinterpret_cast<float4*>(s_dw + er * 64 + ec);
#pragma unroll
            for (int i = 0; i < V / 2; i++) dst[i] = make_float4(dwv[2 * i].x, dwv[2 * i].y, dwv[2 * i + 1].x, dwv[2 * i + 1].y);
        }
#pragma unroll
        for (int m = 0; m < EBC; m++) {
            const int f = m * NT + tid;
            const int j = f / NP, k = f % NP;
            const int w = k / NSW, q = k % NSW;
            const bool ok = k < n;
            float* dst = s_bc + ((j * S + w) * 2) * NSW + q;
            dst[0] = ok ? R::f(rb[m]) : 0.0f;
            dst[NSW] = ok ? R::f(rc[m]) : 0.0f;
        }
        __syncthreads();

        // Loads for the next chunk and the gate of this one, in flight during the recurrence.
        if (gated) {
            const int64_t t = min(tc + er, L - 1);
            sz.load(zp, (bi * L + t) * d_in + ech_c, evalid);
        }
        if (tc + T < t_end) load_ud(tc + T);

        // Recurrence over the chunk: this wave's NSW states of every channel.
        // (delta', delta' u) and the wave's B/C values are read from LDS
        // kSeqAhead steps before they are used.  Steps past nt have delta' = 0,
        // which leaves the state unchanged.
        {
            constexpr int D = kSeqAhead;
            constexpr int NQ = NSW / 4;
            float2 dw[D];
            float4 bq[D][NQ], cq[D][NQ];
            const float* bcw = s_bc + wave * 2 * NSW;
            auto fetch = [&](int j, int slot) {
                dw[slot] = s_dw[j * 64 + lane];
                const float4* r = reinterpret_cast<const float4*>(bcw + j * S * 2 * NSW);
#pragma unroll
                for (int qq = 0; qq < NQ; qq++) {
                    bq[slot][qq] = r[qq];
                    cq[slot][qq] = r[NQ + qq];
                }
            };
#pragma unroll
            for (int j = 0; j < D; j++) fetch(j, j);
            float* ypw = s_yp + wave * T * 64;
#pragma unroll
            for (int j = 0; j < T; j++) {
                const int slot = j % D;
                const float2 dj = dw[slot];
                float bv[NSW], cv[NSW];
#pragma unroll
                for (int qq = 0; qq < NQ; qq++) {
                    bv[4 * qq] = bq[slot][qq].x; bv[4 * qq + 1] = bq[slot][qq].y;
                    bv[4 * qq + 2] = bq[slot][qq].z; bv[4 * qq + 3] = bq[slot][qq].w;
                    cv[4 * qq] = cq[slot][qq].x; cv[4 * qq + 1] = cq[slot][qq].y;
                    cv[4 * qq + 2] = cq[slot][qq].z; cv[4 * qq + 3] = cq[slot][qq].w;
                }
                if (j + D < T) fetch(j + D, slot);
                float acc = 0.0f;
#pragma unroll
                for (int q = 0; q < NSW; q++) {
                    const float a = exp2_hw(dj.x * A2[q]);
                    h[q] = fmaf(a, h[q], dj.y * bv[q]);
                    acc = fmaf(cv[q], h[q], acc);
                }
                ypw[j * 64 + lane] = acc;
            }
        }
        __syncthreads();

        // Per-element phase 2: sum the partial readouts, D skip, gate, store.
        {
            float yv[V];
#pragma unroll
            for (int i = 0; i < V; i++) yv[i] = 0.0f;
#pragma unroll
            for (int w = 0; w < S; w++) {
                const float4* src = reinterpret_cast<const float4*>(s_yp + (w * T + er) * 64 + ec);
#pragma unroll
                for (int i = 0; i < V / 4; i++) {
                    const float4 v4 = src[i];
                    yv[4 * i] += v4.x;
                    yv[4 * i + 1] += v4.y;
                    yv[4 * i + 2] += v4.z;
                    yv[4 * i + 3] += v4.w;
                }
            }
#pragma unroll
            for (int i = 0; i < V; i++) {
                yv[i] = fmaf(Dv[i], uv[i], yv[i]);
                if (gated) yv[i] *= silu(sz.f(i));
            }
            if (rv && evalid > 0) store_span<TIn, V, VEC>(yp, (bi * L + tc + er) * d_in + ech, yv, evalid);
        }
    }

    if (seg + 1 < p.K) {
        // Publish the state for the next segment.
        float* dst = p.handoff + (seg * G + g) * n * 64;
#pragma unroll
        for (int q = 0; q < NSW; q++)
            if (n0 + q < n) dst[(n0 + q) * 64 + lane] = h[q];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(p.ctl + kFlagOffset + seg * G + g, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else if (p.last_state && dv) {
#pragma unroll
        for (int q = 0; q < NSW; q++)
            if (n0 + q < n) p.last_state[(bi * d_in + d) * n + n0 + q] = h[q];
    }
}

// Clears the ticket counter, the error word and the segment flags.
__global__ void scan_ctl_reset(uint32_t* ctl, int64_t words) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < words; i += int64_t(gridDim.x) * blockDim.x)
        ctl[i] = 0u;
}

constexpr int kTparSteps = 16;   // TS: steps per wave per chunk

template <typename TIn, int NS, int W>
__global__ __launch_bounds__(W * 64) void scan_tpar(const ScanParams p) {
    constexpr int TS = kTparSteps;
    __shared__ float2 s_agg[2][W][NS][64];     // (P, h) per wave, double-buffered by chunk parity

    const TIn* __restrict__ u = static_cast<const TIn*>(p.u);
    const TIn* __restrict__ dlt = static_cast<const TIn*>(p.delta);
    const TIn* __restrict__ Bm = static_cast<const TIn*>(p.B);
    const TIn* __restrict__ Cm = static_cast<const TIn*>(p.C);
    const TIn* __restrict__ zp = static_cast<const TIn*>(p.z);
    TIn* __restrict__ yp = static_cast<TIn*>(p.y);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t L = p.L, d_in = p.d_in, n = p.n;
    const int64_t bi = blockIdx.x / p.nblk_d;
    const int64_t d = (blockIdx.x - bi * p.nblk_d) * 64 + lane;
    const bool dv = d < d_in;

    float A2[NS], hc[NS];
#pragma unroll
    for (int q = 0; q < NS; q++) {
        A2[q] = (dv && q < n) ? a2_from_alog(p.A_log[d * n + q]) : 0.0f;
        hc[q] = 0.0f;                           // state at the start of the current chunk
    }
    const float Dd = dv ? p.D[d] : 0.0f;
    const float bias_d = (dv && p.bias) ? p.bias[d] : 0.0f;

    int parity = 0;
    for (int64_t tc = 0; tc < L; tc += int64_t(W) * TS, parity ^= 1) {
        const int64_t t0 = tc + int64_t(wave) * TS;        // first step of this wave's sub-chunk
        const int nt = int(max<int64_t>(0, min<int64_t>(TS, L - t0)));
        const int64_t row0 = bi * L + t0;

        float uv[TS], dv_[TS];
#pragma unroll
        for (int j = 0; j < TS; j++) {
            uv[j] = 0.0f;
            dv_[j] = 0.0f;
            if (j < nt && dv) {
                const int64_t e = (row0 + j) * d_in + d;
                uv[j] = Elem<TIn>::load(u, e);
                dv_[j] = Elem<TIn>::load(dlt, e);
            }
        }
        float yl[TS], pc[TS][NS];
        float h[NS], P[NS];
#pragma unroll
        for (int q = 0; q < NS; q++) { h[q] = 0.0f; P[q] = 1.0f; }
#pragma unroll
        for (int j = 0; j < TS; j++) {
            const bool tv = j < nt;
            const float dl = (tv && dv) ? step_size(dv_[j], bias_d, p.softplus) : 0.0f;
            const float wv = dl * uv[j];
            float acc = Dd * uv[j];
#pragma unroll
            for (int q = 0; q < NS; q++) {
                const bool qv = tv && q < n;
                const float Bq = qv ? Elem<TIn>::load(Bm, (row0 + j) * n + q) : 0.0f;
                const float Cq = qv ? Elem<TIn>::load(Cm, (row0 + j) * n + q) : 0.0f;
                const float a = exp2_hw(dl * A2[q]);
                h[q] = fmaf(a, h[q], wv * Bq);
                P[q] *= a;
                acc = fmaf(Cq, h[q], acc);
                pc[j][q] = Cq * P[q];
            }
            yl[j] = acc;
        }
#pragma unroll
        for (int q = 0; q < NS; q++) s_agg[parity][wave][q][lane] = make_float2(P[q], h[q]);
        __syncthreads();

        // State entering this wave's sub-chunk, and the state after the whole chunk.
        float hin[NS];
#pragma unroll
        for (int q = 0; q < NS; q++) hin[q] = hc[q];
        for (int w = 0; w < W; w++) {
            if (w == wave) {
#pragma unroll
                for (int q = 0; q < NS; q++) hin[q] = hc[q];
            }
#pragma unroll
            for (int q = 0; q < NS; q++) {
                const float2 ag = s_agg[parity][w][q][lane];
                hc[q] = fmaf(ag.x, hc[q], ag.y);
            }
        }
#pragma unroll
        for (int j = 0; j < TS; j++) {
            if (j < nt && dv) {
                float acc = yl[j];
#pragma unroll
                for (int q = 0; q < NS; q++) acc = fmaf(pc[j][q], hin[q], acc);
                const int64_t e = (row0 + j) * d_in + d;
                if (zp) acc *= silu(Elem<TIn>::load(zp, e));
                Elem<TIn>::store(yp, e, acc);
            }
        }
    }
    if (p.last_state && dv && wave == 0) {
#pragma unroll
        for (int q = 0; q < NS; q++)
            if (q < n) p.last_state[(bi * d_in + d) * n + q] = hc[q];
    }
}

}  // namespace ss
