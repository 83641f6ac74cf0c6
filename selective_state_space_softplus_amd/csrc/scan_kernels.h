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

// Chunk length of scan_seq: the workgroup advances T steps per barrier.
constexpr int kSeqChunk = 16;

// Steps of B and C a wave reads ahead of the step it computes.
constexpr int kSeqAhead = 4;

// LDS of scan_seq, double-buffered by chunk parity: (delta', delta' u) per
// (t, d), two steps interleaved per channel; the S partial readouts per
// (t, d); B and C of the chunk as fp32, grouped per wave; then 16 bytes for
// the ticket.  It is one dynamic block that starts 16-byte aligned: a static
// __shared__ variable would shift it by its size and leave the 8- and 16-byte
// LDS accesses misaligned, which the LDS serialises.
template <int S, int NSW>
constexpr size_t seq_lds_bytes() {
    return 2 * size_t(kSeqChunk) * (64 * (sizeof(float2) + S * sizeof(float)) + 2 * S * NSW * sizeof(float)) + 16;
}

// V consecutive input elements of one row, kept as the raw 32-bit words that
// were loaded (one wide load when VEC, else V bounds-checked element loads,
// past-the-end elements reading as 0) and widened to fp32 only when used, so
// a load stays in flight until its value is needed.
template <typename TIn, int V, bool VEC>
struct Span {
    static constexpr bool kHalf = sizeof(TIn) == 2;
    static constexpr int NW = VEC ? (V * int(sizeof(TIn)) + 3) / 4 : V;
    uint32_t w[NW];

    __device__ __forceinline__ void load(const TIn* base, uint32_t e, int valid) {
        const TIn* p = base;
        if constexpr (VEC) {
            constexpr int BYTES = V * int(sizeof(TIn));
            if constexpr (BYTES == 4) {
                w[0] = *reinterpret_cast<const uint32_t*>(p + e);
            } else if constexpr (BYTES == 8) {
                const uint2 v = *reinterpret_cast<const uint2*>(p + e);
                w[0] = v.x;
                w[1] = v.y;
            } else {
                static_assert(BYTES % 16 == 0, "wide loads of 4, 8 or 16k bytes");
#pragma unroll
                for (int c = 0; c < BYTES / 16; c++) {
                    const uint4 v = reinterpret_cast<const uint4*>(p + e)[c];
                    w[4 * c] = v.x;
                    w[4 * c + 1] = v.y;
                    w[4 * c + 2] = v.z;
                    w[4 * c + 3] = v.w;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; i++) {
                if constexpr (kHalf)
                    w[i] = i < valid ? uint32_t(reinterpret_cast<const uint16_t*>(p)[e + i]) : 0u;
                else
                    w[i] = i < valid ? __float_as_uint(reinterpret_cast<const float*>(p)[e + i]) : 0u;
            }
        }
    }
    __device__ __forceinline__ float f(int i) const {
        if constexpr (!kHalf) return __uint_as_float(w[i]);
        else if constexpr (!VEC) return __uint_as_float(w[i] << 16);
        else return (i & 1) ? __uint_as_float(w[i / 2] & 0xffff0000u) : __uint_as_float(w[i / 2] << 16);
    }
};

template <typename TIn, int V, bool VEC>
__device__ __forceinline__ void store_span(TIn* p, uint32_t e, const float* y, int valid) {
    if constexpr (VEC && sizeof(TIn) == 2) {
        uint32_t ww[(V + 1) / 2];
#pragma unroll
        for (int i = 0; i < V / 2; i++)
            ww[i] = uint32_t(f32_to_bf16(y[2 * i])) | (uint32_t(f32_to_bf16(y[2 * i + 1])) << 16);
        if constexpr (V == 2) {
            *reinterpret_cast<uint32_t*>(p + e) = ww[0];
        } else if constexpr (V == 4) {
            *reinterpret_cast<uint2*>(p + e) = make_uint2(ww[0], ww[1]);
        } else {
#pragma unroll
            for (int c = 0; c < V / 8; c++)
                reinterpret_cast<uint4*>(p + e)[c] = make_uint4(ww[4 * c], ww[4 * c + 1], ww[4 * c + 2], ww[4 * c + 3]);
        }
    } else if constexpr (VEC) {
        if constexpr (V == 2) {
            *reinterpret_cast<float2*>(p + e) = make_float2(y[0], y[1]);
        } else {
#pragma unroll
            for (int c = 0; c < V / 4; c++)
                reinterpret_cast<float4*>(p + e)[c] = make_float4(y[4 * c], y[4 * c + 1], y[4 * c + 2], y[4 * c + 3]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; i++)
            if (i < valid) Elem<TIn>::store(p, e + i, y[i]);
    }
}

// VEC: d_in is a multiple of the per-thread span V and the tensors are
// aligned for it, so the per-element phases use wide loads and stores.
// SP: delta' = softplus(delta + bias) (else delta + bias).  GATE: z is given.
//
// One barrier per chunk c of T steps.  Between two barriers every wave
//   - reads (delta', delta' u) of chunk c for its 64 lanes from LDS, and the
//     partial readouts of chunk c-1, all up front;
//   - runs the recurrence of chunk c from registers, reading its B and C
//     values of each step from LDS kSeqAhead steps ahead (the only LDS
//     accesses inside the loop, so every wait is for a read issued steps
//     earlier);
//   - interleaves the per-element work: phase 2 of chunk c-1 (partial sums,
//     D skip, gate) and phase 1 of chunk c+1 (step size, delta' u), whose
//     global loads were issued two chunks earlier;
//   - then writes its partial readouts of chunk c, the phase-1 results and the
//     B, C values of chunk c+1 to LDS, and stores y of chunk c-1.
// LDS buffers alternate with the chunk parity, so no buffer is written and
// read by different waves between two barriers.
template <typename TIn, int S, int NSW, bool VEC, bool SP, bool GATE>
__global__ __launch_bounds__(S * 64) void scan_seq(const ScanParams p) {
    constexpr int T = kSeqChunk;
    constexpr int NT = S * 64;                     // threads
    constexpr int V = T / S;                       // consecutive channels per thread in the per-element phases
    constexpr int TPR = 64 / V;                    // threads per step row
    constexpr int DW_BUF = T * 64 * 2;             // floats per (delta', delta' u) buffer
    constexpr int YP_BUF = S * T * 64;             // floats per partial-readout buffer
    constexpr int NP = S * NSW;                    // states per channel, padded
    constexpr int BC_BUF = T * 2 * NP;             // floats per B/C buffer
    constexpr int EBC = (T * NP + NT - 1) / NT;    // B (and C) values each thread stages per chunk
    constexpr int D = kSeqAhead;
    constexpr int NR = NSW / 2;                    // float4 reads per step: NSW values of B then NSW of C
    static_assert(T % S == 0 && 64 % V == 0 && NT / TPR == T, "thread tiling of a chunk");
    static_assert(NSW % 2 == 0 && T % 2 == 0 && T % D == 0, "tiles split evenly");
    extern __shared__ __align__(16) float smem[];
    float* s_dw = smem;                            // [2][T/2][64][4]: (delta'_j, w_j, delta'_j+1, w_j+1)
    float* s_yp = smem + 2 * DW_BUF;               // [2][S][T][64]
    float* s_bc = s_yp + 2 * YP_BUF;               // [2][T][S][2][NSW]
    int& s_ticket = *reinterpret_cast<int*>(s_bc + 2 * BC_BUF);
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
    const int64_t t_end = imin(L, t_begin + p.Lseg);
    const int nchunks = int((t_end - t_begin + T - 1) / T);
    const int n0 = wave * NSW;

    // Per-element phases: thread owns step row er of a chunk, channels ec .. ec+V.
    const int er = tid / TPR;
    const int ec = (tid - er * TPR) * V;
    const int64_t ech = dbase + ec;
    const int evalid = int(imax(0, imin(V, d_in - ech)));
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

    // Address arithmetic: uniform 64-bit chunk bases (scalar unit) plus
    // per-thread 32-bit offsets; rows past the end of L are clamped to the
    // last row (those values are masked and never stored).  The host keeps
    // d_in < 2^24 and T * d_in below 2^31.
    const uint32_t d_in32 = uint32_t(d_in);
    const int64_t brow = bi * L;                  // first (b, t) row of this batch
    auto rows_left = [&](int k) -> int { return int(imax(-1, imin(T, t_end - (t_begin + int64_t(k) * T)))); };
    auto row_off = [&](int k) -> uint32_t {       // element offset of this thread's row in chunk k
        const int64_t lim = imin(T - 1, L - 1 - (t_begin + int64_t(k) * T));
        return uint32_t(__umul24(umin(uint32_t(er), uint32_t(imax(lim, 0))), d_in32)) + uint32_t(ech_c);
    };
    auto chunk_row = [&](int k) -> int64_t { return brow + imin(t_begin + int64_t(k) * T, L - 1); };

    // B/C staging: thread owns tile slots f = m*NT + tid, step f / NP, state f % NP.
    const uint32_t n32 = uint32_t(n);
    uint32_t bc_row[EBC], bc_col[EBC];
#pragma unroll
    for (int m = 0; m < EBC; m++) {
        const int f = int(imin(m * NT + tid, T * NP - 1));
        bc_row[m] = uint32_t(f / NP);
        bc_col[m] = uint32_t(imin(f % NP, n - 1));
    }
    auto load_bc = [&](uint32_t* rb, uint32_t* rc, int k) {
        const int64_t tcl = imin(t_begin + int64_t(k) * T, L - 1);
        const uint32_t blim = uint32_t(imax(0, imin(T - 1, L - 1 - tcl)));
        const TIn* Bc = Bm + (brow + tcl) * n;
        const TIn* Cc = Cm + (brow + tcl) * n;
#pragma unroll
        for (int m = 0; m < EBC; m++) {
            const uint32_t o = uint32_t(__umul24(umin(bc_row[m], blim), n32)) + bc_col[m];
            if constexpr (sizeof(TIn) == 2) {
                rb[m] = reinterpret_cast<const uint16_t*>(Bc)[o];
                rc[m] = reinterpret_cast<const uint16_t*>(Cc)[o];
            } else {
                rb[m] = __float_as_uint(reinterpret_cast<const float*>(Bc)[o]);
                rc[m] = __float_as_uint(reinterpret_cast<const float*>(Cc)[o]);
            }
        }
    };
    auto stage_bc = [&](const uint32_t* rb, const uint32_t* rc, int k) {
        const int left = rows_left(k);
#pragma unroll
        for (int m = 0; m < EBC; m++) {
            const int f = m * NT + tid;
            if ((T * NP) % NT != 0 && f >= T * NP) break;
            const int j = f / NP, kk = f % NP;
            const int w = kk / NSW, q = kk % NSW;
            const bool ok = j < left && kk < n;
            float* dst = s_bc + (k & 1) * BC_BUF + ((j * S + w) * 2) * NSW + q;
            dst[0] = ok ? (sizeof(TIn) == 2 ? __uint_as_float(rb[m] << 16) : __uint_as_float(rb[m])) : 0.0f;
            dst[NSW] = ok ? (sizeof(TIn) == 2 ? __uint_as_float(rc[m] << 16) : __uint_as_float(rc[m])) : 0.0f;
        }
    };

    auto load_chunk = [&](Span<TIn, V, VEC>& su, Span<TIn, V, VEC>& sd, int k) {
        const int64_t base = chunk_row(k) * d_in;
        const uint32_t off = row_off(k);
        su.load(u + base, off, evalid);
        sd.load(dlt + base, off, evalid);
    };
    auto load_z = [&](Span<TIn, V, VEC>& zs, int k) { zs.load(zp + chunk_row(k) * d_in, row_off(k), evalid); };

    // Phase 1 of element i of chunk k: (delta', delta' u); returns u via uv.
    auto phase1 = [&](const Span<TIn, V, VEC>& su, const Span<TIn, V, VEC>& sd, int k, int i, float& uv) {
        const bool ok = er < rows_left(k) && i < evalid;
        const float x = sd.f(i) + bias_v[i];
        const float dl = ok ? (SP ? softplus(x) : x) : 0.0f;
        uv = ok ? su.f(i) : 0.0f;
        return make_float2(dl, dl * uv);
    };
    auto store_dw = [&](int k, const float2* dwv) {
#pragma unroll
        for (int i = 0; i < V; i++) {
            float* dst = s_dw + (k & 1) * DW_BUF + ((er >> 1) * 64 + ec + i) * 4 + (er & 1) * 2;
            *reinterpret_cast<float2*>(dst) = dwv[i];
        }
    };
    auto store_y = [&](int k, const float* yv) {
        if (k >= 0 && er < rows_left(k) && evalid > 0)
            store_span<TIn, V, VEC>(yp + (brow + t_begin + int64_t(k) * T) * d_in, uint32_t(er) * d_in32 + uint32_t(ech),
                                    yv, evalid);
    };

    // Pipeline fill: phase 1 of chunk 0 into LDS; loads of chunk 1 in flight.
    Span<TIn, V, VEC> su_n, sd_n, su_n2, sd_n2, z_cur, z_prev;
#pragma unroll
    for (int i = 0; i < Span<TIn, V, VEC>::NW; i++) z_prev.w[i] = 0u;
    float uv_prev[V], uv_cur[V], uv_next[V];
    uint32_t rb_n[EBC], rc_n[EBC], rb_n2[EBC], rc_n2[EBC];
    {
        load_chunk(su_n, sd_n, 0);
        load_bc(rb_n, rc_n, 0);
        float2 dwv[V];
#pragma unroll
        for (int i = 0; i < V; i++) dwv[i] = phase1(su_n, sd_n, 0, i, uv_cur[i]);
        store_dw(0, dwv);
        stage_bc(rb_n, rc_n, 0);
    }
    load_chunk(su_n, sd_n, 1);
    load_bc(rb_n, rc_n, 1);
    if (GATE) load_z(z_cur, 0);
#pragma unroll
    for (int i = 0; i < V; i++) uv_prev[i] = 0.0f;
    __syncthreads();

    for (int c = 0; c < nchunks; c++) {
        const int64_t tc = t_begin + int64_t(c) * T;
        // Global loads two chunks ahead and the gate of the next chunk.
        load_chunk(su_n2, sd_n2, c + 2);
        load_bc(rb_n2, rc_n2, c + 2);
        Span<TIn, V, VEC> z_new;
        if (GATE) load_z(z_new, c + 1);

        // All LDS reads of this chunk, up front.
        float4 dwq[T / 2];
        {
            const float4* src = reinterpret_cast<const float4*>(s_dw + (c & 1) * DW_BUF) + lane;
#pragma unroll
            for (int pr = 0; pr < T / 2; pr++) dwq[pr] = src[pr * 64];
        }
        float ypv[S][V];
        {
            const float* src = s_yp + ((c - 1) & 1) * YP_BUF + er * 64 + ec;
#pragma unroll
            for (int w = 0; w < S; w++)
#pragma unroll
                for (int i = 0; i < V; i++) ypv[w][i] = src[w * T * 64 + i];
        }

        float ypart[T];
        float yout[V];
        float2 dwn[V];
        const float* bcw = s_bc + (c & 1) * BC_BUF + wave * 2 * NSW;
        float4 bcq[D][NR];
        auto fetch_bc = [&](int j) {
            const float4* r = reinterpret_cast<const float4*>(bcw + j * S * 2 * NSW);
#pragma unroll
            for (int qq = 0; qq < NR; qq++) bcq[j % D][qq] = r[qq];
        };
#pragma unroll
        for (int j = 0; j < D; j++) fetch_bc(j);
#pragma unroll
        for (int j = 0; j < T; j++) {
            const int slot = j % D;
            const float4 dq = dwq[j / 2];
            const float dl = (j & 1) ? dq.z : dq.x;
            const float wv = (j & 1) ? dq.w : dq.y;
            float bcv[2 * NSW];
#pragma unroll
            for (int qq = 0; qq < NR; qq++) {
                bcv[4 * qq] = bcq[slot][qq].x;
                bcv[4 * qq + 1] = bcq[slot][qq].y;
                bcv[4 * qq + 2] = bcq[slot][qq].z;
                bcv[4 * qq + 3] = bcq[slot][qq].w;
            }
            if (j + D < T) fetch_bc(j + D);
            float acc = 0.0f;
#pragma unroll
            for (int q = 0; q < NSW; q++) {
                const float a = exp2_hw(dl * A2[q]);
                h[q] = fmaf(a, h[q], wv * bcv[q]);
                acc = fmaf(bcv[NSW + q], h[q], acc);
            }
            ypart[j] = acc;
            // Interleaved per-element work after every T/V steps.
            if ((j + 1) % (T / V) == 0) {
                const int i = (j + 1) / (T / V) - 1;
                float acc2 = 0.0f;
#pragma unroll
                for (int w = 0; w < S; w++) acc2 += ypv[w][i];
                acc2 = fmaf(Dv[i], uv_prev[i], acc2);
                if (GATE) acc2 *= silu(z_prev.f(i));
                yout[i] = acc2;
                dwn[i] = phase1(su_n, sd_n, c + 1, i, uv_next[i]);
            }
        }
        // LDS writes of this chunk, then the y store of chunk c-1.
        {
            float* dst = s_yp + (c & 1) * YP_BUF + wave * T * 64 + lane;
#pragma unroll
            for (int j = 0; j < T; j++) dst[j * 64] = ypart[j];
        }
        store_dw(c + 1, dwn);
        stage_bc(rb_n, rc_n, c + 1);
        store_y(c - 1, yout);
#pragma unroll
        for (int i = 0; i < V; i++) {
            uv_prev[i] = uv_cur[i];
            uv_cur[i] = uv_next[i];
        }
        z_prev = z_cur;
        z_cur = z_new;
        su_n = su_n2;
        sd_n = sd_n2;
#pragma unroll
        for (int m = 0; m < EBC; m++) {
            rb_n[m] = rb_n2[m];
            rc_n[m] = rc_n2[m];
        }
        __syncthreads();
    }
    // Pipeline drain: phase 2 of the last chunk.
    {
        const float* src = s_yp + ((nchunks - 1) & 1) * YP_BUF + er * 64 + ec;
        float yout[V];
#pragma unroll
        for (int i = 0; i < V; i++) {
            float acc2 = 0.0f;
#pragma unroll
            for (int w = 0; w < S; w++) acc2 += src[w * T * 64 + i];
            acc2 = fmaf(Dv[i], uv_prev[i], acc2);
            if (GATE) acc2 *= silu(z_prev.f(i));
            yout[i] = acc2;
        }
        store_y(nchunks - 1, yout);
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
        const int nt = int(imax(0, imin(TS, L - t0)));
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
