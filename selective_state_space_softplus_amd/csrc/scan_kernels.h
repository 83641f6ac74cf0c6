// scan_kernels.h -- forward selective-scan kernels for gfx950.
//
// Both kernels compute, for every batch b, channel d and time t, with h = 0
// at t = 0 (mhpn.cn selective_scan walk-through, sections 3-5 and 7;
// jiafeimiao.top Mamba.step for the bias and the gate):
//     delta' = softplus(delta + bias[d])
//     h[k]   = exp(delta' A[d,k]) h[k] + delta' B[b,t,k] u      (A = -exp(A_log))
//     y      = sum_k C[b,t,k] h[k] + D[d] u,   then y *= silu(z) if z is given.
// exp(delta' A) and delta' B u are formed in registers and never stored.
// scan_seq also takes a given initial state h0 and the zero-order-hold input
// term (exp(delta' A) - 1) / A B u of the same page's section 6, and runs
// VMamba's cross scan (githubissues.com VMamba issue 206): batch row 4m + k is
// traversal direction k of feature map m, whose u rows are read from the map
// in that direction's order; cross_merge then adds the four outputs back.
//
// scan_seq  (state sizes n >= 3).  One lane per channel d, 64 channels per
//   workgroup; the n states of a channel are split across the SC recurrence
//   waves of the workgroup, NSW states per wave (2, 4 or 8), so the B and C
//   values a wave needs at step t are the same for all its lanes (wave-uniform
//   LDS reads).  The per-(b,t,d) work -- softplus, delta' u, the D skip, the
//   gate and the sum of the SC partial readouts -- is done once per element by
//   the workgroup's element waves, not once per recurrence wave.  Time is walked in chunks of T
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

#include <type_traits>

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
    const float* h0;     // (b, d_in, n) initial state, or null for zero (scan_seq)
    float* ckpt;         // (b, nck, n, d_in) states after every kCkptSteps steps, or null (scan_seq)
    const void* dy;      // gradient of y: with dz, scan_seq writes dz in place of y (gated scans)
    void* dz;
    void* ypre;          // gated scans: the readout before the gate, (b, L, d_in), or null (scan_seq)
    int nck;             // checkpoints per batch row: (L - 1) / kCkptSteps
    int64_t b, L, d_in, n;
    int softplus;
    int cross_h, cross_w; // cross scan: map height and width (L = cross_h * cross_w)
    // plan
    int nblk_d;          // ceil(d_in / 64)
    int K;               // segments along L (scan_seq)
    int64_t Lseg;        // steps per segment (a multiple of the chunk length)
    uint32_t* ctl;       // [0] ticket counter, [kFlagOffset + i] segment-done flags
    float* handoff;      // (K - 1) * G * n * 64 states published between segments
    uint32_t* err;       // status words of the call: [0] nonzero once a segment wait gave up, [1] never set
    int spin_limit;      // polls before a segment wait gives up
    int wait_never;      // nonzero: segment waits poll err[1] (never set), so each gives up after spin_limit polls
};

constexpr int kFlagOffset = 64;

// Steps between the states the forward scan saves for the backward pass, and
// the chunk length of the backward pass.
constexpr int kCkptSteps = 8;
constexpr int kSpinLimit = 1 << 25;   // ~2 s of s_sleep before a wait gives up and flags an error

// One thread waits until the segment flag `flag` is set, or gives up after
// `limit` polls: then it sets err[0] and returns true.  The flag and the
// state it guards are device-coherent atomics (see the end of scan_seq).
__device__ __forceinline__ bool wait_segment_flag(const uint32_t* flag, uint32_t* err, int limit) {
    int spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > limit) {
            atomicOr(err, 1u);
            return true;
        }
    }
    return false;
}

// Steps of (delta', delta' u) a recurrence wave reads from LDS ahead of the
// step it computes.
constexpr int kSeqAhead = 4;

// Element waves per workgroup of scan_seq (one per SIMD).
constexpr int kSeqElemWaves = 4;

// Byte layout of the LDS of scan_seq<T, SC recurrence waves, NP padded
// states, ES-byte inputs>.  All rings are indexed by chunk % 3 (partial
// readouts: chunk % 2).  Raw inputs arrive by direct-to-LDS loads: a u, delta
// or z tile holds T rows of 64 channels, ES bytes per element when WIDE
// (16-byte loads) else 4 bytes per element (one element load per lane, which
// fills a 4-byte slot); B and C hold T * NP consecutive elements of their
// (b, L, n) array in 4-byte slots.  The block starts 16-byte aligned: a
// static __shared__ variable would shift it by its size and leave the wide
// LDS accesses misaligned, which the LDS serialises.
template <int T, int SC, int NP, int ES, bool WIDE>
struct SeqLds {
    static constexpr int XES = WIDE ? ES : 4;                  // bytes per raw u/delta/z element
    static constexpr int DW = T * 64 * 8;                      // (delta', delta' u) of a chunk
    static constexpr int YP = SC * T * 64 * 4;                 // partial readouts of a chunk
    static constexpr int BC = T * 2 * NP * 4;                  // B and C of a chunk as fp32, grouped per wave
    static constexpr int RX = T * 64 * XES;                    // raw u, delta or z tile
    static constexpr int RBC = (T * NP + 63) / 64 * 256;       // raw B or C block (whole 64-lane loads)
    static constexpr int off_dw = 0;
    static constexpr int off_yp = off_dw + 3 * DW;
    static constexpr int off_bc = off_yp + 2 * YP;
    static constexpr int off_ru = off_bc + 3 * BC;             // [3][u, delta] tiles
    static constexpr int off_rbc = off_ru + 6 * RX;            // [3][B, C] blocks
    static constexpr int off_rz = off_rbc + 6 * RBC;           // [3] z tiles
    static constexpr int off_ticket = off_rz + 3 * RX;
    static constexpr int bytes = off_ticket + 16;
};

// Chunk length of scan_seq: 16 steps, or 8 where the LDS of 16 would not fit
// (raw tiles of 4-byte slots with n > 32).
template <typename TIn, int SC, int NSW, bool WIDE>
constexpr int seq_chunk() {
    return SeqLds<16, SC, SC * NSW, int(sizeof(TIn)), WIDE>::bytes <= 160 * 1024 ? 16 : 8;
}

// VEC-style output store of V consecutive elements (one wide store), or V
// element stores of which the first `valid` happen.
template <typename TIn, int V, bool VEC>
__device__ __forceinline__ void store_span(TIn* p, uint32_t e, const float* y, int valid) {
    if constexpr (VEC && sizeof(TIn) == 2) {
        uint32_t ww[(V + 1) / 2];
#pragma unroll
        for (int i = 0; i < V / 2; i++) ww[i] = f32x2_to_bf16x2(y[2 * i], y[2 * i + 1]);
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

// V consecutive raw elements of one row of a u/delta/z tile in LDS, widened
// to fp32.  WIDE tiles pack ES-byte elements; the others hold one element per
// 4-byte slot (a bf16 element in its low half).
template <typename TIn, int V, bool WIDE>
struct RawRow {
    static constexpr bool kHalf = sizeof(TIn) == 2;
    static constexpr int NW = (WIDE && kHalf) ? V / 2 : V;
    uint32_t w[NW];
    __device__ __forceinline__ void read(const char* tile, int row, int col) {
        constexpr int XES = WIDE ? int(sizeof(TIn)) : 4;
        const char* src = tile + (row * 64 + col) * XES;
        if constexpr (NW == 1) {
            w[0] = *reinterpret_cast<const uint32_t*>(src);
        } else if constexpr (NW == 2) {
            const uint2 v = *reinterpret_cast<const uint2*>(src);
            w[0] = v.x;
            w[1] = v.y;
        } else {
#pragma unroll
            for (int c = 0; c < NW / 4; c++) {
                const uint4 v = reinterpret_cast<const uint4*>(src)[c];
                w[4 * c] = v.x;
                w[4 * c + 1] = v.y;
                w[4 * c + 2] = v.z;
                w[4 * c + 3] = v.w;
            }
        }
    }
    // The same V elements from a row in global memory at `src`: one vector
    // load when WIDE (src aligned to V elements), else element loads, of
    // which those past `valid` read element 0 again.
    __device__ __forceinline__ void load(const TIn* src, int valid) {
        if constexpr (WIDE) {
            const char* c = reinterpret_cast<const char*>(src);
            if constexpr (NW == 1) {
                w[0] = *reinterpret_cast<const uint32_t*>(c);
            } else if constexpr (NW == 2) {
                const uint2 v = *reinterpret_cast<const uint2*>(c);
                w[0] = v.x;
                w[1] = v.y;
            } else {
#pragma unroll
                for (int q = 0; q < NW / 4; q++) {
                    const uint4 v = reinterpret_cast<const uint4*>(c)[q];
                    w[4 * q] = v.x;
                    w[4 * q + 1] = v.y;
                    w[4 * q + 2] = v.z;
                    w[4 * q + 3] = v.w;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; i++) {
                const int e = i < valid ? i : 0;
                if constexpr (kHalf) w[i] = reinterpret_cast<const uint16_t*>(src)[e];
                else w[i] = __float_as_uint(reinterpret_cast<const float*>(src)[e]);
            }
        }
    }
    __device__ __forceinline__ float f(int i) const {
        if constexpr (!kHalf) return __uint_as_float(w[i]);
        else if constexpr (!WIDE) return __uint_as_float(w[i] << 16);
        else return (i & 1) ? __uint_as_float(w[i / 2] & 0xffff0000u) : __uint_as_float(w[i / 2] << 16);
    }
};

// scan_seq: WIDE = d_in * sizeof(TIn) is a multiple of 16 and u, delta, z
// and y are aligned for 16-byte accesses, so u/delta/z tiles arrive by
// 16-byte direct-to-LDS loads and y leaves by wide stores.
// SP: delta' = softplus(delta + bias) (else delta + bias).  GATE: z is given.
// ZOH: the input term is the zero-order hold's (exp(delta' A) - 1) / A B u
// (else delta' B u).  CROSS: cross scan -- batch row bi is direction bi % 4
// (0 row-major, 1 column-major, 2 and 3 those backwards) of map bi / 4; u is
// the (maps, H, W, d_in) map, A_log, D and the bias hold one set per
// direction, and y is fp32 (b, L, d_in), each direction in its own step order.
// DZ (with GATE): the pass inside the backward -- instead of y it writes the
// gradient of the gate input, dz = dy y_pre silu'(z), y_pre = sum C h + D u
// (dy read by the element waves one chunk ahead of its use).
//
// Waves 0 .. SC-1 ("recurrence waves") each hold NSW states of the 64
// channels and run nothing but the recurrence.  Waves SC .. SC+3 ("element
// waves") do the per-element work: step size and delta' u, the sum of the SC
// partial readouts, the D skip, the gate, and the stores of y.  The last wave
// (the "loader") streams u, delta, z, B and C into LDS with direct-to-LDS
// loads and waits for them with explicit counts, so no wave ever holds data
// that is still on its way from memory and no barrier waits for global
// memory.  Each SIMD gets the same mix of recurrence and element waves.
//
// Software pipeline, one barrier per chunk c of T steps.  Between two barriers
//   - every recurrence wave runs chunk c from registers: the (delta', delta' u)
//     pairs and B, C values of each step are read from LDS a few steps ahead
//     (near the end of the chunk these reads run into chunk c+1, whose LDS data
//     was written two chunks earlier), and its partial readout of each step
//     goes to LDS as soon as it is known;
//   - the element waves finish chunk c-1 and prepare chunk c+2 from its raw
//     tiles (loaded two chunks earlier);
//   - the loader issues the loads of chunk c+4 (u, delta, B, C) and of chunk
//     c+1 (z), then waits until those of chunk c+3 and c are complete.
template <typename TIn, int SC, int NSW, int T, bool WIDE, bool SP, bool GATE, bool ZOH, bool CROSS, bool DZ = false>
__global__ __launch_bounds__((SC + kSeqElemWaves + 1) * 64) void scan_seq(const ScanParams p) {
    constexpr int P = kSeqElemWaves;
    constexpr int ES = int(sizeof(TIn));
    using TOut = std::conditional_t<CROSS, float, TIn>;   // element type of y
    constexpr int NE = P * 64;                     // element threads
    constexpr int V = T / P;                       // consecutive channels per element thread
    constexpr int TPR = 64 / V;                    // element threads per step row
    constexpr int NP = SC * NSW;                   // states per channel, padded
    using Lds = SeqLds<T, SC, NP, ES, WIDE>;
    constexpr int EBC = (T * NP + NE - 1) / NE;    // B (and C) values each element thread stages per chunk
    constexpr int PA = kSeqAhead / 2;              // step pairs of (delta', delta' u) read ahead
    constexpr int RDW = 4;                         // register ring of step pairs (divides T / 2)
    constexpr int NR = NSW / 2;                    // float4 per step: NSW values of B then NSW of C
    constexpr int RBC = NR >= 2 ? 2 : 4;           // register ring of B, C steps (divides T)
    constexpr int LB = RBC - 1;                    // steps of B, C read ahead
    // Loads the loader issues per chunk: u and delta, B and C, z.
    constexpr int XI = WIDE ? T * 64 * ES / 1024 : T;          // per u, delta or z tile
    constexpr int BI = (T * NP + 63) / 64;                     // per B or C block
    constexpr int N_UDBC = 2 * XI + 2 * BI, N_Z = GATE ? XI : 0;
    static_assert(T % P == 0 && 64 % V == 0 && NE / TPR == T, "thread tiling of a chunk");
    static_assert(NSW % 2 == 0 && (T / 2) % RDW == 0 && T % RBC == 0 && PA + 1 <= RDW, "tiles split evenly");
    static_assert(!WIDE || (T * 64 * ES) % 1024 == 0, "whole loads per tile");
    static_assert(Lds::bytes <= 160 * 1024, "LDS of one workgroup");
    static_assert(T % kCkptSteps == 0, "checkpoints fall at chunk-internal step boundaries");
    static_assert(!DZ || (GATE && !CROSS), "dz is the gradient of a gated scan");
    extern __shared__ __align__(16) float smem[];
    char* const lds = reinterpret_cast<char*>(smem);
    const lds_ptr lds3 = dynamic_lds_base();       // the same block as an LDS-space pointer (direct-to-LDS loads)
    float* s_dw = reinterpret_cast<float*>(lds + Lds::off_dw);   // [3][T/2][64][4]: (delta'_j, w_j, delta'_j+1, w_j+1)
    // Channel c of a (delta', delta' u) row sits in 16-byte slot dw_slot(c): an
    // element thread writes its V consecutive channels at a 16*V-byte stride
    // from its neighbours, which without the swizzle would put 16 lanes of a
    // row on 4 bank groups.
    auto dw_slot = [](int c) { return c ^ ((c >> 4) & 3); };
    float* s_yp = reinterpret_cast<float*>(lds + Lds::off_yp);   // [2][SC][T][64]
    float* s_bc = reinterpret_cast<float*>(lds + Lds::off_bc);   // [3][T][SC][2][NSW]
    int& s_ticket = *reinterpret_cast<int*>(lds + Lds::off_ticket);
    constexpr int DW_BUF = Lds::DW / 4, YP_BUF = Lds::YP / 4, BC_BUF = Lds::BC / 4;   // floats

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool rec = wave < SC;                    // uniform per wave
    const bool loader = wave == SC + P;
    // The host keeps L < 2^31, d_in < 2^24, n <= 64 and G * K < 2^22, so every
    // per-segment index below fits 32 bits; element offsets of whole rows are
    // formed in 64 bits.
    const int L = int(p.L), d_in = int(p.d_in), n = int(p.n);
    const int G = int(p.b) * p.nblk_d;

    int ticket;
    if (p.K == 1) {
        ticket = blockIdx.x;
        // Without segments nothing waits, so nothing can set the status word
        // while it is cleared here (with segments scan_ctl_reset clears it).
        if (blockIdx.x == 0 && tid < 2 && p.err) p.err[tid] = 0u;
    } else {
        if (tid == 0) s_ticket = int(atomicAdd(p.ctl, 1u));
        __syncthreads();
        ticket = s_ticket;
    }
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    int seg = 0, g = ticket;
    while (g >= G) {                               // at most 16 rounds, uniform
        g -= G;
        seg++;
    }
    const int bi = __builtin_amdgcn_readfirstlane(g / p.nblk_d);
    const int dbase = __builtin_amdgcn_readfirstlane((g - bi * p.nblk_d) * 64);
    const int t_begin = seg * int(p.Lseg);
    const int t_end = min(L, t_begin + int(p.Lseg));
    const int nchunks = (t_end - t_begin + T - 1) / T;
    const int nch3 = (nchunks + 2) / 3 * 3;       // chunks the loop runs (past the end: empty)

    // Cross scan: direction and map of this batch row, and the map position of
    // step t of that direction (the host keeps H * W < 2^31).
    const int dir = CROSS ? bi % 4 : 0;
    const int64_t mrow = CROSS ? int64_t(bi / 4) * L : 0;
    auto cross_pos = [&](int t) -> int {
        const int s = dir >= 2 ? L - 1 - t : t;
        if (!(dir & 1)) return s;
        const uint32_t w = uint32_t(s) / uint32_t(p.cross_h);
        const int h = s - int(w) * p.cross_h;
        return h * p.cross_w + int(w);
    };
    const int64_t prow = int64_t(dir) * d_in;     // this direction's row of A_log, D, bias

    // Recurrence waves: lane = channel d, states n0 .. n0+NSW.
    const int d = dbase + lane;
    const bool dv = d < d_in;
    const int n0 = wave * NSW;
    float A2[NSW], h[NSW];
    const float* h0 = (seg == 0 && p.h0) ? p.h0 + (int64_t(bi) * d_in + d) * n + n0 : nullptr;
#pragma unroll
    for (int q = 0; q < NSW; q++) {
        const bool ok = rec && dv && n0 + q < n;
        A2[q] = ok ? a2_from_alog(p.A_log[(prow + d) * n + n0 + q]) : 0.0f;
        h[q] = (ok && h0) ? h0[q] : 0.0f;
    }

    // Element waves: thread owns step row er of a chunk, channels ec .. ec+V.
    const bool elem = !rec && !loader;
    const int etid = elem ? tid - SC * 64 : 0;
    const int er = etid / TPR;
    const int ec = (etid - er * TPR) * V;
    const int ech = dbase + ec;
    const int evalid = elem ? max(0, min(V, d_in - ech)) : 0;
    const bool whole_span = evalid == V;           // all V channels of this thread exist
    const uint32_t off_el = uint32_t(er) * uint32_t(d_in) + uint32_t(evalid > 0 ? ech : 0);
    float Dv[V], bias_v[V];
#pragma unroll
    for (int i = 0; i < V; i++) {
        Dv[i] = i < evalid ? p.D[prow + ech + i] : 0.0f;
        bias_v[i] = (i < evalid && p.bias) ? p.bias[prow + ech + i] : 0.0f;
    }

    if (seg > 0) {
        // Wait for the previous segment of this channel group, then take its
        // state.  The wait cannot deadlock (the predecessor holds an earlier
        // ticket); should it still time out, the status word is set and this
        // piece continues from a NaN state, so its outputs show it.
        int& s_timeout = *(reinterpret_cast<int*>(lds + Lds::off_ticket) + 1);
        if (tid == 0) {
            const uint32_t* flag = p.wait_never ? p.err + 1 : p.ctl + kFlagOffset + (seg - 1) * G + g;
            s_timeout = wait_segment_flag(flag, p.err, p.spin_limit) ? 1 : 0;
        }
        __syncthreads();
        const bool timed_out = __builtin_amdgcn_readfirstlane(s_timeout) != 0;
        if (rec) {
            const uint32_t* src = reinterpret_cast<const uint32_t*>(p.handoff) + (int64_t(seg - 1) * G + g) * n * 64;
#pragma unroll
            for (int q = 0; q < NSW; q++)
                if (n0 + q < n)
                    h[q] = timed_out ? __builtin_nanf("")
                                     : __uint_as_float(__hip_atomic_load(src + (n0 + q) * 64 + lane,
                                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
    }

    // Chunk k covers steps t_begin + k*T .. of this segment; rows(k) of them
    // exist (0 for chunks past the end, whose values are masked to zero: a
    // zero step size leaves the state unchanged).
    const int64_t brow = int64_t(bi) * L;         // (b, t = 0) row of this batch
    auto rows = [&](int k) -> int { return max(0, min(T, t_end - t_begin - k * T)); };
    auto ev = [&](int k) -> int { return er < rows(k) ? evalid : 0; };   // valid channels of this thread's row

    // ---- loader: direct-to-LDS loads of chunk k (rows past the segment's end
    // read its last row, channels past d_in read channel dbase; both are masked).
    // `mapped`: rows of the cross scan's map (u), else rows of this batch row.
    auto xrow = [&](bool mapped, int t) -> int64_t { return CROSS && mapped ? mrow + cross_pos(t) : brow + t; };
    auto dma_x = [&](const TIn* src, lds_ptr tile, int k, bool mapped) {
        const int t0 = t_begin + k * T;
        if constexpr (WIDE) {
            constexpr int EPL = 16 / ES;           // elements per lane
            constexpr int LPR = 64 / EPL;          // lanes per row
            constexpr int RPI = 64 / LPR;          // rows per load
            const int q = lane % LPR;
            const int ch = dbase + q * EPL < d_in ? dbase + q * EPL : dbase;
#pragma unroll
            for (int ii = 0; ii < XI; ii++) {
                const int t = min(t0 + ii * RPI + lane / LPR, t_end - 1);
                load_to_lds<16>(src + (xrow(mapped, t) * d_in + ch), tile + ii * 1024);
            }
        } else {
            const int ch = min(dbase + lane, d_in - 1);
#pragma unroll 2
            for (int r = 0; r < T; r++) {
                const int t = min(t0 + r, t_end - 1);
                load_to_lds<ES>(src + (xrow(mapped, t) * d_in + ch), tile + r * 256);
            }
        }
    };
    auto dma_bc = [&](const TIn* src, lds_ptr block, int k) {
        const int t0 = min(t_begin + k * T, t_end - 1);
        // Last element of the chunk's valid rows (at most T of them: the rows
        // left in a long segment times n would overflow 32 bits).
        const int last = min(T, t_end - t0) * n - 1;
        const TIn* base = src + (brow + t0) * n;
#pragma unroll
        for (int ii = 0; ii < BI; ii++)
            load_to_lds<ES>(base + min(ii * 64 + lane, last), block + ii * 256);
    };
    // Whole chunks (all T rows inside the segment, and the B/C block within
    // the segment's rows) are loaded through buffer descriptors based at the
    // chunk's first row: per-lane byte offsets fixed at the start, per-load
    // offsets in scalar registers, so the loader issues no vector
    // instruction for them.  Each descriptor covers exactly the bytes its
    // loads read.  The other chunks take the clamped loads above.
    // The forms for whole chunks below (loads, the step-size phase, the B/C
    // staging) are taken by the Euler forward only: in the zero-order-hold
    // and dz forms, whose recurrence waves already fill the register file,
    // they made one fp32 build (8 x 4 states, zero-order hold, dz) compute a
    // wrong dz, though the same source run on the host is correct.  Nor by
    // the 8 x 8 shape (n above 32), which spills registers with them: its
    // gated bf16 form faulted the GPU in the one run it had (its cause not
    // found; the same source runs clean on the host).
    constexpr bool kWholeForms = !ZOH && !DZ && !CROSS && SC * NSW <= 32;
    constexpr bool kFastLoads = WIDE && kWholeForms;
    constexpr int XEPL = 16 / ES, XLPR = 64 / XEPL, XRPI = 64 / XLPR;   // elements, lanes, rows per 16-byte load
    uint32_t vo_x = 0;
    if constexpr (kFastLoads) {
        const int q = lane % XLPR;
        vo_x = uint32_t(lane / XLPR) * uint32_t(d_in) * ES + uint32_t(dbase + q * XEPL < d_in ? q * XEPL : 0) * ES;
    }
    auto whole_chunk = [&](int k) -> bool {
        const int t0 = t_begin + k * T;
        return t0 + T <= t_end && BI * 64 <= (t_end - t0) * n;
    };
    auto fast_x = [&](const TIn* src, lds_ptr tile, int k) {
        const int64_t row0 = brow + t_begin + int64_t(k) * T;
        const auto rs = buffer_rsrc(src + row0 * d_in + dbase, uint32_t(T) * uint32_t(d_in) * ES);
#pragma unroll
        for (int ii = 0; ii < XI; ii++)
            buffer_load_to_lds<16>(rs, tile + ii * 1024, vo_x, uint32_t(ii * XRPI) * uint32_t(d_in) * ES);
    };
    auto fast_bc = [&](const TIn* src, lds_ptr block, int k) {
        const int64_t row0 = brow + t_begin + int64_t(k) * T;
        const auto rs = buffer_rsrc(src + row0 * n, uint32_t(BI * 64 * ES));
#pragma unroll
        for (int ii = 0; ii < BI; ii++)
            buffer_load_to_lds<ES>(rs, block + ii * 256, uint32_t(lane * ES), uint32_t(ii * 64 * ES));
    };
    auto dma_chunk = [&](int k, int slot) {        // u, delta, B, C of chunk k into ring slot `slot`
        // (LDS offsets formed here: hoisted, the 3 ring slots' dozen
        // destination addresses would not fit the scalar registers.)
        const lds_ptr ru = lds3 + opaque_scalar(Lds::off_ru + slot * 2 * Lds::RX);
        const lds_ptr rbc = lds3 + opaque_scalar(Lds::off_rbc + slot * 2 * Lds::RBC);
        if (kFastLoads && whole_chunk(k)) {
            fast_x(static_cast<const TIn*>(p.u), ru, k);
            fast_x(static_cast<const TIn*>(p.delta), ru + Lds::RX, k);
            fast_bc(static_cast<const TIn*>(p.B), rbc, k);
            fast_bc(static_cast<const TIn*>(p.C), rbc + Lds::RBC, k);
        } else {
            dma_x(static_cast<const TIn*>(p.u), ru, k, true);
            dma_x(static_cast<const TIn*>(p.delta), ru + Lds::RX, k, false);
            dma_bc(static_cast<const TIn*>(p.B), rbc, k);
            dma_bc(static_cast<const TIn*>(p.C), rbc + Lds::RBC, k);
        }
    };
    auto dma_z = [&](int k, int slot) {
        if (!GATE) return;
        const lds_ptr tile = lds3 + opaque_scalar(Lds::off_rz + slot * Lds::RX);
        if (kFastLoads && whole_chunk(k)) fast_x(static_cast<const TIn*>(p.z), tile, k);
        else dma_x(static_cast<const TIn*>(p.z), tile, k, false);
    };

    // ---- element waves
    using Row = RawRow<TIn, V, WIDE>;
    // Phase 1 of chunk k (ring slot `slot` = k % 3): (delta', delta' u) into LDS,
    // or (delta', u) with the zero-order hold; u kept for the D skip.
    auto phase1 = [&](int k, int slot, float* uv) {
        const char* ru = lds + Lds::off_ru + slot * 2 * Lds::RX;
        Row su, sd;
        su.read(ru, er, ec);
        sd.read(ru + Lds::RX, er, ec);
        float* buf = s_dw + slot * DW_BUF;
        // A whole row (for the Euler forward: of a whole chunk) has nothing to mask.
        if (kWholeForms ? rows(k) == T && whole_span : ev(k) == V) {
#pragma unroll
            for (int i = 0; i < V; i++) {
                const float x = sd.f(i) + bias_v[i];
                const float dl = SP ? softplus(x) : x;
                uv[i] = su.f(i);
                *reinterpret_cast<float2*>(buf + ((er >> 1) * 64 + dw_slot(ec + i)) * 4 + (er & 1) * 2) =
                    make_float2(dl, ZOH ? uv[i] : dl * uv[i]);
            }
        } else {
            const int valid = ev(k);
#pragma unroll
            for (int i = 0; i < V; i++) {
                const bool ok = i < valid;
                const float x = sd.f(i) + bias_v[i];
                const float dl = ok ? (SP ? softplus(x) : x) : 0.0f;
                uv[i] = ok ? su.f(i) : 0.0f;
                *reinterpret_cast<float2*>(buf + ((er >> 1) * 64 + dw_slot(ec + i)) * 4 + (er & 1) * 2) =
                    make_float2(dl, ZOH ? uv[i] : dl * uv[i]);
            }
        }
    };

    // B and C of chunk k (ring slot `slot` = k % 3) as fp32, zero for missing rows and states.
    auto stage_bc = [&](int k, int slot) {
        const uint32_t* rb = reinterpret_cast<const uint32_t*>(lds + Lds::off_rbc + slot * 2 * Lds::RBC);
        const uint32_t* rcc = rb + Lds::RBC / 4;
        float* buf = s_bc + slot * BC_BUF;
        const int r = rows(k);
        auto widen = [](uint32_t w) { return ES == 2 ? __uint_as_float(w << 16) : __uint_as_float(w); };
        // Every row and state exists: no masks.  (Not in the 8-state-per-wave
        // shape, where this form makes the compiler emit an invalid compare.)
        if (kWholeForms && NSW <= 4 && r == T && n == NP) {
#pragma unroll
            for (int m = 0; m < EBC; m++) {
                const int f = m * NE + etid;
                if ((T * NP) % NE != 0 && f >= T * NP) break;
                const int j = f / NP, kk = f % NP;
                float* dst = buf + ((j * SC + kk / NSW) * 2) * NSW + kk % NSW;
                dst[0] = widen(rb[f]);
                dst[NSW] = widen(rcc[f]);
            }
            return;
        }
#pragma unroll
        for (int m = 0; m < EBC; m++) {
            const int f = m * NE + etid;
            if ((T * NP) % NE != 0 && f >= T * NP) break;
            const int j = f / NP, kk = f % NP;
            const bool ok = j < r && kk < n;
            const int e = ok ? j * n + kk : 0;
            float bv = ES == 2 ? __uint_as_float(rb[e] << 16) : __uint_as_float(rb[e]);
            float cv = ES == 2 ? __uint_as_float(rcc[e] << 16) : __uint_as_float(rcc[e]);
            float* dst = buf + ((j * SC + kk / NSW) * 2) * NSW + kk % NSW;
            dst[0] = ok ? bv : 0.0f;
            dst[NSW] = ok ? cv : 0.0f;
        }
    };
    // dy of chunk k (DZ): this thread's V channels of its step row, issued one
    // chunk before phase 2 uses them (rows past the segment read its last row).
    auto load_dy = [&](int k, Row& r) {
        const int t = min(t_begin + k * T + er, t_end - 1);
        const int valid = max(evalid, 1);
        r.load(static_cast<const TIn*>(p.dy) + (brow + t) * d_in + (evalid > 0 ? ech : dbase), valid);
    };
    // Phase 2 of chunk k: sum of the partial readouts, D skip, gate (z slot `zslot`), store
    // (DZ: dz from that sum, z and dy row `dyk`).
    auto phase2 = [&](int k, const float* uvk, int zslot, const Row& dyk) {
        float ypv[SC][V];
        const float* src = s_yp + (k & 1) * YP_BUF + er * 64 + ec;
#pragma unroll
        for (int w = 0; w < SC; w++)
#pragma unroll
            for (int i = 0; i < V; i++) ypv[w][i] = src[w * T * 64 + i];
        Row zr;
        if (GATE) zr.read(lds + Lds::off_rz + zslot * Lds::RX, er, ec);
        float yv[V], ypre[V];
#pragma unroll
        for (int i = 0; i < V; i++) {
            float acc = ypv[0][i];
#pragma unroll
            for (int w = 1; w < SC; w++) acc += ypv[w][i];
            acc = fmaf(Dv[i], uvk[i], acc);
            ypre[i] = acc;
            if constexpr (DZ) {
                const float z = zr.f(i);
                const float sg = rcp_hw(1.0f + exp2_hw(-z * kLog2e));
                acc = dyk.f(i) * acc * sg * fmaf(z, 1.0f - sg, 1.0f);
            } else if (GATE) {
                acc *= silu(zr.f(i));
            }
            yv[i] = acc;
        }
        const int valid = ev(k);
        TOut* yp = static_cast<TOut*>(DZ ? p.dz : p.y);
        if (valid > 0 && yp)
            store_span<TOut, V, WIDE>(yp + (brow + t_begin + int64_t(k) * T) * d_in, off_el, yv, valid);
        if constexpr (GATE && !DZ && !CROSS) {
            // The readout before the gate, for a backward pass that starts from saved states.
            if (valid > 0 && p.ypre)
                store_span<TOut, V, WIDE>(static_cast<TOut*>(p.ypre) + (brow + t_begin + int64_t(k) * T) * d_in,
                                          off_el, ypre, valid);
        }
    };

    // ---- fill: loads of chunks 0 .. 2 and the gate of chunk 0; phase 1 and
    // B/C of chunks 0 and 1.
    float uvm1[V], uv0[V], uv1[V], uv2[V];
    Row dyr[3];                                   // DZ: dy of chunk c in dyr[c % 3]
    if (loader) {
        dma_chunk(0, 0);
        dma_chunk(1, 1);
        dma_chunk(2, 2);
        dma_z(0, 0);
        wait_vmem<N_UDBC + N_Z>();   // chunks 0 and 1 are in LDS
        __builtin_amdgcn_s_barrier();
        wait_vmem<N_Z>();            // and chunk 2
        __builtin_amdgcn_s_barrier();
    } else {
        barrier_lds();
        if (elem) {
            phase1(0, 0, uv0);
            stage_bc(0, 0);
            phase1(1, 1, uv1);
            stage_bc(1, 1);
#pragma unroll
            for (int i = 0; i < V; i++) uvm1[i] = 0.0f;
        }
        barrier_lds();
    }

    // Recurrence-wave LDS read-ahead: step pairs and B/C steps.
    float4 dwq[RDW];
    float4 bcq[RBC][NR];
    if (rec) {
#pragma unroll
        for (int pr = 0; pr < PA; pr++) dwq[pr % RDW] = reinterpret_cast<const float4*>(s_dw)[pr * 64 + dw_slot(lane)];
#pragma unroll
        for (int j = 0; j < LB; j++) {
            const float4* r = reinterpret_cast<const float4*>(s_bc + (j * SC + wave) * 2 * NSW);
#pragma unroll
            for (int qq = 0; qq < NR; qq++) bcq[j % RBC][qq] = r[qq];
        }
    }

    // One chunk c of each kind of wave, with c % 3 == PH (ring slots are
    // compile-time constants).  Each kind runs its own loop: the three never
    // share control flow inside the loop, so the compiler's wait analysis of
    // one (the loader's loads in flight) does not spill into the others.
    // ZOH: the input weight is the zero-order hold's (invA[q] = 1 / A).
    float invA[NSW];
#pragma unroll
    for (int q = 0; q < NSW; q++)
        invA[q] = (ZOH && rec && dv && n0 + q < n) ? inv_a_from_alog(p.A_log[(prow + d) * n + n0 + q]) : 0.0f;
    // Checkpoints for the backward pass.  Checkpoint i holds the state after
    // step kCkptSteps (i + 1); t_begin and T are multiples of kCkptSteps, so
    // they fall at fixed steps of every chunk, and the offset of the next one
    // is kept as a running (wave-uniform) count rather than formed from the
    // step index at every store.  A checkpoint is written only for steps of
    // this segment (past its end the state is not its own) and not after the
    // last step.
    float* const ck_lane = p.ckpt ? p.ckpt + int64_t(n0) * d_in + dbase + lane : nullptr;
    const int64_t ck_stride = int64_t(n) * d_in;   // floats between consecutive checkpoints
    int64_t ck_off = (int64_t(bi) * p.nck + t_begin / kCkptSteps - 1) * ck_stride;   // before the segment's first
    const int ck_last = min(t_end, L - 1);         // checkpoints after steps s <= ck_last are kept
    auto rec_chunk = [&](auto ph, int c) {
        constexpr int PH = decltype(ph)::value;
        constexpr int K0 = PH, K1 = (PH + 1) % 3;    // ring slots of chunks c, c+1
        float* ypw = s_yp + (c & 1) * YP_BUF + wave * T * 64 + lane;
        const float* dw_c = s_dw + K0 * DW_BUF;
        const float* dw_n = s_dw + K1 * DW_BUF;
        const float* bc_c = s_bc + K0 * BC_BUF + wave * 2 * NSW;
        const float* bc_n = s_bc + K1 * BC_BUF + wave * 2 * NSW;
        float ylast = 0.0f;
#pragma unroll
        for (int j = 0; j < T; j++) {
            if (j % 2 == 0) {
                const int pr = j / 2 + PA;       // read ahead, into chunk c+1 near the end
                const float* src = pr < T / 2 ? dw_c : dw_n;
                dwq[pr % RDW] = reinterpret_cast<const float4*>(src)[(pr % (T / 2)) * 64 + dw_slot(lane)];
            }
            {
                const int jb = j + LB;
                const float4* r = reinterpret_cast<const float4*>((jb < T ? bc_c : bc_n) + (jb % T) * SC * 2 * NSW);
#pragma unroll
                for (int qq = 0; qq < NR; qq++) bcq[jb % RBC][qq] = r[qq];
            }
            const float4 dq = dwq[(j / 2) % RDW];
            const float dl = (j & 1) ? dq.z : dq.x;
            const float wv = (j & 1) ? dq.w : dq.y;
            float bcv[2 * NSW];
#pragma unroll
            for (int qq = 0; qq < NR; qq++) {
                bcv[4 * qq] = bcq[j % RBC][qq].x;
                bcv[4 * qq + 1] = bcq[j % RBC][qq].y;
                bcv[4 * qq + 2] = bcq[j % RBC][qq].z;
                bcv[4 * qq + 3] = bcq[j % RBC][qq].w;
            }
            float acc = 0.0f;
#pragma unroll
            for (int q = 0; q < NSW; q++) {
                const float x2 = dl * A2[q];
                const float a = exp2_hw(x2);
                if constexpr (ZOH)
                    h[q] = fmaf(a, h[q], zoh_weight(dl, x2, a, invA[q]) * (wv * bcv[q]));
                else
                    h[q] = fmaf(a, h[q], wv * bcv[q]);
                acc = fmaf(bcv[NSW + q], h[q], acc);
            }
            if (j & 1) {
                ypw[(j - 1) * 64] = ylast;
                ypw[j * 64] = acc;
            } else {
                ylast = acc;
            }
            if (j % kCkptSteps == kCkptSteps - 1 && ck_lane) {
                ck_off += ck_stride;                       // the checkpoint after step t_begin + c T + j + 1
                if (t_begin + c * T + j + 1 <= ck_last && dv) {
                    float* dst = ck_lane + ck_off;
#pragma unroll
                    for (int q = 0; q < NSW; q++)
                        if (n0 + q < n) dst[int64_t(q) * d_in] = h[q];
                }
            }
        }
        barrier_lds();
    };
    auto elem_chunk = [&](auto ph, int c) {
        constexpr int PH = decltype(ph)::value;
        constexpr int K2 = (PH + 2) % 3;         // ring slot of chunks c+2 and c-1
        if (DZ) load_dy(c, dyr[PH]);
        if (c > 0) phase2(c - 1, uvm1, K2, dyr[K2]);
        phase1(c + 2, K2, uv2);
        stage_bc(c + 2, K2);
#pragma unroll
        for (int i = 0; i < V; i++) {
            uvm1[i] = uv0[i];
            uv0[i] = uv1[i];
            uv1[i] = uv2[i];
        }
        barrier_lds();
    };
    auto load_chunk = [&](auto ph, int c) {
        constexpr int PH = decltype(ph)::value;
        constexpr int K1 = (PH + 1) % 3;         // ring slot of chunks c+1 and c+4
        if (c == 0) dma_chunk(3, 0);
        dma_chunk(c + 4, K1);
        dma_z(c + 1, K1);
        wait_vmem<N_UDBC + N_Z>();   // chunk c+3 and z of chunk c are in LDS
        __builtin_amdgcn_s_barrier();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (rec) {
        for (int c = 0; c < nch3; c += 3) {
            rec_chunk(I0{}, c);
            rec_chunk(I1{}, c + 1);
            rec_chunk(I2{}, c + 2);
        }
    } else if (elem) {
        for (int c = 0; c < nch3; c += 3) {
            elem_chunk(I0{}, c);
            elem_chunk(I1{}, c + 1);
            elem_chunk(I2{}, c + 2);
        }
    } else {
        for (int c = 0; c < nch3; c += 3) {
            load_chunk(I0{}, c);
            load_chunk(I1{}, c + 1);
            load_chunk(I2{}, c + 2);
        }
    }

    if (elem) {
        phase2(nch3 - 1, uvm1, 2, dyr[2]);        // drain: the last chunk's outputs (nch3 - 1 = 2 mod 3)
    } else if (loader) {
        wait_vmem<0>();   // no load may land after the workgroup ends
    } else if (seg + 1 < p.K) {
        // Publish the state for the next segment.
        uint32_t* dst = reinterpret_cast<uint32_t*>(p.handoff) + (int64_t(seg) * G + g) * n * 64;
#pragma unroll
        for (int q = 0; q < NSW; q++)
            if (n0 + q < n)
                __hip_atomic_store(dst + (n0 + q) * 64 + lane, __float_as_uint(h[q]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    } else if (p.last_state && dv) {
#pragma unroll
        for (int q = 0; q < NSW; q++)
            if (n0 + q < n) p.last_state[(int64_t(bi) * d_in + d) * n + n0 + q] = h[q];
    }
    if (seg + 1 < p.K) {
        // The handed-off state and the flag are device-coherent atomic
        // accesses, ordered by the hardware: every wave waits until its state
        // stores are acknowledged, the workgroup meets, then one thread sets
        // the flag; the next segment reads the state only after it has seen
        // the flag.  Release/acquire fences at device scope would write back
        // and invalidate the whole L2 of the compute die at every segment
        // boundary, which costs far more than this exchange.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(p.ctl + kFlagOffset + seg * G + g, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// CrossMerge: y[m, p, :] = sum over the four directions k of ys[m, k, t_k(p), :],
// t_k(p) the step at which direction k visits map position p (the inverse of
// the cross scan's traversal), added in the order k = 0, 1, 2, 3.  One thread
// per VEC consecutive channels of a position, grid-stride (the host caps the
// grid, so any size launches); every read and the write are whole rows of
// d_in channels.
template <int VEC>
__global__ __launch_bounds__(256) void cross_merge(const float* __restrict__ ys, float* __restrict__ y, int64_t maps,
                                                   int H, int W, int64_t d_in) {
    const int64_t L = int64_t(H) * W;
    const int64_t cpr = d_in / VEC;                           // thread columns per row
    const int64_t total = maps * L * cpr;
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
        const int64_t row = i / cpr;                          // (m, p)
        const int64_t c = (i - row * cpr) * VEC;
        const int64_t m = row / L;
        const int64_t pos = row - m * L;
        const int64_t h = pos / W, w = pos - h * W;
        const int64_t tc = w * H + h;                         // step of the column-major direction
        const int64_t steps[4] = {pos, tc, L - 1 - pos, L - 1 - tc};
        float acc[VEC];
#pragma unroll
        for (int v = 0; v < VEC; v++) acc[v] = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float* src = ys + ((m * 4 + k) * L + steps[k]) * d_in + c;
            if constexpr (VEC == 4) {
                const float4 q = *reinterpret_cast<const float4*>(src);
                acc[0] += q.x;
                acc[1] += q.y;
                acc[2] += q.z;
                acc[3] += q.w;
            } else {
                acc[0] += src[0];
            }
        }
        float* dst = y + row * d_in + c;
        if constexpr (VEC == 4) *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        else dst[0] = acc[0];
    }
}

// Clears the ticket counter and the segment flags (ctl[0 .. words)) and, when
// err is given, the call's two status words.
static __global__ void scan_ctl_reset(uint32_t* ctl, int64_t words, uint32_t* err) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < words; i += int64_t(gridDim.x) * blockDim.x)
        ctl[i] = 0u;
    if (err && blockIdx.x == 0 && threadIdx.x < 2) err[threadIdx.x] = 0u;
}

// The status code a call left in its status word: SS_OK (0), or
// SS_ERR_TIMEOUT (-10) once a segment wait gave up.
static __global__ void scan_status_copy(const uint32_t* err, int32_t* status) {
    if (threadIdx.x == 0) *status = __hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ? -10 : 0;
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
