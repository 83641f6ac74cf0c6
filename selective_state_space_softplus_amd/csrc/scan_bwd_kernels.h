// scan_bwd_kernels.h -- gradient of the selective scan (Euler input term) on
// gfx950.  The pages only name the autograd wrappers around the scan; the
// formulas below are the chain rule applied to the forward recurrence
// (mhpn.cn selective_scan walk-through, sections 3-5 and 7; jiafeimiao.top
// Mamba.step for the bias and the gate).  Per (b, d) channel, with
// w_t = Delta_t u_t, a_tk = exp(Delta_t A_k), y'_t = sum_k C_tk h_tk + D u_t:
//     dy'_t    = dy_t silu(z_t)                   (dy_t without a gate)
//     g_tk     = dL/dh_tk = dy'_t C_tk + a_(t+1)k g_(t+1)k,   g_Lk = dlast_k
//     S1_t     = sum_k g_tk B_tk,   S2_t = sum_k g_tk A_k a_tk h_(t-1)k
//     du_t     = Delta_t S1_t + dy'_t D
//     dDelta_t = S2_t + u_t S1_t,   ddelta_t = dDelta_t sigmoid(delta_t + bias)  (softplus' = sigmoid)
//     dz_t     = dy_t y'_t silu'(z_t)
//     dB_tk    = sum_d g_tk w_t,    dC_tk = sum_d dy'_t h_tk
//     dA_log_k = sum_(b,t) g_tk Delta_t a_tk h_(t-1)k A_k,   dD = sum dy' u,   dbias = sum ddelta
//     dh0_k    = a_0k g_0k
//
// ZOH: the zero-order-hold input weight beta = (exp(Delta A) - 1)/A in place
// of Delta (mhpn.cn page, section 6): du_t = dy'_t D + sum_k g_tk beta_tk B_tk,
// dDelta_t gains a_tk where Euler has 1 in its input term, dB = g beta u, and
// dA_k gains g_tk B_tk u_t (Delta_t a_tk - beta_tk)/A_k.
//
// scan_bwd<TIn, SC, NSW, SL, SP, GATE, ZOH, PR>: one workgroup per (slice of NP =
// SC NSW states (SL: n is taken in several slices), b, 64-channel group,
// segment of L) walks its segment backwards in chunks of kCkptSteps = 8
// steps; segments are taken last first, each starting from the adjoint the
// later one handed on (as the forward hands on states), which balances the
// workgroups over the compute units.  The forward pass
// saved the state every 8 steps; the SC recurrence waves (NSW states of the
// 64 channels each) reload the state entering the chunk, run the chunk's 8
// steps forward again keeping every h and decay in registers, then run the
// adjoint back through them.  The 4 element waves load and prepare the next
// chunk (delta', delta' u, dy', the fp32 B and C rows, the entering state;
// their global loads are issued one chunk earlier still), and finish the
// previous one (sums of the waves' S1, S2 partials, du, ddelta, and the
// chunk's dB, dC rows).  PR: each element thread owns two adjacent channels
// (d_in even, tensors aligned), so a row's two elements move in one access.
// dz needs the readout y'_t and nothing else does: the forward pass that
// saves the states writes it (scan_seq with DZ), or, from saved states, the
// element waves form it from the saved pre-gate readout; the readout is
// never recomputed here.  Sums over the 64 channels (dB, dC) are
// cross-lane reductions inside each recurrence wave; sums over the channel groups,
// batch rows and time (dB, dC, dA_log, dD, dbias) go through per-workgroup
// partials that reduce_groups adds in a fixed order, so every gradient is
// the same bit for bit on every run.
#pragma once

#include <type_traits>

#include "scan_kernels.h"
#include "ss_device.h"

namespace ss {

struct BwdParams {
    const void* u;
    const void* delta;
    const float* A_log;
    const void* B;
    const void* C;
    const float* D;
    const void* z;
    const float* bias;
    const float* h0;          // (b, d_in, n) or null
    const void* dy;           // (b, L, d_in)
    const void* ypre;         // gated, from saved states: the forward's readout before the gate (b, L, d_in), else null
    void* dz;                 // with ypre: dz is written here
    const float* dlast;       // (b, d_in, n) or null
    const float* ckpt;        // (b, nck, n, d_in): state after steps 8 (i + 1)
    void* du;
    void* ddelta;
    float* dh0;               // null unless asked
    float* part_B;            // (nblk_d, b, L, n) dB per channel group
    float* part_C;            // (nblk_d, b, L, n)
    float* part_A;            // (K, b, d_in, n) dA_log per segment and batch row
    float* part_D;            // (K, b, d_in)
    float* part_bias;         // (K, slices, b, d_in)
    float* part_du;           // (slices, b, L, d_in) when slices > 1, else null
    float* part_dd;           // (slices, b, L, d_in) when slices > 1, else null
    int64_t b, L, d_in, n;
    int nck, nblk_d, softplus;
    // The states are taken in slices of SC NSW (the kernel's NP) by separate
    // workgroups; with more than one slice, du and ddelta are sums of the
    // slices' parts (part_du, part_dd), which reduce_groups adds.
    int slices;
    // L segments: pieces taken in ticket order, last segment first; a piece
    // starts from the adjoint its successor segment handed on.
    int K;
    int64_t Lseg;             // steps per segment, a multiple of kCkptSteps
    uint32_t* ctl;            // [0] ticket counter, [kFlagOffset + s G + g] flags
    float* handoff;           // (K - 1, G slices, NP, 64) adjoints handed between segments
    uint32_t* err;            // status words of the call (as ScanParams::err; cleared by the forward pass)
    int spin_limit;           // polls before a segment wait gives up
    int wait_never;           // nonzero: waits poll err[1] (never set) and give up after spin_limit polls
};

// Partial sums over the 64 lanes of the wave of four values at once (the
// first two steps of a transposing butterfly; every lane of the wave must be
// active):
//   1. v_permlane32_swap pairs the lower halves of (v0, v1) and of (v2, v3):
//      a = [v0_lo + v0_hi | v1_lo + v1_hi], b likewise for v2, v3;
//   2. v_permlane16_swap pairs odd rows of a with even rows of b.
// Rows 0, 1, 2, 3 of the result then hold 16 partial sums (over 4 lanes
// each) of v0, v2, v1, v3: 6 VALU instructions for the four values.
__device__ __forceinline__ float wave_part4(float v0, float v1, float v2, float v3) {
    const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v1), false, false);
    const auto y = __builtin_amdgcn_permlane32_swap(__float_as_uint(v2), __float_as_uint(v3), false, false);
    const float a = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const float b = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    const auto z = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(z[0]) + __uint_as_float(z[1]);
}

// LDS of scan_bwd<SC recurrence waves, NP padded states>, T = 8 steps.
// The recurrence waves leave the dB, dC sums over the 64 channels at 16
// partials per (step, state) -- a row of 16 floats -- and the element waves
// add them up.
//
// gfx950's LDS has 64 banks of 4 bytes; a 16-byte access serves 16 lanes a
// cycle, a 4-byte access all 64.  So: the per-(step, channel) values are
// kept as four planes of floats, not as float4s, since the recurrence waves
// read one or two of them at a time (a 4-byte read at a 16-byte lane stride
// meets each bank four times); and the partial rows are RS = 20 floats apart,
// so that the 16 rows that one 16-byte read of a row per lane touches in a
// cycle start on 16 different groups of 4 banks (20 g mod 64, g = 0 .. 15,
// are distinct multiples of 4).
template <int SC, int NP>
struct BwdLds {
    static constexpr int T = kCkptSteps;
    static_assert(NP <= 16, "states per workgroup (larger n is taken in slices)");
    static constexpr int RS = 20;                             // floats per partial row (16 used)
    static constexpr int ROWS = T * 2 * NP;                   // (step, state, B or C) rows of a chunk
    static constexpr int PLANE = 3 * T * 64 * 4;              // one of Delta, w, dy', u per (slot, step, channel)
    static constexpr int PREP = 4 * PLANE;                    // the four planes, three ring slots each
    static constexpr int PART = SC * T * 64 * 8;              // (S1, S2) per (wave, step, channel)
    static constexpr int CK = NP * 64 * 4;                    // state entering the chunk
    static constexpr int BC = T * 2 * NP * 4;                 // B, C rows as fp32, grouped per wave
    static constexpr int DBC = ROWS * RS * 4;                 // dB, dC partial rows of the chunk
    static constexpr int row_off(int g) { return g * RS; }
    static constexpr int off_prep = 0;                        // [4 planes][3 slots]
    static constexpr int off_part = off_prep + PREP;          // [2]
    static constexpr int off_ck = off_part + 2 * PART;        // [2]
    static constexpr int off_bc = off_ck + 2 * CK;            // [2]
    static constexpr int off_dbc = off_bc + 2 * BC;           // [2]
    static constexpr int off_ticket = off_dbc + 2 * DBC;      // ticket, timeout flag
    static constexpr int bytes = off_ticket + 16;
};

template <typename TIn, int SC, int NSW, bool SL, bool SP, bool GATE, bool ZOH, bool PR>
__global__ __launch_bounds__((SC + 4) * 64) void scan_bwd(const BwdParams p) {
    constexpr int T = kCkptSteps;
    constexpr int NE = 4 * 64;                     // element threads
    constexpr int V = T * 64 / NE;                 // consecutive channels per element thread
    constexpr int TPR = 64 / V;                    // element threads per step row
    constexpr int NP = SC * NSW;
    constexpr int EBC = (T * NP + NE - 1) / NE;    // B (and C) values each element thread stages per chunk
    constexpr int ECK = (NP * 64 + NE - 1) / NE;   // entering-state values each element thread stages
    using Lds = BwdLds<SC, NP>;
    static_assert(Lds::bytes <= 160 * 1024, "LDS of one workgroup");
    static_assert(NE / TPR == T, "thread tiling of a chunk");
    static_assert(NSW % 2 == 0, "states reduced two at a time");
    extern __shared__ __align__(16) float smem[];
    char* const lds = reinterpret_cast<char*>(smem);
    // (Delta, w, dy', u) of (slot, step, channel) at s_prep[plane * PL + (slot T + step) 64 + channel].
    float* s_prep = reinterpret_cast<float*>(lds + Lds::off_prep);
    constexpr int PL = Lds::PLANE / 4;
    float2* s_part = reinterpret_cast<float2*>(lds + Lds::off_part);   // [2][SC][T][64]
    float* s_ck = reinterpret_cast<float*>(lds + Lds::off_ck);         // [2][NP][64]
    float* s_bc = reinterpret_cast<float*>(lds + Lds::off_bc);         // [2][T][SC][2][NSW]
    float* s_dbc = reinterpret_cast<float*>(lds + Lds::off_dbc);       // [2][T][2][NP], or [2][ROWS][RS] rows
    constexpr int RS = Lds::RS, ROWS = Lds::ROWS;
    static_assert(ROWS % 4 == 0, "groups of 4 partial rows");
    constexpr int RPT = (ROWS + NE - 1) / NE;      // partial rows each element thread adds up per chunk

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool rec = wave < SC;
    const int L = int(p.L), d_in = int(p.d_in), n = int(p.n);
    const int G = int(p.b) * p.nblk_d * p.slices;   // (slice, batch row, channel group) triples
    int& s_ticket = *reinterpret_cast<int*>(lds + Lds::off_ticket);
    int ticket;
    if (p.K == 1) {
        ticket = blockIdx.x;
    } else {
        if (tid == 0) s_ticket = int(atomicAdd(p.ctl, 1u));
        __syncthreads();
        ticket = s_ticket;
    }
    ticket = __builtin_amdgcn_readfirstlane(ticket);
    int seg = p.K - 1, gi = ticket;                // later segments take the earlier tickets
    while (gi >= G) {                              // at most 16 rounds, uniform
        gi -= G;
        seg--;
    }
    const int slice = SL ? __builtin_amdgcn_readfirstlane(gi / (int(p.b) * p.nblk_d)) : 0;
    const int gb = gi - slice * int(p.b) * p.nblk_d;
    const int bi = __builtin_amdgcn_readfirstlane(gb / p.nblk_d);
    const int grp = __builtin_amdgcn_readfirstlane(gb - bi * p.nblk_d);
    const int k0 = slice * NP;                     // first state of the slice
    const int ns = min(NP, n - k0);                // states of the slice
    const int dbase = grp * 64;
    const int t_begin = seg * int(p.Lseg);
    const int t_end = min(L, t_begin + int(p.Lseg));
    const int kc0 = t_begin / T;                   // first and last chunk of this segment
    const int kcl = (t_end + T - 1) / T - 1;
    const int64_t brow = int64_t(bi) * L;

    // Recurrence waves: lane = channel d, states n0 .. n0 + NSW.
    const int d = dbase + lane;
    const bool dv = d < d_in;
    const int n0 = wave * NSW;
    float A2[NSW], An[NSW], g[NSW], dA[NSW], invA[NSW];
#pragma unroll
    for (int q = 0; q < NSW; q++) {
        const bool ok = rec && dv && n0 + q < ns;
        const int64_t kq = int64_t(d) * n + k0 + n0 + q;             // (d, state) in A_log
        A2[q] = ok ? a2_from_alog(p.A_log[kq]) : 0.0f;
        An[q] = A2[q] * kLn2;                                          // A itself
        invA[q] = (ZOH && ok) ? inv_a_from_alog(p.A_log[kq]) : 0.0f;
        g[q] = (ok && p.dlast && seg == p.K - 1) ? p.dlast[int64_t(bi) * d_in * n + kq] : 0.0f;
        dA[q] = 0.0f;
    }
    if (seg < p.K - 1) {
        // Wait for the adjoint of the later segment of these channels (it holds
        // an earlier ticket, so the wait cannot deadlock; on a timeout the status
        // word is set and this piece goes on from NaN, so its outputs show it).
        int& s_timeout = *(reinterpret_cast<int*>(lds + Lds::off_ticket) + 1);
        if (tid == 0) {
            const uint32_t* flag = p.wait_never ? p.err + 1 : p.ctl + kFlagOffset + seg * G + gi;
            s_timeout = wait_segment_flag(flag, p.err, p.spin_limit) ? 1 : 0;
        }
        __syncthreads();
        const bool timed_out = __builtin_amdgcn_readfirstlane(s_timeout) != 0;
        if (rec) {
            const uint32_t* src = reinterpret_cast<const uint32_t*>(p.handoff) + (int64_t(seg) * G + gi) * NP * 64;
#pragma unroll
            for (int q = 0; q < NSW; q++)
                if (n0 + q < ns)
                    g[q] = timed_out ? __builtin_nanf("")
                                     : __uint_as_float(__hip_atomic_load(src + (n0 + q) * 64 + lane,
                                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        }
    }

    // Element waves: thread owns step row er of a chunk and channels cofs(i)
    // (i < V) of the group: ec + i TPR, or with PR (d_in even, every
    // per-element tensor aligned to two elements) the adjacent pair 2 ec,
    // 2 ec + 1, whose two elements of a row are one 4-byte (bf16) or 8-byte
    // (fp32) load or store.  Either way consecutive lanes take consecutive
    // channels.
    static_assert(!PR || V == 2, "channel pairs");
    const int etid = rec ? 0 : tid - SC * 64;
    const int er = etid / TPR;
    const int ec = etid - er * TPR;
    auto cofs = [&](int i) __attribute__((always_inline)) { return PR ? 2 * ec + i : ec + i * TPR; };
    bool evok[V];
#pragma unroll
    for (int i = 0; i < V; i++) evok[i] = !rec && dbase + cofs(i) < d_in;
    float Dv[V], bias_v[V], accD[V], accBias[V];
#pragma unroll
    for (int i = 0; i < V; i++) {
        Dv[i] = evok[i] && slice == 0 ? p.D[dbase + cofs(i)] : 0.0f;   // the D term once
        bias_v[i] = (evok[i] && p.bias) ? p.bias[dbase + cofs(i)] : 0.0f;
        accD[i] = accBias[i] = 0.0f;
    }

    // Global words of one chunk as loaded by an element thread.  Every load is
    // issued unconditionally (an element outside the tensor reads a valid word
    // of the same array instead) and kept as loaded; masking and the bf16
    // widening happen when the chunk is prepared, one iteration later, so the
    // loads stay in flight across the recurrence waves' work on the current
    // chunk.  Addresses are a per-chunk base, uniform over the workgroup, plus
    // a 32-bit byte offset fixed per thread.
    using RawIn = Raw<TIn>;
    using Word = typename RawIn::type;
    constexpr int ES = int(sizeof(TIn));
    struct Chunk {
        Word u[V], dl[V], z[V], dy[V], yp[V];
        Word b[EBC], c[EBC];
        float ck[ECK];
    };
    // Values an element thread keeps from preparing a chunk to finishing it.
    struct Keep {
        float x[V];                                // delta + bias
    };
    Chunk raw[3];
    Keep keep[3];

    // Per-thread parts of the element, B/C and entering-state addresses, and
    // which of them exist whatever the chunk.
    uint32_t off_row[V];                           // (er, dbase + cofs(i)) from (chunk row 0, dbase)
#pragma unroll
    for (int i = 0; i < V; i++) off_row[i] = evok[i] ? uint32_t(er * d_in + cofs(i)) * uint32_t(ES) : 0u;
    int bc_row[EBC];                               // step row j of the B/C word, -1 if none
    uint32_t off_bc[EBC];                          // (j, kk) from (chunk row 0, state 0)
#pragma unroll
    for (int m = 0; m < EBC; m++) {
        const int f = m * NE + etid;
        const int j = f / NP, kk = f - (f / NP) * NP;
        const bool ok = !rec && f < T * NP && kk < ns;
        bc_row[m] = ok ? j : -1;
        off_bc[m] = ok ? uint32_t((j * n + k0 + kk) * ES) : 0u;
    }
    uint32_t off_ck[ECK], off_h0[ECK];             // (kk, dd) in a checkpoint and in h0
    bool ck_has[ECK];
#pragma unroll
    for (int m = 0; m < ECK; m++) {
        const int f = m * NE + etid;
        const int kk = f / 64, dd = dbase + (f & 63);
        ck_has[m] = !rec && f < NP * 64 && kk < ns && dd < d_in;
        off_ck[m] = ck_has[m] ? uint32_t((k0 + kk) * d_in + dd) * 4u : 0u;
        off_h0[m] = ck_has[m] ? uint32_t(dd * n + k0 + kk) * 4u : 0u;
    }
    // Partial row g = ((j SC + w) NSW/2 + pair) 4 + r of a chunk holds,
    // for r = 0, 1, 2, 3, dB of state 2 pair, its dC, dB of the next state,
    // its dC (the row order of wave_part4); element thread etid adds rows
    // etid, etid + NE, ...
    int red_j[RPT], red_off[RPT];
    bool red_c[RPT], red_ok[RPT];
#pragma unroll
    for (int m = 0; m < RPT; m++) {
        const int g = m * NE + etid;
        const int r = g & 3, pq = (g >> 2) % (NSW / 2), w = (g / (2 * NSW)) % SC, j = g / (2 * NP);
        const int kk = w * NSW + pq * 2 + (r >> 1);
        red_ok[m] = !rec && g < ROWS && kk < ns;
        red_c[m] = (r & 1) != 0;
        red_j[m] = j;
        red_off[m] = j * n + k0 + kk;
    }
    // Recurrence lane's place in a group of 4 partial rows: row lane / 16, column lane % 16.
    const int red_lane = (lane >> 4) * RS + (lane & 15);

    // Uniform bases of chunk k (clamped into the segment, so always inside the tensors).
    auto row_base = [&](int k) __attribute__((always_inline)) {
        return (brow + int64_t(max(k, kc0)) * T) * d_in + dbase;      // element index
    };
    auto ld = [&](const void* base, int64_t idx, uint32_t boff) __attribute__((always_inline)) {
        const TIn* q = static_cast<const TIn*>(base) + idx;
        return RawIn::load(reinterpret_cast<const TIn*>(reinterpret_cast<const char*>(q) + boff), 0);
    };
    // PR: both elements of the thread's row in one access (bf16: the pair's
    // 32-bit word in w[0]; fp32: the two floats).
    auto ld_pair = [&](Word* w, const void* base, int64_t idx, uint32_t boff) __attribute__((always_inline)) {
        const char* q = reinterpret_cast<const char*>(static_cast<const TIn*>(base) + idx) + boff;
        if constexpr (ES == 2) {
            w[0] = *reinterpret_cast<const uint32_t*>(q);
        } else {
            const float2 v = *reinterpret_cast<const float2*>(q);
            w[0] = v.x;
            w[1] = v.y;
        }
    };
    // Element i of a thread's row as loaded, widened to fp32.
    auto raw_f = [&](const Word* w, int i) __attribute__((always_inline)) -> float {
        if constexpr (PR && ES == 2) return i == 0 ? __uint_as_float(w[0] << 16) : __uint_as_float(w[0] & 0xffff0000u);
        else return RawIn::f(w[i]);
    };
    // Store of the thread's V values of one row of a (b, L, d_in) tensor
    // (rb: the chunk's row base), element i only where ok_i.
    auto store_row = [&](void* base, int64_t rb, const float* v, bool ok0, bool ok1) __attribute__((always_inline)) {
        TIn* q = static_cast<TIn*>(base) + rb;
        if constexpr (PR) {
            if (!ok0) return;
            char* a = reinterpret_cast<char*>(q) + off_row[0];
            if constexpr (ES == 2) *reinterpret_cast<uint32_t*>(a) = f32x2_to_bf16x2(v[0], v[1]);
            else *reinterpret_cast<float2*>(a) = make_float2(v[0], v[1]);
        } else {
            if (ok0) Elem<TIn>::store(reinterpret_cast<TIn*>(reinterpret_cast<char*>(q) + off_row[0]), 0, v[0]);
            if (ok1) Elem<TIn>::store(reinterpret_cast<TIn*>(reinterpret_cast<char*>(q) + off_row[1]), 0, v[1]);
        }
    };
    auto row_ok = [&](int k) __attribute__((always_inline)) { return k >= kc0 && k * T + er < L; };
    auto bc_ok = [&](int k, int m) __attribute__((always_inline)) {
        return k >= kc0 && bc_row[m] >= 0 && k * T + bc_row[m] < L;
    };
    auto ck_ok = [&](int k, int m) __attribute__((always_inline)) {
        return k >= kc0 && ck_has[m] && (k > 0 || p.h0 != nullptr);
    };
    auto load_chunk = [&](Chunk& r, int k) __attribute__((always_inline)) {       // issue the global loads of chunk k
        const bool rv = row_ok(k);
        const int64_t rb = row_base(k);
        if constexpr (PR) {
            const uint32_t o = rv ? off_row[0] : 0u;
            ld_pair(r.u, p.u, rb, o);
            ld_pair(r.dl, p.delta, rb, o);
            if (GATE) ld_pair(r.z, p.z, rb, o);
            ld_pair(r.dy, p.dy, rb, o);
            if (GATE && p.ypre) ld_pair(r.yp, p.ypre, rb, o);
        } else {
#pragma unroll
            for (int i = 0; i < V; i++) {
                const uint32_t o = rv ? off_row[i] : 0u;
                r.u[i] = ld(p.u, rb, o);
                r.dl[i] = ld(p.delta, rb, o);
                if (GATE) r.z[i] = ld(p.z, rb, o);
                r.dy[i] = ld(p.dy, rb, o);
                if (GATE && p.ypre) r.yp[i] = ld(p.ypre, rb, o);
            }
        }
        const int64_t bb = (brow + int64_t(max(k, kc0)) * T) * n;
#pragma unroll
        for (int m = 0; m < EBC; m++) {
            const uint32_t o = bc_ok(k, m) ? off_bc[m] : 0u;
            r.b[m] = ld(p.B, bb, o);
            r.c[m] = ld(p.C, bb, o);
        }
        // Entering state: checkpoint k - 1, or h0 for the first chunk.
        const float* cb = k > 0 ? p.ckpt + (int64_t(bi) * p.nck + k - 1) * n * d_in
                                : (p.h0 ? p.h0 + int64_t(bi) * d_in * n : p.A_log);
#pragma unroll
        for (int m = 0; m < ECK; m++) {
            const uint32_t o = ck_ok(k, m) ? (k > 0 ? off_ck[m] : off_h0[m]) : 0u;
            r.ck[m] = *reinterpret_cast<const float*>(reinterpret_cast<const char*>(k >= kc0 ? cb : p.A_log) + o);
        }
    };
    // Prepare chunk k from its raw values: LDS ring slots s3 (of 3) and s2 (of 2).
    auto prepare = [&](const Chunk& r, Keep& kp, int k, int s3, int s2) __attribute__((always_inline)) {
        const bool rv = row_ok(k);
        float dzv[V], pv[4][V];
#pragma unroll
        for (int i = 0; i < V; i++) {
            const bool ok = rv && evok[i];
            const float u = ok ? raw_f(r.u, i) : 0.0f;
            const float x = (ok ? raw_f(r.dl, i) : 0.0f) + bias_v[i];
            const float z = (GATE && ok) ? raw_f(r.z, i) : 0.0f;
            const float dy = ok ? raw_f(r.dy, i) : 0.0f;
            const float dl = ok ? (SP ? softplus(x) : x) : 0.0f;
            // dy' = dy silu(z); from saved states also dz = dy y' silu'(z),
            // silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z))).
            const float sg = GATE ? rcp_hw(1.0f + exp2_hw(-z * kLog2e)) : 1.0f;
            const float dyp = GATE ? dy * (z * sg) : dy;
            dzv[i] = (GATE && p.ypre) ? dy * raw_f(r.yp, i) * sg * fmaf(z, 1.0f - sg, 1.0f) : 0.0f;
            if (!PR && GATE && p.ypre && ok) {
                TIn* q = static_cast<TIn*>(p.dz) + row_base(k);
                Elem<TIn>::store(reinterpret_cast<TIn*>(reinterpret_cast<char*>(q) + off_row[i]), 0, dzv[i]);
            }
            pv[0][i] = dl;
            pv[1][i] = ZOH ? u : dl * u;
            pv[2][i] = dyp;
            pv[3][i] = u;
            kp.x[i] = x;
        }
        // The four planes: one 8-byte write per plane for a channel pair.
#pragma unroll
        for (int pl = 0; pl < 4; pl++) {
            float* dst = s_prep + pl * PL + (s3 * T + er) * 64;
            if constexpr (PR) {
                *reinterpret_cast<float2*>(dst + cofs(0)) = make_float2(pv[pl][0], pv[pl][1]);
            } else {
#pragma unroll
                for (int i = 0; i < V; i++) dst[cofs(i)] = pv[pl][i];
            }
        }
        if (PR && GATE && p.ypre) store_row(p.dz, row_base(k), dzv, rv && evok[0], rv && evok[V - 1]);
#pragma unroll
        for (int m = 0; m < EBC; m++) {
            const int f = m * NE + etid;
            if ((T * NP) % NE != 0 && f >= T * NP) break;
            const int j = f / NP, kk = f - (f / NP) * NP;
            const bool ok = bc_ok(k, m);
            float* dst = s_bc + s2 * (T * 2 * NP) + ((j * SC + kk / NSW) * 2) * NSW + kk % NSW;
            dst[0] = ok ? RawIn::f(r.b[m]) : 0.0f;
            dst[NSW] = ok ? RawIn::f(r.c[m]) : 0.0f;
        }
#pragma unroll
        for (int m = 0; m < ECK; m++) {
            const int f = m * NE + etid;
            if ((NP * 64) % NE != 0 && f >= NP * 64) break;
            s_ck[s2 * NP * 64 + f] = ck_ok(k, m) ? r.ck[m] : 0.0f;
        }
    };
    // Finish chunk k: sums of the recurrence waves' partials, the per-element
    // gradients, and the chunk's dB, dC rows of this channel group.
    auto finalize = [&](const Keep& kp, int k, int s3, int s2) __attribute__((always_inline)) {
        const bool rv = row_ok(k);
        const int64_t rb = row_base(k);
        // This thread's (step row, channel) in the partials of wave 0; wave w at + w T 64.
        const float2* pp = s_part + (s2 * SC * T + er) * 64;
        float2 q[SC][V];
        float pq[3][V];                            // Delta, dy', u of the thread's elements
        const float* sp = s_prep + (s3 * T + er) * 64;
        if constexpr (PR) {
            // A channel pair's partials and planes as 16- and 8-byte reads.
#pragma unroll
            for (int w = 0; w < SC; w++) {
                const float4 v = *reinterpret_cast<const float4*>(pp + w * T * 64 + cofs(0));
                q[w][0] = make_float2(v.x, v.y);
                q[w][1] = make_float2(v.z, v.w);
            }
#pragma unroll
            for (int j = 0; j < 3; j++) {
                const float2 v = *reinterpret_cast<const float2*>(sp + (j == 0 ? 0 : j + 1) * PL + cofs(0));
                pq[j][0] = v.x;
                pq[j][1] = v.y;
            }
        } else {
#pragma unroll
            for (int w = 0; w < SC; w++)
#pragma unroll
                for (int i = 0; i < V; i++) q[w][i] = pp[w * T * 64 + cofs(i)];
#pragma unroll
            for (int j = 0; j < 3; j++)
#pragma unroll
                for (int i = 0; i < V; i++) pq[j][i] = sp[(j == 0 ? 0 : j + 1) * PL + cofs(i)];
        }
        float du_v[V], dd_v[V];
#pragma unroll
        for (int i = 0; i < V; i++) {
            const float4 pr = make_float4(pq[0][i], 0.0f, pq[1][i], pq[2][i]);   // (Delta, -, dy', u)
            float S1 = q[0][i].x, S2 = q[0][i].y;
#pragma unroll
            for (int w = 1; w < SC; w++) {
                S1 += q[w][i].x;
                S2 += q[w][i].y;
            }
            // Euler: S1 = sum g B, dDelta = S2 + u S1, du = Delta S1 + dy' D; the hold:
            // S1 = sum g beta B, S2 already holds the input term, du = S1 + dy' D.
            const float dDelta = ZOH ? S2 : fmaf(pr.w, S1, S2);
            const float sgx = SP ? rcp_hw(1.0f + exp2_hw(-kp.x[i] * kLog2e)) : 1.0f;   // softplus' = sigmoid
            const float ddl = SP ? dDelta * sgx : dDelta;
            const float du = ZOH ? fmaf(pr.z, Dv[i], S1) : fmaf(pr.x, S1, pr.z * Dv[i]);
            du_v[i] = du;
            dd_v[i] = ddl;
            if (rv && evok[i]) {
                if constexpr (!PR) {
                    if constexpr (!SL) {
                        auto st = [&](void* base, float v) __attribute__((always_inline)) {
                            TIn* q = static_cast<TIn*>(base) + rb;
                            Elem<TIn>::store(reinterpret_cast<TIn*>(reinterpret_cast<char*>(q) + off_row[i]), 0, v);
                        };
                        st(p.du, du);
                        st(p.ddelta, ddl);
                    } else {
                        // This slice's parts of du and ddelta (both are linear in S1, S2).
                        const int64_t e = int64_t(slice) * p.b * L * d_in + rb + off_row[i] / uint32_t(ES);
                        p.part_du[e] = du;
                        p.part_dd[e] = ddl;
                    }
                }
                if (slice == 0) accD[i] = fmaf(pr.z, pr.w, accD[i]);
                // Written as the FMA it is, so that no kernel form is left to
                // the compiler's choice of contracting the product into it.
                accBias[i] = SP ? fmaf(dDelta, sgx, accBias[i]) : accBias[i] + dDelta;
            }
        }
        if constexpr (PR) {
            const bool ok = rv && evok[0];   // d_in even: both channels or neither
            if constexpr (!SL) {
                store_row(p.du, rb, du_v, ok, ok);
                store_row(p.ddelta, rb, dd_v, ok, ok);
            } else if (ok) {
                const int64_t e = int64_t(slice) * p.b * L * d_in + rb + off_row[0] / uint32_t(ES);
                *reinterpret_cast<float2*>(p.part_du + e) = make_float2(du_v[0], du_v[1]);
                *reinterpret_cast<float2*>(p.part_dd + e) = make_float2(dd_v[0], dd_v[1]);
            }
        }
        // dB, dC of the chunk's rows: T * n consecutive values of each.
        const int64_t ob = ((int64_t(grp) * p.b + bi) * L + int64_t(k) * T) * n;
        {
#pragma unroll
            for (int m = 0; m < RPT; m++) {
                if (!red_ok[m] || k * T + red_j[m] >= L) continue;
                const float4* src = reinterpret_cast<const float4*>(s_dbc + Lds::row_off(s2 * ROWS + m * NE + etid));
                const float4 a = src[0], b = src[1], c = src[2], e = src[3];
                float sum = a.x;                   // the 16 partials in row order
                sum += a.y; sum += a.z; sum += a.w;
                sum += b.x; sum += b.y; sum += b.z; sum += b.w;
                sum += c.x; sum += c.y; sum += c.z; sum += c.w;
                sum += e.x; sum += e.y; sum += e.z; sum += e.w;
                (red_c[m] ? p.part_C : p.part_B)[ob + red_off[m]] = sum;
            }
        }
    };
    // Recurrence waves, chunk c: recompute its states, then the adjoint back through them.
    auto process = [&](int c, int s3, int s2) __attribute__((always_inline)) {
        float hstart[NSW];
#pragma unroll
        for (int q = 0; q < NSW; q++) hstart[q] = s_ck[(s2 * NP + n0 + q) * 64 + lane];
        const float* bcw = s_bc + s2 * (T * 2 * NP) + wave * 2 * NSW;
        float h[NSW];                                               // running state
        float hs[T][NSW], as[T][NSW], bs[ZOH ? T : 1][NSW];        // states, decays, hold weights of the chunk
        float dls[T], wvs[T];                                       // Delta and w of the chunk's steps, read once
#pragma unroll
        for (int q = 0; q < NSW; q++) h[q] = hstart[q];
#pragma unroll
        for (int j = 0; j < T; j++) {
            const int e = (s3 * T + j) * 64 + lane;
            const float4 pr = make_float4(s_prep[e], s_prep[PL + e], 0.0f, 0.0f);
            dls[j] = pr.x;
            wvs[j] = pr.y;
#pragma unroll
            for (int q = 0; q < NSW; q++) {
                const float x2 = pr.x * A2[q];
                const float a = exp2_hw(x2);
                if constexpr (ZOH) {
                    const float beta = zoh_weight(pr.x, x2, a, invA[q]);
                    h[q] = fmaf(a, h[q], beta * (pr.y * bcw[j * SC * 2 * NSW + q]));
                    bs[j][q] = beta;
                } else {
                    h[q] = fmaf(a, h[q], pr.y * bcw[j * SC * 2 * NSW + q]);
                }
                hs[j][q] = h[q];
                as[j][q] = a;
            }
        }
#pragma unroll
        for (int j = T - 1; j >= 0; j--) {
            const int e = (s3 * T + j) * 64 + lane;
            const float4 pr = make_float4(dls[j], wvs[j], s_prep[2 * PL + e], ZOH ? s_prep[3 * PL + e] : 0.0f);
            float S1 = 0.0f, S2 = 0.0f, S3 = 0.0f, dBv[NSW], dCv[NSW];
#pragma unroll
            for (int q = 0; q < NSW; q++) {
                const float Bq = bcw[j * SC * 2 * NSW + q], Cq = bcw[j * SC * 2 * NSW + NSW + q];
                g[q] = fmaf(pr.z, Cq, g[q]);
                const float hp = j > 0 ? hs[j - 1][q] : hstart[q];
                const float ga = g[q] * as[j][q];
                const float gah = ga * hp;
                S2 = fmaf(gah, An[q], S2);
                dA[q] = fmaf(gah, pr.x, dA[q]);
                dCv[q] = pr.z * hs[j][q];
                if constexpr (ZOH) {
                    // beta = (a - 1)/A: d beta/dDelta = a, d beta/dA = (Delta a - beta)/A.
                    const float beta = bs[j][q];
                    const float gb = g[q] * beta;
                    S1 = fmaf(gb, Bq, S1);
                    S3 = fmaf(ga, Bq, S3);
                    dA[q] = fmaf(g[q] * (pr.y * Bq), fmaf(pr.x, as[j][q], -beta) * invA[q], dA[q]);
                    dBv[q] = gb * pr.y;
                } else {
                    S1 = fmaf(g[q], Bq, S1);
                    dBv[q] = g[q] * pr.y;
                }
                g[q] = ga;
            }
            if constexpr (ZOH) S2 = fmaf(pr.w, S3, S2);   // the input term of dDelta: u sum g a B
            s_part[((s2 * SC + wave) * T + j) * 64 + lane] = make_float2(S1, S2);
            // dB, dC of this step over the 64 channels, two states at a time:
            // 16 partials each, to LDS for the element waves to add up.
            float* dst = s_dbc + ((s2 * T + j) * SC + wave) * (NSW / 2) * 4 * RS + red_lane;
#pragma unroll
            for (int q = 0; q < NSW; q += 2)
                dst[(q / 2) * 4 * RS] = wave_part4(dBv[q], dBv[q + 1], dCv[q], dCv[q + 1]);
        }
    };

    // (The lambdas are forced inline: called from three unrolled copies, the
    // compiler would otherwise emit them as functions, with their arrays in
    // scratch memory and LDS reached through generic pointers.)
    // Iteration i: the recurrence waves take chunk c = kcl - i; the
    // element waves issue the loads of chunk c - 1 - AHEAD, finish chunk c + 1
    // and prepare chunk c - 1.  Ring slots: LDS (Delta, w, dy', u) and the kept
    // values by i % 3 (compile-time: the loops are unrolled by three), the raw
    // words of chunk x in slot (kcl - x - 2) % 3, the two-slot LDS rings by
    // i & 1.  AHEAD = 2 (loads two iterations before their use) where the
    // registers allow the third chunk in flight, else 1.
    constexpr int AHEAD = NP <= 16 ? 2 : 1;
    const int niter = (kcl - kc0 + 2 + 2) / 3 * 3;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (!rec) {
        load_chunk(raw[1], kcl);
        prepare(raw[1], keep[0], kcl, 0, 0);
        load_chunk(raw[2], kcl - 1);
        if (AHEAD == 2) load_chunk(raw[0], kcl - 2);
    }
    barrier_lds();
    auto rec_iter = [&](auto ph, int i) __attribute__((always_inline)) {
        constexpr int PH = decltype(ph)::value;
        const int c = kcl - i;
        if (c >= kc0) process(c, PH, i & 1);
        barrier_lds();
    };
    auto elem_iter = [&](auto ph, int i) __attribute__((always_inline)) {
        constexpr int PH = decltype(ph)::value;
        const int c = kcl - i;
        load_chunk(raw[(PH + AHEAD - 1) % 3], c - 1 - AHEAD);
        if (c + 1 >= kc0 && c + 1 <= kcl) finalize(keep[(PH + 2) % 3], c + 1, (PH + 2) % 3, (i + 1) & 1);
        if (c - 1 >= kc0) prepare(raw[(PH + 2) % 3], keep[(PH + 1) % 3], c - 1, (PH + 1) % 3, (i + 1) & 1);
        barrier_lds();
    };
    if (rec) {
        for (int i = 0; i < niter; i += 3) {
            rec_iter(I0{}, i);
            rec_iter(I1{}, i + 1);
            rec_iter(I2{}, i + 2);
        }
    } else {
        for (int i = 0; i < niter; i += 3) {
            elem_iter(I0{}, i);
            elem_iter(I1{}, i + 1);
            elem_iter(I2{}, i + 2);
        }
    }

    const int64_t pb = int64_t(seg) * p.b + bi;    // partials of this segment and batch row
    if (rec) {
        if (dv) {
#pragma unroll
            for (int q = 0; q < NSW; q++) {
                if (n0 + q >= ns) continue;
                p.part_A[(pb * d_in + d) * n + k0 + n0 + q] = dA[q] * An[q];
                if (p.dh0 && seg == 0) p.dh0[(int64_t(bi) * d_in + d) * n + k0 + n0 + q] = g[q];
            }
        }
        if (seg > 0) {
            // Hand the adjoint on to the earlier segment.
            uint32_t* dst = reinterpret_cast<uint32_t*>(p.handoff) + (int64_t(seg - 1) * G + gi) * NP * 64;
#pragma unroll
            for (int q = 0; q < NSW; q++)
                if (n0 + q < ns)
                    __hip_atomic_store(dst + (n0 + q) * 64 + lane, __float_as_uint(g[q]), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
        barrier_lds();
        barrier_lds();
    } else {
        // dD and dbias: sum the T step rows of each channel (fixed order).
        float* s_red = reinterpret_cast<float*>(lds + Lds::off_prep);   // [T][64][2]
#pragma unroll
        for (int i = 0; i < V; i++) {
            s_red[(er * 64 + cofs(i)) * 2] = accD[i];
            s_red[(er * 64 + cofs(i)) * 2 + 1] = accBias[i];
        }
        barrier_lds();
        if (etid < 64 && dbase + etid < d_in) {
            float sD = 0.0f, sB = 0.0f;
            for (int r = 0; r < T; r++) {
                sD += s_red[(r * 64 + etid) * 2];
                sB += s_red[(r * 64 + etid) * 2 + 1];
            }
            if (slice == 0) p.part_D[pb * d_in + dbase + etid] = sD;
            p.part_bias[((int64_t(seg) * p.slices + slice) * p.b + bi) * d_in + dbase + etid] = sB;
        }
        barrier_lds();
    }
    if (seg > 0) {
        // As in the forward hand-off: every wave's stores acknowledged, the
        // workgroup met, then one thread sets the flag.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(p.ctl + kFlagOffset + (seg - 1) * G + gi, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// out[i] = sum over g of part[g * count + i], added in the order g = 0, 1, ...
// and written as TOut (fp32 or bf16 words); grid-stride, so the host may cap
// the grid.
template <typename TOut>
__global__ __launch_bounds__(256) void reduce_groups(const float* __restrict__ part, TOut* __restrict__ out,
                                                     int64_t count, int groups) {
    for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count; i += int64_t(gridDim.x) * blockDim.x) {
        float s = 0.0f;
        for (int g = 0; g < groups; g++) s += part[int64_t(g) * count + i];
        Elem<TOut>::store(out, i, s);
    }
}

}  // namespace ss
