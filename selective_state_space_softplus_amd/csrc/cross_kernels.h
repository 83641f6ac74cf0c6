// cross_kernels.h -- VMamba's cross scan with the merge done in LDS, in one
// kernel (githubissues.com VMamba issue 206: CrossScan and CrossMerge only
// arrange the sequence around the selective scan, whose d_state is 1 there).
//
// Each H x W map is read as four sequences of L = H * W steps (direction 0
// row-major, 1 column-major, 2 and 3 the same orders backwards), each scanned
// as one batch row of the selective scan (mhpn.cn selective_scan walk-through,
// sections 3-5: delta' = softplus(delta + bias), h = exp(delta' A) h +
// delta' B u, y = C h + D u), and the four outputs are summed at the map
// position each step came from.
//
// cross_fused<TIn, NS>: one workgroup per (map, block of 8 channels), four
// waves, wave k scanning direction k.  Every direction visits every position,
// and each position's last visit comes after the middle of the sequence, so
// the sum of a map slice is complete only at the end: the workgroup keeps it
// in LDS (L x 8 fp32, 128 KB at L = 4096) and writes it to y once.
//
// Time is walked in chunks of 64 steps.  Lane 8c + s of a wave holds channel
// c and the 8 steps s*8 .. s*8+7 of the chunk: it forms the decays
// a_j = exp(delta'_j A) and inputs b_j = delta'_j B_j u_j of its steps, folds
// them into the pair (P, H) = (prod a_j, state after the 8 steps from zero),
// and the 8 sub-chunks of a channel (8 neighbouring lanes) are combined by an
// inclusive scan over s with DPP row shifts, (P1, H1) then (P2, H2) ->
// (P1 P2, P2 H1 + H2), which gives every lane the state entering its
// sub-chunk from the chunk's carried state; it then walks its 8 steps again
// from there, producing the outputs.  The decays and inputs stay in
// registers between the two walks, so the second costs one FMA per step and
// state.  The first half (all but the carried state) of chunk c + 1 runs
// beside the second half of chunk c.  Each chunk's inputs are loaded two
// iterations ahead by buffer loads (issued unconditionally: past the end they
// read 0, so the compiler sees every load issued and waits only for the
// oldest).
//
// The outputs of a chunk go to a staging area in LDS (one per direction,
// double-buffered).  After the barrier that ends the chunk's iteration, the
// next iteration, once it has computed its own chunk, has thread (k, i) add
// step i of direction k into the sum of its map position, together with the
// contributions of the other directions that visited the same position in
// the same chunk -- the thread of the lowest such direction does all of
// them, the others skip it.  So every position is updated by one thread per
// chunk, in the order (chunk, direction): no atomics, and the same bits on
// every run.
//
// ss_cross_scan_fwd_ex selects this kernel for SS_CROSS_ONE_PASS.  It moves
// 2.3x fewer bytes than the two-pass form but is slower on MI355X (8
// channels per workgroup, all its LDS allows, means 32-byte row segments and
// one workgroup per compute unit), so the two-pass form is the default.
#pragma once

#include "ss_device.h"

namespace ss {

struct CrossParams {
    const void* x;        // (maps, H, W, d_in)
    const void* delta;    // (maps, 4, L, d_in)
    const float* A_log;   // (4, d_in, n)
    const void* B;        // (maps, 4, L, n)
    const void* C;        // (maps, 4, L, n)
    const float* D;       // (4, d_in)
    const float* bias;    // (4, d_in) or null
    float* y;             // (maps, H, W, d_in) fp32
    float* last_state;    // (maps, 4, d_in, n) or null
    uint32_t* err;        // the call's two status words (cleared: nothing here waits)
    int maps, H, W, L, d_in, n;
    int softplus;
    int ncb;              // blocks of 8 channels: ceil(d_in / 8)
    int vec_y;            // y rows take 16-byte stores (d_in % 4 == 0, y 16-byte aligned)
    uint32_t magic_h, magic_w;   // ceil(2^32 / H), ceil(2^32 / W) for H, W > 1: exact division of 0 <= v < 2^16
};

constexpr int kCrossCh = 8;          // channels per workgroup
constexpr int kCrossChunk = 64;      // steps per chunk
constexpr int kCrossAhead = 2;       // iterations a chunk's loads are issued ahead of their use
constexpr int kCrossStage = 520;     // words of one staged chunk: 8 channels x 65 (one word of padding)

// Words of the LDS sum of a map slice: 8 per position, and 4 more after every
// 8 positions so that rows W positions apart fall in different banks.
__host__ __device__ constexpr int cross_acc_words(int L) { return L * 8 + (L + 7) / 8 * 4; }
__device__ __forceinline__ int cross_acc_row(int p) { return p * 8 + (p >> 3) * 4; }

// Dynamic LDS of cross_fused: the sum, 2 x 4 staged chunks, each wave's B and
// C values of one chunk (64 steps x NS states, two tensors), and one spare row
// per wave that threads with nothing to add write to instead of the sum.
__host__ __device__ constexpr size_t cross_lds_bytes(int L, int NS) {
    return size_t(cross_acc_words(L) + 2 * 4 * kCrossStage + 4 * 2 * kCrossChunk * NS + 4 * 8) * 4;
}

// Block index -> (map, channel block), so that the workgroups one XCD runs at
// the same time take neighbouring channel blocks of one map: consecutive
// dispatches go to the 8 XCDs in turn, and the four 8-channel blocks that
// share a 128-byte row segment then meet in one L2.
__device__ __forceinline__ int cross_logical_block(int b, int nb) {
    const int xcd = b & 7, idx = b >> 3, q = nb >> 3, r = nb & 7;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// Lane l takes the value of lane l - K of its row of 16 lanes (DPP row_shr:K;
// lanes l % 16 < K keep their own value, which the callers do not use).
template <int K>
__device__ __forceinline__ float dpp_row_shr(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x110 + K, 0xf, 0xf, false));
}

template <typename TIn, int NS>
struct CrossTile {
    typename Raw<TIn>::type u[8], dl[8];   // this lane's channel at its 8 steps
    typename Raw<TIn>::type b[NS], c[NS];  // B and C of step `lane` of the chunk
};

// One element of a buffer (raw bf16 word or fp32) at byte offset `off`; an
// offset at or past the buffer's end (a negative one included) reads 0.
template <typename TIn>
__device__ __forceinline__ typename Raw<TIn>::type buffer_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (sizeof(TIn) == 2)
        return uint32_t(__builtin_amdgcn_raw_buffer_load_b16(r, int(off), 0, 0));
    else
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0));
}

template <typename TIn, int NS, bool SP>
__global__ __launch_bounds__(256) void cross_fused(CrossParams p) {
    extern __shared__ __align__(16) float smem[];
    using RT = Raw<TIn>;
    constexpr uint32_t es = sizeof(TIn);
    const int lane = threadIdx.x & 63;
    const int k = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));   // direction of this wave
    const int s = lane & 7, ci = lane >> 3;   // sub-chunk, channel in the block
    const int blk = cross_logical_block(int(blockIdx.x), int(gridDim.x));
    const int m = blk / p.ncb, cb = blk - m * p.ncb;
    const int L = p.L, H = p.H, W = p.W, n = p.n;
    const int d_in = p.d_in;
    const int ch = cb * kCrossCh + ci;
    const bool cv = ch < d_in;
    const int nch = (L + kCrossChunk - 1) / kCrossChunk;

    // Buffers of this map's x and of direction k's delta, B and C (each below
    // 2^31 bytes); reads past their ends return 0 and are never used.
    const uint32_t rowb = uint32_t(d_in) * es;
    const uint32_t choff = uint32_t(cv ? ch : d_in - 1) * es;
    const auto rx = buffer_rsrc(static_cast<const TIn*>(p.x) + int64_t(m) * L * d_in, uint32_t(L) * rowb);
    const auto rd = buffer_rsrc(static_cast<const TIn*>(p.delta) + (int64_t(m) * 4 + k) * L * d_in, uint32_t(L) * rowb);
    const auto rB = buffer_rsrc(static_cast<const TIn*>(p.B) + (int64_t(m) * 4 + k) * L * n, uint32_t(L * n) * es);
    const auto rC = buffer_rsrc(static_cast<const TIn*>(p.C) + (int64_t(m) * 4 + k) * L * n, uint32_t(L * n) * es);

    // Parameters of direction k, channel ch.
    float A2[NS];
#pragma unroll
    for (int q = 0; q < NS; q++) A2[q] = (cv && q < n) ? a2_from_alog(p.A_log[(int64_t(k) * d_in + ch) * n + q]) : 0.0f;
    const float Dv = cv ? p.D[int64_t(k) * d_in + ch] : 0.0f;
    const float bias = (cv && p.bias) ? p.bias[int64_t(k) * d_in + ch] : 0.0f;

    float* acc = smem;
    float* stage = smem + cross_acc_words(L);
    float* bcw = stage + 2 * 4 * kCrossStage + k * (2 * kCrossChunk * NS);   // this wave's B (then C) of a chunk

    // Column-major step v -> map position, and map position -> column-major
    // step (0 <= v, pp < 2^16: exact by the multiply-high with ceil(2^32 / H)).
    auto colmajor_pos = [&](int v) -> int {
        const int w = H == 1 ? v : int(__umulhi(uint32_t(v), p.magic_h));
        return (v - w * H) * W + w;
    };
    auto colmajor_step = [&](int pp) -> int {
        const int h = W == 1 ? pp : int(__umulhi(uint32_t(pp), p.magic_w));
        return (pp - h * W) * H + h;
    };
    // Map position of step t of this wave's direction (t < L).
    auto pos_of = [&](int t) -> int {
        const int v = k >= 2 ? L - 1 - t : t;
        return (k & 1) ? colmajor_pos(v) : v;
    };

    // x offsets of a lane's 8 steps.  Row-major directions step one row at a
    // time; column-major ones W rows at a time, wrapping to the next (previous)
    // column at most once in 8 steps when H >= 8, else by division.
    const bool inc_col = H >= 8;
    auto x_offsets = [&](int t0, uint32_t (&o)[8]) __attribute__((always_inline)) {
        if (!(k & 1)) {
            const int p0 = k >= 2 ? L - 1 - t0 : t0;    // past either end: reads 0
            const uint32_t o0 = uint32_t(p0) * rowb + choff;
#pragma unroll
            for (int j = 0; j < 8; j++) o[j] = k >= 2 ? o0 - j * rowb : o0 + j * rowb;
        } else if (inc_col) {
            const int tc = min(t0, L - 1);             // past the end: any position in the map
            const int v0 = k >= 2 ? L - 1 - tc : tc;
            const int w0 = int(__umulhi(uint32_t(v0), p.magic_h));
            const int h0 = v0 - w0 * H;
            const int p0 = h0 * W + w0;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                int pj;
                if (k >= 2) pj = h0 - j >= 0 ? p0 - j * W : p0 - j * W + L - 1;
                else pj = h0 + j < H ? p0 + j * W : p0 + j * W - (L - 1);
                pj = t0 + j < L ? pj : p0;
                o[j] = uint32_t(pj) * rowb + choff;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; j++) o[j] = uint32_t(pos_of(min(t0 + j, L - 1))) * rowb + choff;
        }
    };

    // Offsets within a map's x, a direction's delta, B and C are below 2^31.
    auto load_tile = [&](CrossTile<TIn, NS>& tl, int c) __attribute__((always_inline)) {
        const int t0 = c * kCrossChunk + s * 8;
        uint32_t ox[8];
        x_offsets(t0, ox);
#pragma unroll
        for (int j = 0; j < 8; j++) tl.u[j] = buffer_elem<TIn>(rx, ox[j]);
        const uint32_t od = uint32_t(t0) * rowb + choff;
#pragma unroll
        for (int j = 0; j < 8; j++) tl.dl[j] = buffer_elem<TIn>(rd, od + j * rowb);
        const uint32_t ob = uint32_t((c * kCrossChunk + lane) * n) * es;
#pragma unroll
        for (int q = 0; q < NS; q++) {
            const uint32_t oq = q < n ? ob + q * es : 0xffffffffu;   // state slots past n read 0
            tl.b[q] = buffer_elem<TIn>(rB, oq);
            tl.c[q] = buffer_elem<TIn>(rC, oq);
        }
    };

    if (blockIdx.x == 0 && threadIdx.x < 2 && p.err) p.err[threadIdx.x] = 0u;
    // The sum starts at zero.
    for (int i = int(threadIdx.x) * 4; i < cross_acc_words(L); i += 256 * 4)
        *reinterpret_cast<float4*>(acc + i) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);

    float hc[NS];   // state of channel ch entering the chunk (the same in all 8 lanes of the channel)
#pragma unroll
    for (int q = 0; q < NS; q++) hc[q] = 0.0f;

    float* spare = bcw + 2 * kCrossChunk * NS * (4 - k) + k * 8;   // this wave's spare row (after all B, C areas)

    // A chunk in two halves.  local(): what needs no carried state -- the
    // step sizes, decays and inputs of the lane's 8 steps, its sub-chunk's
    // (P, H) from a zero state and their scan over the 8 sub-chunks (steps
    // past L decay by 1 and add nothing).  finish(): the carried state applied,
    // the 8 steps walked again, the outputs staged.  The loop below runs
    // chunk c + 1's local() beside chunk c's finish(): two independent chains.
    struct Local {
        float a[8][NS], bu[8][NS], cc[8][NS], yv[8], P[NS], Hh[NS];
    };
    auto local = [&](const CrossTile<TIn, NS>& tl, int c, Local& r) __attribute__((always_inline)) {
        const int t0 = c * kCrossChunk + s * 8;
        // B and C of the chunk through this wave's LDS: [step][state].
#pragma unroll
        for (int q = 0; q < NS; q++) {
            bcw[lane * NS + q] = RT::f(tl.b[q]);
            bcw[kCrossChunk * NS + lane * NS + q] = RT::f(tl.c[q]);
        }
        // The wave's own lanes read what the others wrote: LDS accesses of one
        // wave complete in order, so only the compiler must keep them so.
        __builtin_amdgcn_wave_barrier();
        float dsum = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            float dl = RT::f(tl.dl[j]) + bias;
            if constexpr (SP) dl = softplus(dl);
            const bool ok = t0 + j < L;
            dl = ok ? dl : 0.0f;
            const float u = RT::f(tl.u[j]);
            const float du = dl * u;
            dsum += dl;
            r.yv[j] = Dv * u;
#pragma unroll
            for (int q = 0; q < NS; q++) {
                r.a[j][q] = exp2_hw(dl * A2[q]);
                const float b = du * bcw[(s * 8 + j) * NS + q];
                r.bu[j][q] = ok ? b : 0.0f;
                r.cc[j][q] = bcw[kCrossChunk * NS + (s * 8 + j) * NS + q];
            }
        }
#pragma unroll
        for (int q = 0; q < NS; q++) {
            float P = exp2_hw(dsum * A2[q]), Hh = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++) Hh = fmaf(r.a[j][q], Hh, r.bu[j][q]);
            static_for<0, 3>([&](auto I) __attribute__((always_inline)) {
                constexpr int off = 1 << decltype(I)::value;
                const float Pp = dpp_row_shr<off>(P), Hp = dpp_row_shr<off>(Hh);
                const bool in = s >= off;
                const float Hn = fmaf(P, Hp, Hh), Pn = P * Pp;
                Hh = in ? Hn : Hh;
                P = in ? Pn : P;
            });
            r.P[q] = P;
            r.Hh[q] = Hh;
        }
    };
    auto finish = [&](const Local& r, int c) __attribute__((always_inline)) {
        float yv[8];
#pragma unroll
        for (int j = 0; j < 8; j++) yv[j] = r.yv[j];
#pragma unroll
        for (int q = 0; q < NS; q++) {
            const float hend = fmaf(r.P[q], hc[q], r.Hh[q]);    // state after sub-chunk s
            const float hprev = dpp_row_shr<1>(hend);
            float h = s == 0 ? hc[q] : hprev;                   // state entering sub-chunk s
            hc[q] = __shfl(hend, ci * 8 + 7, 64);               // state after the chunk
#pragma unroll
            for (int j = 0; j < 8; j++) {
                h = fmaf(r.a[j][q], h, r.bu[j][q]);
                yv[j] = fmaf(r.cc[j][q], h, yv[j]);
            }
        }
        float* st = stage + ((c & 1) * 4 + k) * kCrossStage + ci * 65 + s * 8;
#pragma unroll
        for (int j = 0; j < 8; j++) st[j] = yv[j];
    };

    // The sums of chunk c's positions, from its staged outputs (after the
    // barrier that follows the chunk's computation).
    auto add_chunk = [&](int c, auto tail) __attribute__((always_inline)) {
        constexpr bool TAIL = decltype(tail)::value;
        // Thread (k, lane): the position pp of step c*64 + lane of direction k.
        // Its other visits are at steps pp and L-1-pp (row-major) and tc and
        // L-1-tc (column-major); every direction visiting pp in this chunk is
        // added by the thread of the lowest of them, in direction order.  A
        // thread with nothing to add reads and writes its wave's spare row.
        const int t = c * kCrossChunk + lane;
        const bool valid = !TAIL || t < L;
        const int tt = TAIL ? min(t, L - 1) : t;
        const int pp = pos_of(tt);
        const int tc = (k & 1) ? (k >= 2 ? L - 1 - tt : tt) : colmajor_step(pp);
        const int cbase = c * kCrossChunk;
        const int rel[4] = {pp - cbase, tc - cbase, L - 1 - pp - cbase, L - 1 - tc - cbase};
        bool lower = false, other = false;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
            const bool in = kk != k && uint32_t(rel[kk]) < uint32_t(kCrossChunk);
            lower |= in && kk < k;
            other |= in;
        }
        const bool mine = valid && !lower;
        float* row = mine ? acc + cross_acc_row(pp) : spare;
        float4 v0 = *reinterpret_cast<float4*>(row), v1 = *reinterpret_cast<float4*>(row + 4);
        auto add_dir = [&](int kk, int r) __attribute__((always_inline)) {
            const float* sv = stage + ((c & 1) * 4 + kk) * kCrossStage + r;
            v0.x += sv[0 * 65]; v0.y += sv[1 * 65]; v0.z += sv[2 * 65]; v0.w += sv[3 * 65];
            v1.x += sv[4 * 65]; v1.y += sv[5 * 65]; v1.z += sv[6 * 65]; v1.w += sv[7 * 65];
        };
        add_dir(k, lane);
        if (other && mine) {
#pragma unroll
            for (int kk = 0; kk < 4; kk++)
                if (kk > k && uint32_t(rel[kk]) < uint32_t(kCrossChunk)) add_dir(kk, rel[kk]);
        }
        *reinterpret_cast<float4*>(row) = v0;
        *reinterpret_cast<float4*>(row + 4) = v1;
    };

    // Iteration c: the loads of chunk c + 3, chunk c + 1's local(), chunk c's
    // finish(), then the adds of chunk c - 1, whose outputs every wave staged
    // before the last barrier: one barrier an iteration.  Loads run two
    // iterations ahead of their use (a ring of three tiles).
    static_assert(kCrossAhead == 2, "the loop below keeps three tiles");
    CrossTile<TIn, NS> tiles[3];
    load_tile(tiles[0], 0);
    load_tile(tiles[1], 1);
    load_tile(tiles[2], 2);
    Local lc[2];
    local(tiles[0], 0, lc[0]);
    for (int c0 = 0; c0 < nch; c0 += 6) {
        static_for<0, 6>([&](auto I) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value;
            const int c = c0 + i;
            if (c < nch) {
                load_tile(tiles[i % 3], c + 3);
                local(tiles[(i + 1) % 3], c + 1, lc[(i + 1) % 2]);
                finish(lc[i % 2], c);
                if (c > 0) add_chunk(c - 1, std::false_type{});
                barrier_lds();
            }
        });
    }
    if (L % kCrossChunk == 0) add_chunk(nch - 1, std::false_type{});
    else add_chunk(nch - 1, std::true_type{});

    if (p.last_state && cv && s == 0) {
#pragma unroll
        for (int q = 0; q < NS; q++)
            if (q < n) p.last_state[((int64_t(m) * 4 + k) * d_in + ch) * n + q] = hc[q];
    }
    barrier_lds();
    // The finished sums to y, 4 channels per thread.
    float* ym = p.y + int64_t(m) * L * d_in + cb * kCrossCh;
    const int nvalid = min(kCrossCh, d_in - cb * kCrossCh);
    for (int i = int(threadIdx.x); i < L * 2; i += 256) {
        const int pp = i >> 1, half = i & 1;
        const float4 v = *reinterpret_cast<const float4*>(acc + cross_acc_row(pp) + half * 4);
        float* dst = ym + int64_t(pp) * d_in + half * 4;
        if (p.vec_y && half * 4 + 4 <= nvalid) {
            *reinterpret_cast<float4*>(dst) = v;
        } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; e++)
                if (half * 4 + e < nvalid) dst[e] = vv[e];
        }
    }
}

}  // namespace ss
