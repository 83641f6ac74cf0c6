// conv_kernels.h -- the convolution step that precedes the SSM step in a
// decode step (jiafeimiao.top, Mamba.step, the "Conv step"): per (b, d)
// channel a window of the last W inputs moves one place towards index 0, the
// new input enters at index W-1, and
//     out = silu(sum_w window[w] * weight[d, w] + bias[d])      (silu optional)
// The window keeps the element type of x, so it holds the inputs exactly.
//
// conv_update<TIn, W, VEC>: one thread per channel.  The window of a channel
// is W consecutive elements, read and written whole (one 8- or 16-byte access
// when VEC), so consecutive threads touch consecutive memory.  Bound by HBM:
// 2 W + 2 elements move per channel, the weights and bias stay in cache.
#pragma once

#include "ss_device.h"

namespace ss {

struct ConvParams {
    void* state;          // (b, d_in, W), TIn
    const void* x;        // (b, d_in), TIn
    const float* weight;  // (d_in, W)
    const float* bias;    // (d_in) or null
    void* out;            // (b, d_in), TIn
    int64_t b, d_in;
    int silu;
};

// W consecutive elements as raw words: fp32 words, or bf16 halves (element i
// is the low half of word i/2 when i is even).
template <typename TIn, int W, bool VEC>
struct Window {
    static constexpr int NW = sizeof(TIn) == 2 ? (W + 1) / 2 : W;
    static_assert(!VEC || ((NW == 2 || NW == 4) && W * int(sizeof(TIn)) == 4 * NW), "whole 8- or 16-byte window");
    uint32_t w[NW];
    __device__ __forceinline__ void load(const TIn* p) {
        if constexpr (VEC && NW == 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(p);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else if constexpr (VEC && NW == 2) {
            const uint2 v = *reinterpret_cast<const uint2*>(p);
            w[0] = v.x; w[1] = v.y;
        } else if constexpr (sizeof(TIn) == 2) {
#pragma unroll
            for (int i = 0; i < NW; i++) w[i] = 0u;
#pragma unroll
            for (int i = 0; i < W; i++) w[i / 2] |= uint32_t(p[i]) << (16 * (i & 1));
        } else {
#pragma unroll
            for (int i = 0; i < W; i++) w[i] = __float_as_uint(p[i]);
        }
    }
    __device__ __forceinline__ void store(TIn* p) const {
        if constexpr (VEC && NW == 4) {
            *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
        } else if constexpr (VEC && NW == 2) {
            *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
        } else if constexpr (sizeof(TIn) == 2) {
#pragma unroll
            for (int i = 0; i < W; i++) p[i] = uint16_t(w[i / 2] >> (16 * (i & 1)));
        } else {
#pragma unroll
            for (int i = 0; i < W; i++) p[i] = __uint_as_float(w[i]);
        }
    }
    __device__ __forceinline__ uint32_t raw(int i) const {
        if constexpr (sizeof(TIn) == 2) return (w[i / 2] >> (16 * (i & 1))) & 0xffffu;
        else return w[i];
    }
    __device__ __forceinline__ void set(int i, uint32_t v) {
        if constexpr (sizeof(TIn) == 2) w[i / 2] = (w[i / 2] & ~(0xffffu << (16 * (i & 1)))) | (v << (16 * (i & 1)));
        else w[i] = v;
    }
    __device__ __forceinline__ float f(int i) const {
        if constexpr (sizeof(TIn) == 2) return __uint_as_float(raw(i) << 16);
        else return __uint_as_float(w[i]);
    }
};

template <typename TIn>
__device__ __forceinline__ uint32_t raw_bits(const TIn* p, int64_t i) {
    if constexpr (sizeof(TIn) == 2) return uint32_t(p[i]);
    else return __float_as_uint(p[i]);
}

template <typename TIn, int W, bool VEC>
__global__ __launch_bounds__(256) void conv_update(const ConvParams p) {
    const int64_t ch = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
    if (ch >= p.b * p.d_in) return;
    const int64_t d = ch % p.d_in;
    TIn* st = static_cast<TIn*>(p.state) + ch * W;

    Window<TIn, W, VEC> win;
    win.load(st);
    // Roll by one towards index 0, newest input last.
#pragma unroll
    for (int i = 0; i + 1 < W; i++) win.set(i, win.raw(i + 1));
    win.set(W - 1, raw_bits(static_cast<const TIn*>(p.x), ch));
    win.store(st);

    const float* wd = p.weight + d * W;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < W; i++) acc = fmaf(win.f(i), wd[i], acc);
    if (p.bias) acc += p.bias[d];
    if (p.silu) acc = silu(acc);
    Elem<TIn>::store(static_cast<TIn*>(p.out), ch, acc);
}

}  // namespace ss
