// Host stand-in for the parts of the HIP device and runtime API that the
// library's sources use, so that the kernels can be compiled for the CPU and
// run there (tests/kernel_host/emu.cpp): every work-item is a host thread,
// workgroups run one after another, LDS is a host buffer whose bytes past
// the launch's dynamic size are poisoned for AddressSanitizer, and every
// global buffer is allocated at its exact size.  Direct-to-LDS loads copy at
// once; waits on them are no-ops.  Cross-lane operations exchange values
// through a per-wave buffer between two wave barriers, so all 64 lanes of a
// wave must take part (as the hardware requires of them).
#pragma once

#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <tuple>
#include <type_traits>

#define __global__
#define __device__
#define __host__
#define __shared__ static   // the one static __shared__ array: one copy, workgroups run in turn
#define __forceinline__ inline __attribute__((always_inline))
#define __launch_bounds__(...)
#define __align__(n) __attribute__((aligned(n)))

// ----------------------------------------------------------------- runtime

typedef int hipError_t;
typedef void* hipStream_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount = 0 };

struct dim3 {
    unsigned x, y, z;
    constexpr dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};

namespace emu {
extern thread_local dim3 tl_thread, tl_block, tl_bdim, tl_gdim;
extern thread_local int tl_lane;
hipError_t get_device(int* dev);
hipError_t device_attribute(int* v, int attr, int dev);
hipError_t occupancy(int* nb, const void* fn, int threads, size_t lds);
hipError_t symbol_address(void** p, const void* sym);
void run_grid(dim3 grid, dim3 block, size_t lds, void (*body)(void*), void* ctx);
void block_barrier();
void wave_barrier();
void sleep_a_little();
unsigned char* lds_base();

template <typename F, typename... A>
struct LaunchCtx {
    F fn;
    std::tuple<A...> args;
};

template <typename F, typename... A>
void launch(F fn, dim3 grid, dim3 block, size_t lds, A... args) {
    LaunchCtx<F, A...> ctx{fn, std::tuple<A...>(args...)};
    run_grid(grid, block, lds, [](void* c) {
        auto* x = static_cast<LaunchCtx<F, A...>*>(c);
        std::apply(x->fn, x->args);
    }, &ctx);
}
}  // namespace emu

#define threadIdx (emu::tl_thread)
#define blockIdx (emu::tl_block)
#define blockDim (emu::tl_bdim)
#define gridDim (emu::tl_gdim)

inline hipError_t hipGetLastError() { return hipSuccess; }
inline hipError_t hipGetDevice(int* d) { return emu::get_device(d); }
inline hipError_t hipDeviceGetAttribute(int* v, int attr, int dev) { return emu::device_attribute(v, attr, dev); }
inline hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* nb, const void* fn, int threads, size_t lds) {
    return emu::occupancy(nb, fn, threads, lds);
}
template <typename F>
inline hipError_t hipOccupancyMaxActiveBlocksPerMultiprocessor(int* nb, F fn, int threads, size_t lds) {
    return emu::occupancy(nb, reinterpret_cast<const void*>(fn), threads, lds);
}
inline hipError_t hipGetSymbolAddress(void** p, const void* sym) { return emu::symbol_address(p, sym); }
#define HIP_SYMBOL(x) (&(x))
#define hipLaunchKernelGGL(fn, grid, block, lds, stream, ...) emu::launch(fn, dim3(grid), dim3(block), size_t(lds), __VA_ARGS__)

// ----------------------------------------------------------------- vector types

struct float2 { float x, y; };
struct float4 { float x, y, z, w; };
struct uint2 { unsigned x, y; };
struct uint4 { unsigned x, y, z, w; };
inline float2 make_float2(float a, float b) { return {a, b}; }
inline float4 make_float4(float a, float b, float c, float d) { return {a, b, c, d}; }
inline uint2 make_uint2(unsigned a, unsigned b) { return {a, b}; }
inline uint4 make_uint4(unsigned a, unsigned b, unsigned c, unsigned d) { return {a, b, c, d}; }

inline float __uint_as_float(unsigned u) { return __builtin_bit_cast(float, u); }
inline unsigned __float_as_uint(float f) { return __builtin_bit_cast(unsigned, f); }
inline float __int_as_float(int u) { return __builtin_bit_cast(float, u); }
inline int __float_as_int(float f) { return __builtin_bit_cast(int, f); }
inline unsigned __umulhi(unsigned a, unsigned b) { return unsigned((uint64_t(a) * b) >> 32); }

template <typename A, typename B>
inline auto min(A a, B b) -> std::common_type_t<A, B> { return a < b ? a : b; }
template <typename A, typename B>
inline auto max(A a, B b) -> std::common_type_t<A, B> { return a > b ? a : b; }

// ----------------------------------------------------------------- device builtins

struct emu_rsrc {
    const unsigned char* base;
    uint32_t bytes;
};
#define __amdgpu_buffer_rsrc_t emu_rsrc

namespace emu {
void global_load_lds(const void* src, void* lds_dst, int bytes);
void buffer_load_lds(emu_rsrc r, uintptr_t lds_off, int bytes, uint32_t voff, uint32_t soff, uint32_t off);
uint32_t buffer_load(emu_rsrc r, uint32_t voff, uint32_t soff, int bytes);
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
u32x2 permlane32_swap(unsigned a, unsigned b);
u32x2 permlane16_swap(unsigned a, unsigned b);
int update_dpp(int old, int src, int ctrl, int row_mask, int bank_mask, bool bound_ctrl);
float shfl_xor(float v, int mask, int width);
float shfl(float v, int src, int width);
}  // namespace emu

#define __builtin_amdgcn_readfirstlane(x) (x)
#define __builtin_amdgcn_s_barrier() emu::block_barrier()
#define __builtin_amdgcn_wave_barrier() emu::wave_barrier()
#define __syncthreads() emu::block_barrier()
#define __builtin_amdgcn_s_waitcnt(x) ((void)(x))
#define __builtin_amdgcn_s_sleep(x) emu::sleep_a_little()
#define __builtin_amdgcn_fence(...) std::atomic_thread_fence(std::memory_order_seq_cst)
#define __builtin_amdgcn_exp2f(x) ::exp2f(x)
#define __builtin_amdgcn_logf(x) ::log2f(x)
#define __builtin_amdgcn_rcpf(x) (1.0f / (x))
#define __builtin_amdgcn_groupstaticsize() 0u
#define __builtin_amdgcn_global_load_lds(src, dst, bytes, off, aux) emu::global_load_lds((src), emu::lds_base() + (uintptr_t)(dst), (bytes))
#define __builtin_amdgcn_make_buffer_rsrc(p, stride, bytes, flags) \
    emu_rsrc{static_cast<const unsigned char*>(static_cast<const void*>(p)), uint32_t(bytes)}
#define __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, bytes, voff, soff, off, aux) \
    emu::buffer_load_lds((r), (uintptr_t)(dst), (bytes), (voff), (soff), (off))
#define __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, aux) emu::buffer_load((r), uint32_t(voff), uint32_t(soff), 4)
#define __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, aux) ((unsigned short)emu::buffer_load((r), uint32_t(voff), uint32_t(soff), 2))
#define __builtin_amdgcn_permlane32_swap(a, b, fi, bc) emu::permlane32_swap((a), (b))
#define __builtin_amdgcn_permlane16_swap(a, b, fi, bc) emu::permlane16_swap((a), (b))
#define __builtin_amdgcn_update_dpp(old, src, ctrl, rm, bm, bc) emu::update_dpp((old), (src), (ctrl), (rm), (bm), (bc))
#define __shfl_xor(v, m, w) emu::shfl_xor((v), (m), (w))
#define __shfl(v, s, w) emu::shfl((v), (s), (w))

#define __HIP_MEMORY_SCOPE_AGENT 0
#define __HIP_MEMORY_SCOPE_WORKGROUP 0
#define __hip_atomic_load(p, order, scope) __atomic_load_n((p), __ATOMIC_SEQ_CST)
#define __hip_atomic_store(p, v, order, scope) __atomic_store_n((p), (v), __ATOMIC_SEQ_CST)
inline unsigned atomicAdd(unsigned* p, unsigned v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }
inline unsigned atomicOr(unsigned* p, unsigned v) { return __atomic_fetch_or(p, v, __ATOMIC_SEQ_CST); }
