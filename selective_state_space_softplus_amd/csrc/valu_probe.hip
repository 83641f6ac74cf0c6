// valu_probe.hip -- issue-rate probe for the VALU roofline (libss_probe.so, a
// measurement aid beside the library; nothing in libss_scan.so uses it).
//
// Every work-item runs `iters` iterations of 8 independent dependence chains
// of one instruction mix; the caller times the launch and divides by the
// number of lane-instructions issued:
//   mix 0: x = fma(x, a, b)            one v_fma_f32 per step
//   mix 1: x = x * a                   one v_mul_f32 per step
//   mix 2: x = exp2(x) * 0.5           one v_exp_f32 and one v_mul_f32 per step
//   mix 3: x = exp2(-x)                one v_exp_f32 per step (the negation is a
//                                      free source modifier)
// The ratio of mix 3's time to mix 1's gives the issue cost of v_exp_f32 in
// units of an ordinary fp32 VALU instruction; mix 2 shows it mixed with other
// work.  The chains stay in (0, 1], and their sum is stored only under a
// condition that never holds, so nothing is optimised away.
#include <hip/hip_runtime.h>

template <int MIX>
__global__ __launch_bounds__(256) void valu_probe(float* out, int iters, float a, float b) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; i++) x[i] = 0.5f + 1e-3f * float(threadIdx.x & 63) + 1e-4f * float(i);
    for (int it = 0; it < iters; it++) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if constexpr (MIX == 0) x[i] = fmaf(x[i], a, b);
            else if constexpr (MIX == 1) x[i] = x[i] * a;
            else if constexpr (MIX == 2) x[i] = __builtin_amdgcn_exp2f(x[i]) * 0.5f;
            else x[i] = __builtin_amdgcn_exp2f(-x[i]);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) s += x[i];
    if (s == -1.0f) out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Launches `blocks` workgroups of 256 work-items of mix `mix` on `stream`.
// Returns 0, -1 for an argument out of range, -6 if the launch failed.
extern "C" __attribute__((visibility("default"))) int ss_probe_valu(int mix, int blocks, int iters, float* out,
                                                                   void* stream) {
    if (mix < 0 || mix > 3 || blocks <= 0 || iters <= 0 || !out) return -1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const float a = 0.9999f, b = 1e-5f;
    if (mix == 0) hipLaunchKernelGGL(valu_probe<0>, dim3(blocks), dim3(256), 0, st, out, iters, a, b);
    else if (mix == 1) hipLaunchKernelGGL(valu_probe<1>, dim3(blocks), dim3(256), 0, st, out, iters, a, b);
    else if (mix == 2) hipLaunchKernelGGL(valu_probe<2>, dim3(blocks), dim3(256), 0, st, out, iters, a, b);
    else hipLaunchKernelGGL(valu_probe<3>, dim3(blocks), dim3(256), 0, st, out, iters, a, b);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
