// layout_probe.hip -- single-wave probes of gfx950 instruction semantics the
// attention kernel relies on: the lane layouts of v_mfma_f32_32x32x16_bf16
// (operands and accumulator), v_permlane32_swap, v_exp_f32 and v_log_f32.
// Test code only; every probe runs one wave64 over caller-provided buffers of
// the documented sizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// a_regs, b_regs: [64 lanes][8] bf16 operand registers; acc: [64 lanes][16] fp32.
__global__ void mfma32_kernel(const bf16x8* a_regs, const bf16x8* b_regs, f32x16* acc) {
    const int l = threadIdx.x;
    f32x16 c = f32x16{};
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_regs[l], b_regs[l], c, 0, 0, 0);
    acc[l] = c;
}

// x: [64] in; lo_out/hi_out: [64] the two results of permlane32_swap(x, x).
__global__ void permlane_kernel(const uint32_t* x, uint32_t* r0, uint32_t* r1) {
    const int l = threadIdx.x;
    const uint32_t v = x[l];
    auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    r0[l] = r[0];
    r1[l] = r[1];
}

// n values: y_exp = v_exp_f32(x) (2^x), y_log = v_log_f32(x) (log2 x).
__global__ void trans_kernel(const float* x, float* y_exp, float* y_log, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        y_exp[i] = __builtin_amdgcn_exp2f(x[i]);
        y_log[i] = __builtin_amdgcn_logf(x[i]);
    }
}

extern "C" {
__attribute__((visibility("default"))) int probe_mfma32(const void* a_regs, const void* b_regs,
                                                        void* acc, hipStream_t s) {
    hipLaunchKernelGGL(mfma32_kernel, dim3(1), dim3(64), 0, s, (const bf16x8*)a_regs,
                       (const bf16x8*)b_regs, (f32x16*)acc);
    return (int)hipGetLastError();
}
__attribute__((visibility("default"))) int probe_permlane32_swap(const void* x, void* r0, void* r1,
                                                                 hipStream_t s) {
    hipLaunchKernelGGL(permlane_kernel, dim3(1), dim3(64), 0, s, (const uint32_t*)x,
                       (uint32_t*)r0, (uint32_t*)r1);
    return (int)hipGetLastError();
}
__attribute__((visibility("default"))) int probe_trans(const void* x, void* y_exp, void* y_log,
                                                       int n, hipStream_t s) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(trans_kernel, dim3((n + 255) / 256), dim3(256), 0, s, (const float*)x,
                       (float*)y_exp, (float*)y_log, n);
    return (int)hipGetLastError();
}
}
