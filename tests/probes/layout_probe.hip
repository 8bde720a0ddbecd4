// layout_probe.hip -- single-wave probes of gfx950 instruction semantics the
// attention kernel relies on: the lane layouts of v_mfma_f32_32x32x16_bf16
// (operands and accumulator), v_permlane32_swap, v_exp_f32 and v_log_f32.
// global_load_lds_dwordx4 (direct global->LDS copy) and ds_read_b64_tr_b16
// (transposing LDS read).  Test code only; every probe runs one wave64 over
// caller-provided buffers of the documented sizes.
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

// global_load_lds_dwordx4: lane l copies 16 bytes from src + 16*perm[l] into
// LDS at (base + 16*l); out receives the whole 4 KB LDS window (sentinel
// 0xdeadbeef where nothing was written).  base = 512 bytes.
__global__ void load_lds_kernel(const uint32_t* src, const int* perm, uint32_t* out) {
    __shared__ uint32_t sm[1024];
    const int l = threadIdx.x;
    for (int i = l; i < 1024; i += 64) sm[i] = 0xdeadbeefu;
    __syncthreads();
    const uint32_t* g = src + 4 * perm[l];
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)(sm + 128), 16, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int i = l; i < 1024; i += 64) out[i] = sm[i];
}

// ds_read_b64_tr_b16: LDS holds 16-bit values sm[i] = i (8192 of them); lane l
// reads at short index addr[l] (multiple of 4, < 8189); out[l][0..3] = result.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__global__ void read_tr_kernel(const int* addr, short* out) {
    __shared__ short sm[8192];
    for (int i = threadIdx.x; i < 8192; i += 64) sm[i] = (short)i;
    __syncthreads();
    int a = addr[threadIdx.x];
    a = (a < 0 || a > 8188) ? 0 : (a & ~3);
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    lds_v4i16* p = (lds_v4i16*)((__attribute__((address_space(3))) short*)sm + a);
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
    for (int e = 0; e < 4; ++e) out[threadIdx.x * 4 + e] = r[e];
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
__attribute__((visibility("default"))) int probe_load_lds(const void* src, const void* perm,
                                                          void* out, hipStream_t s) {
    hipLaunchKernelGGL(load_lds_kernel, dim3(1), dim3(64), 0, s, (const uint32_t*)src,
                       (const int*)perm, (uint32_t*)out);
    return (int)hipGetLastError();
}
__attribute__((visibility("default"))) int probe_read_tr(const void* addr, void* out, hipStream_t s) {
    hipLaunchKernelGGL(read_tr_kernel, dim3(1), dim3(64), 0, s, (const int*)addr, (short*)out);
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
