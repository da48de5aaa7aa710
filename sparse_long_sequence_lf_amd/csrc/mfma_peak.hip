// mfma_peak.hip -- the achievable dense bf16 MFMA rate of this GPU, for the
// benchmark's roofline (a measured ceiling beside the published one).  Not
// part of the attention library: libmfmapeak.so is loaded by the benchmark
// only.
//
// Every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on register
// operands into four independent accumulators (so no product waits for the
// one before it); 32*32*16*2 FLOPs each.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop(float* out, int iters, float seed) {
    const float x = seed + 1e-3f * (float)(threadIdx.x & 63);
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        a[i] = (__bf16)(x + 0.125f * i);
        b[i] = (__bf16)(x - 0.0625f * i);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; it++) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i++) s += c0[i] + c1[i] + c2[i] + c3[i];
    // a store the compiler cannot drop, taken only for an impossible seed
    if (seed == -1.0f) out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// FLOPs of one launch of lf_mfma_peak_launch(blocks, iters, ...)
extern "C" double lf_mfma_peak_flops(int blocks, int iters) {
    return (double)blocks * 4.0 * (double)iters * 4.0 * 32.0 * 32.0 * 16.0 * 2.0;
}

// blocks of 256 threads, iters groups of four MFMAs per wave; out is never
// written (pass any device pointer, or null)
extern "C" int lf_mfma_peak_launch(int blocks, int iters, void* out, void* stream) {
    if (blocks < 1 || iters < 1) return (int)hipErrorInvalidValue;
    mfma_loop<<<blocks, 256, 0, (hipStream_t)stream>>>((float*)out, iters, 0.5f);
    return (int)hipGetLastError();
}
