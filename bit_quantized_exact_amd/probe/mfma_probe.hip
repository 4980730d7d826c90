// Sustained matrix-core rate of gfx950, measured with a dense MFMA loop: the
// practical ceiling the attention kernels are compared with beside the
// published peaks.  Not part of the attention path.
//
// Each wave keeps its A and B operands in registers and runs `iters` rounds of
// four independent accumulator chains (v_mfma_f32_32x32x16_f16 or
// v_mfma_i32_32x32x32_i8), so the matrix pipe never waits on a result; the
// accumulators are summed into one value per lane at the end (so the loop is
// not removed).  Two 256-thread workgroups per compute unit give two waves
// per SIMD, as in the forward kernels.  A streaming read of a large buffer
// gives the practical HBM read bandwidth the same way.
#include "mfma_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16x __attribute__((ext_vector_type(16)));
typedef int i16x __attribute__((ext_vector_type(16)));
typedef int i4x __attribute__((ext_vector_type(4)));

constexpr int kChains = 4;

__global__ __launch_bounds__(256) void mfma_loop_f16(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    h8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<_Float16>(0.001f * static_cast<float>((lane + e) & 7));
        b[e] = static_cast<_Float16>(0.001f * static_cast<float>((lane * 3 + e) & 7));
    }
    f16x acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f16x{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_loop_i8(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    i4x a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = (lane + e) & 0x03030303;
        b[e] = (lane * 3 + e) & 0x03030303;
    }
    i16x acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = i16x{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = static_cast<float>(s);
}

// Softmax-like vector work beside the FP16 loop (VALU = true, MFMA = true),
// or alone (MFMA = false): per MFMA slot one exp2 and five FMAs on four
// independent chains that never touch the MFMA registers, the mix of a tile
// of the forward's online softmax (about one exponential and five other
// vector instructions per MFMA).
template <bool MFMA>
__global__ __launch_bounds__(256) void mfma_valu_mix(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    h8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = static_cast<_Float16>(0.001f * static_cast<float>((lane + e) & 7));
        b[e] = static_cast<_Float16>(0.001f * static_cast<float>((lane * 3 + e) & 7));
    }
    f16x acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f16x{};
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = -0.001f * static_cast<float>(lane + c);
    const float k0 = 0.999f, k1 = -0.0001f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            if constexpr (MFMA) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
            float y = __builtin_amdgcn_exp2f(x[c]);
#pragma unroll
            for (int f = 0; f < 5; ++f) y = __builtin_fmaf(y, k0, k1);
            x[c] = __builtin_fminf(y, 0.0f) * 0.5f - 0.25f;
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        s += x[c];
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    }
    sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// One pass over n16 16-byte chunks: thread t of the grid reads chunks
// t, t + T, t + 2T, ... (T threads in all), four loads in flight per round,
// with the non-temporal (streaming) cache policy.
__global__ __launch_bounds__(256) void hbm_read(const i4x* __restrict__ p, unsigned long long n16,
                                                float* __restrict__ sink) {
    const unsigned long long T = static_cast<unsigned long long>(gridDim.x) * blockDim.x;
    unsigned long long i = static_cast<unsigned long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    i4x x = {0, 0, 0, 0};
    for (; i + 3 * T < n16; i += 4 * T) {
        const i4x a = __builtin_nontemporal_load(p + i), b = __builtin_nontemporal_load(p + i + T);
        const i4x c = __builtin_nontemporal_load(p + i + 2 * T), d = __builtin_nontemporal_load(p + i + 3 * T);
        x ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += T) x ^= __builtin_nontemporal_load(p + i);
    sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] =
        static_cast<float>(x[0] ^ x[1] ^ x[2] ^ x[3]);
}

}  // namespace

extern "C" int attn_probe_hbm_read(const void* buf, unsigned long long bytes, int blocks, float* sink,
                                   void* stream) {
    if (!buf || !sink || blocks <= 0 || bytes == 0 || bytes % 16 != 0 ||
        reinterpret_cast<unsigned long long>(buf) % 16 != 0)
        return -1;
    hipLaunchKernelGGL(hbm_read, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const i4x*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int attn_probe_mfma(int kind, int blocks, int iters, float* sink, double* ops, void* stream) {
    if (kind < 0 || kind > 3 || blocks <= 0 || iters <= 0 || !sink) return -1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (kind == 0)
        hipLaunchKernelGGL(mfma_loop_f16, dim3(blocks), dim3(256), 0, st, iters, sink);
    else if (kind == 1)
        hipLaunchKernelGGL(mfma_loop_i8, dim3(blocks), dim3(256), 0, st, iters, sink);
    else if (kind == 2)
        hipLaunchKernelGGL(mfma_valu_mix<true>, dim3(blocks), dim3(256), 0, st, iters, sink);
    else
        hipLaunchKernelGGL(mfma_valu_mix<false>, dim3(blocks), dim3(256), 0, st, iters, sink);
    if (ops) {
        // per MFMA: 2 * 32 * 32 * K operations (K = 16 fp16, 32 int8); kinds 2
        // and 3 count the FP16 MFMAs of kind 2 (kind 3 issues none)
        const double per = 2.0 * 32.0 * 32.0 * (kind == 1 ? 32.0 : 16.0);
        *ops = per * kChains * static_cast<double>(iters) * (static_cast<double>(blocks) * 4.0);
    }
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int attn_probe_compute_units(int* cus) {
    int dev = 0;
    if (!cus || hipGetDevice(&dev) != hipSuccess) return -1;
    return hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? 0 : -3;
}
