// Calibration kernels for the rooflines.
//
// Matrix-core calibration: the rate at which this GPU sustains the attention
// kernel's MFMA instruction (v_mfma_f32_32x32x16_bf16) at the clock it holds
// under that load. The roofline's peak is the vendor's dense bf16 figure at
// the nominal clock; under a sustained MFMA load the chip lowers its clock to
// stay within its power limit, so the attainable rate sits below it. This
// kernel measures that rate with the attention kernel's occupancy (one
// workgroup of 8 waves per CU, two waves per SIMD) and the same instruction
// mix of its MFMAs: per step, 16 MFMAs into two score blocks and 16 into four
// output blocks, operands in registers holding nonzero bf16 values (operands
// of zero draw less power and would overstate the rate). No memory traffic,
// no softmax: an upper bound for the attention kernel at that clock.
#include <hip/hip_runtime.h>

#include "wf_internal.h"

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8 lane_values(uint32_t seed) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // a small integer hash -> a bf16 value in (-1, 1), never zero
        uint32_t h = (seed + (uint32_t)i) * 2654435761u;
        h ^= h >> 15;
        const float f = ((float)(h & 0xFFFF) + 0.5f) / 32768.f - 1.f;
        v[i] = (__bf16)f;
    }
    return v;
}

__global__ __launch_bounds__(512, 1) void mfma_calibrate_kernel(int32_t steps, float* out) {
    const uint32_t id = blockIdx.x * 512u + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = lane_values(id * 64u + 16u * i);
        b[i] = lane_values(id * 64u + 16u * i + 8u);
    }
    f32x16 s0 = {}, s1 = {}, o[4] = {};
    for (int t = 0; t < steps; ++t) {
        // 16 MFMAs into two score blocks (a QK^T tile), 16 into four output
        // blocks (a PV tile), as one attention step issues them
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k & 3], b[(k + 1) & 3], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 2) & 3], b[k & 3], s1, 0, 0, 0);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int d = 0; d < 4; ++d) o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[d], b[g], o[d], 0, 0, 0);
    }
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) acc += s0[j] + s1[j] + o[0][j] + o[1][j] + o[2][j] + o[3][j];
    out[id] = acc;                                   // keeps every MFMA live
}

// HBM streaming copy: the rate this GPU moves a byte count between two
// device buffers (half read, half written) when the kernel does nothing else,
// for the publish kernels' rooflines (their traffic is such a read/write mix).
// Each thread copies two 16-byte vectors, loaded non-temporally (each byte is
// read once) and stored plainly: on gfx950 this form measured fastest (four
// or eight vectors per thread, cached loads or non-temporal stores slower).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 512 + threadIdx.x;
    u32x4 v0, v1;
    if (i < n) v0 = __builtin_nontemporal_load(src + i);
    if (i + 256 < n) v1 = __builtin_nontemporal_load(src + i + 256);
    if (i < n) dst[i] = v0;
    if (i + 256 < n) dst[i + 256] = v1;
}

}  // namespace

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, hipStream_t st) {
    const int64_t n = bytes / 16;
    const int64_t blocks = (n + 511) / 512;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    return hipGetLastError();
}

hipError_t launch_mfma_calibrate(int32_t blocks, int32_t steps, float* out, hipStream_t st) {
    hipLaunchKernelGGL(mfma_calibrate_kernel, dim3(blocks), dim3(512), 0, st, steps, out);
    return hipGetLastError();
}

}  // namespace wf
