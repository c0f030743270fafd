// Weight preparation on the GPU (done once, at load time):
//  * f32 -> binary16, round to nearest even (f32_to_f16 / make_buffer_f16,
//    lattice-inference 0.1.2, metal_qwen35.rs).  v_cvt_f16_f32 rounds to
//    nearest even in the default mode and keeps f16 subnormals; f32
//    subnormals lie far below half the smallest f16 subnormal and give +-0.
//  * f32 -> Q8_0 blocks (quantize_row_q8_0 / make_buffer_q8_0, same page),
//    every step in f32 as on the page: amax = max |v|, d = amax / 127,
//    id = 1 / d (0 when d == 0), scale bytes = f16(d) little-endian,
//    q = clamp(round(v * id), -127, 127), round() taking halves away from zero.
//    HIP compiles f32 division correctly rounded, so d and id are the IEEE
//    quotients; v * id is a single rounded product (nothing to contract).
#include "wq_internal.h"

namespace wq {
namespace {

__device__ __forceinline__ uint16_t f32_to_half_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

__global__ __launch_bounds__(256) void pack_f16_kernel(const float *__restrict__ w, uint16_t *__restrict__ out,
                                                       int64_t count) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride)
        out[i] = f32_to_half_bits(w[i]);
}

// One thread per 32-value block.
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const float *__restrict__ w, uint8_t *__restrict__ out,
                                                            int64_t nblocks) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t blk = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; blk < nblocks; blk += stride) {
        const float *v = w + blk * 32;
        float x[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = v[i];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
        const float d = amax / 127.0f;
        const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        uint16_t *o16 = reinterpret_cast<uint16_t *>(out + blk * 34);  // blocks are 2-byte aligned
        o16[0] = f32_to_half_bits(d);                                  // little-endian scale
#pragma unroll
        for (int i = 0; i < 32; i += 2) {
            int q[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const float t = roundf(x[i + u] * id);
                q[u] = (t != t) ? 0 : static_cast<int>(fminf(fmaxf(t, -127.0f), 127.0f));
            }
            o16[1 + i / 2] = static_cast<uint16_t>((q[0] & 0xff) | ((q[1] & 0xff) << 8));
        }
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ c, int64_t count) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) c[i] = 0.f;
}

int64_t grid_for(int64_t items) {
    const int64_t g = (items + 255) / 256;
    return g < 65536 ? (g > 0 ? g : 1) : 65536;
}

}  // namespace

hipError_t launch_pack_f16(const float *w, uint16_t *out, int64_t count, hipStream_t s) {
    hipLaunchKernelGGL(pack_f16_kernel, dim3(grid_for(count)), dim3(256), 0, s, w, out, count);
    return hipGetLastError();
}

hipError_t launch_quantize_q8_0(const float *w, uint8_t *out, int64_t count, hipStream_t s) {
    const int64_t nblocks = count / 32;
    hipLaunchKernelGGL(quantize_q8_0_kernel, dim3(grid_for(nblocks)), dim3(256), 0, s, w, out, nblocks);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float *c, int64_t count, hipStream_t s) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(count)), dim3(256), 0, s, c, count);
    return hipGetLastError();
}

}  // namespace wq
