// Read-bandwidth probe: a kernel that only streams bytes from HBM, the
// achievable ceiling the bandwidth-bound kernels of this library are measured
// against (a plain read of the same number of bytes, with the same 128-bit
// non-temporal loads the GEMVs use).  Not part of any product: a measurement
// hook, reached through wq_read_probe.
//
// Workgroups of 256 lanes; lane l of workgroup g reads 16-byte chunks
// g * 256 * U + u * 256 + l for u < U (every load instruction coalesced over
// 4 KiB), XORs them and each wave writes one dword, so the loads cannot be
// dropped and the writes are one dword per 1 KiB * U read.  One block per
// workgroup, no grid stride, as in the f16 GEMV.
#include "wq_internal.h"

#include <cstdio>

namespace wq {
namespace {

template <int U>
__global__ __launch_bounds__(256) void read_probe(const uint4 *__restrict__ p, int64_t chunks,
                                                  uint32_t *__restrict__ out) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * U + threadIdx.x;
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + u * 256;
        v[u] = i < chunks ? load_nt16(p + i) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), d, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) out[(static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) / kWave] = x;
}

}  // namespace

hipError_t launch_read_probe(const void *p, int64_t bytes, uint32_t *out, int variant, hipStream_t s) {
    const int64_t chunks = bytes / 16;
    const int u = 1 << variant;  // chunks per lane: 1, 2, 4 or 8
    const int64_t blocks = (chunks + 256LL * u - 1) / (256LL * u);
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (trace_enabled())
        fprintf(stderr, "[wqmm] read_probe<U=%d> bytes=%lld grid=%lld block=256\n", u, (long long)bytes,
                (long long)blocks);
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    const uint4 *q = static_cast<const uint4 *>(p);
    switch (variant) {
        case 0: hipLaunchKernelGGL(read_probe<1>, grid, block, 0, s, q, chunks, out); break;
        case 1: hipLaunchKernelGGL(read_probe<2>, grid, block, 0, s, q, chunks, out); break;
        case 2: hipLaunchKernelGGL(read_probe<4>, grid, block, 0, s, q, chunks, out); break;
        default: hipLaunchKernelGGL(read_probe<8>, grid, block, 0, s, q, chunks, out); break;
    }
    return hipGetLastError();
}

}  // namespace wq
