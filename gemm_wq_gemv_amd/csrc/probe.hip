// Read-bandwidth probe: a kernel that only streams bytes from HBM, the
// achievable ceiling the bandwidth-bound kernels of this library are measured
// against (a plain read of the same number of bytes, with the same 128-bit
// non-temporal loads the GEMVs use).  Not part of any product: a measurement
// hook, reached through wq_read_probe.
//
// Workgroups of 4 waves read U slabs of 4 KiB each (16 KiB for U = 4, the
// f16 GEMV's row block at K = 2048): lane l of wave w loads chunk w * 64 + l of
// every slab, so each load instruction covers 1 KiB contiguously.  Full
// workgroups load unconditionally (guarded loads measured 4-6 % slower on
// MI355X at 331-622 MB); only the last workgroup checks the end.  Each lane
// XORs its chunks and stores only if the result hits a fixed value, so the
// loads cannot be dropped and in practice nothing is written.  One slab block
// per workgroup, no grid stride.
#include "wq_internal.h"

#include <cstdio>

namespace wq {
namespace {

constexpr int kProbeLanes = 256;                 // 4 waves
constexpr int kSlabChunks = kProbeLanes;         // 16-byte chunks per 4 KiB slab
constexpr uint32_t kProbeMagic = 0x9e3779b9u;

template <int U, bool FULL>
__global__ __launch_bounds__(kProbeLanes) void read_probe(const uint4 *__restrict__ p, int64_t chunks,
                                                          int64_t first_block, uint32_t *__restrict__ out) {
    const int64_t blk = first_block + blockIdx.x;
    const int64_t base = blk * U * kSlabChunks + threadIdx.x;
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * kSlabChunks;
        v[u] = (FULL || i < chunks) ? load_nt16(p + i) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    if (x == kProbeMagic) out[blk] = x;  // one dword per workgroup of 16 KiB * U / 4 read
}

template <int U>
hipError_t launch_u(const uint4 *q, int64_t chunks, uint32_t *out, hipStream_t s) {
    const int64_t per = static_cast<int64_t>(U) * kSlabChunks;
    const int64_t full = chunks / per, tail = chunks % per != 0;
    if (full + tail > 0x7fffffffLL) return hipErrorInvalidValue;
    if (trace_enabled())
        fprintf(stderr, "[wqmm] read_probe<U=%d> chunks=%lld full=%lld tail=%lld block=%d\n", U, (long long)chunks,
                (long long)full, (long long)tail, kProbeLanes);
    if (full > 0)
        hipLaunchKernelGGL((read_probe<U, true>), dim3(static_cast<unsigned>(full)), dim3(kProbeLanes), 0, s, q,
                           chunks, int64_t{0}, out);
    if (tail)
        hipLaunchKernelGGL((read_probe<U, false>), dim3(1), dim3(kProbeLanes), 0, s, q, chunks, full, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_read_probe(const void *p, int64_t bytes, uint32_t *out, int variant, hipStream_t s) {
    const int64_t chunks = bytes / 16;
    if (chunks == 0) return hipSuccess;
    const uint4 *q = static_cast<const uint4 *>(p);
    switch (variant) {  // 4 KiB slabs per workgroup: 1, 2, 4 or 8
        case 0: return launch_u<1>(q, chunks, out, s);
        case 1: return launch_u<2>(q, chunks, out, s);
        case 2: return launch_u<4>(q, chunks, out, s);
        default: return launch_u<8>(q, chunks, out, s);
    }
}

}  // namespace wq
