// Internal declarations shared by the libwqmm translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

// ----------------------------------------------------------------- device --
// Wavefront size on CDNA4.
constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 128-bit non-temporal (streaming) global load: weights are read exactly once.
__device__ __forceinline__ uint4 load_nt16(const uint4 *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left free).  Used once after loads
// whose registers stay live across a loop that issues newer loads, so the
// compiler does not re-wait for them inside the loop.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// binary16 bits -> f32, exact (the hardware conversion keeps subnormals).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of G lanes (G a power of two up to 64); every lane
// of a group receives the group's sum.  Within a 16-lane DPP row:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror;
// across rows: lane xor 16 and 32.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group size");
    if constexpr (G >= 2) v += dpp_f32<0xb1>(v);
    if constexpr (G >= 4) v += dpp_f32<0x4e>(v);
    if constexpr (G >= 8) v += dpp_f32<0x141>(v);
    if constexpr (G >= 16) v += dpp_f32<0x140>(v);
    if constexpr (G >= 32) v += __shfl_xor(v, 16, kWave);
    if constexpr (G >= 64) v += __shfl_xor(v, 32, kWave);
    return v;
}

// The value of a partner lane that differs from this one in bit log2(H) and is
// a perfect matching of the lanes with that bit clear to those with it set
// (lane xor H for H >= 8; the DPP mirrors pair lanes inside a row).
template <int H>
__device__ __forceinline__ float bit_partner(float v) {
    if constexpr (H == 32 || H == 16) return __shfl_xor(v, H, kWave);
    else if constexpr (H == 8) return dpp_f32<0x128>(v);  // row_ror:8
    else if constexpr (H == 4) return dpp_f32<0x141>(v);  // row_half_mirror
    else if constexpr (H == 2) return dpp_f32<0x4e>(v);
    else return dpp_f32<0xb1>(v);
}

// N row sums per lane, reduced over aligned groups of G lanes (N <= G, both
// powers of two).  Each butterfly step pairs lanes across the group's top
// bit; the lane with the bit set keeps the upper half of the rows, adds its
// partner's copy of them, and the number of values halves.  Afterwards lane
// g of a group (g = lane % G) holds the complete sum of row g / (G / N).
template <int N, int G>
__device__ __forceinline__ float rows_sum(const float (&v)[N], int g) {
    if constexpr (N == 1) {
        return group_sum<G>(v[0]);
    } else {
        constexpr int H = G / 2;
        const bool hi = (g & H) != 0;
        float w[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float send = hi ? v[i] : v[N / 2 + i];
            const float keep = hi ? v[N / 2 + i] : v[i];
            w[i] = keep + bit_partner<H>(send);
        }
        return rows_sum<N / 2, H>(w, g);
    }
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// SiLU as on the pages' silu_mul kernel: x / (1 + e^-x), in f32.
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Epilogues (the values of wq_epilogue in wqmm.h).  Residual: C += A.B^T.
// GLU: the weights hold 2*NO rows (gate rows, then up rows) and
// C[m, j] = silu(g) * u for the gate sum g (row j) and up sum u (row NO + j).
constexpr int kEpiNone = 0, kEpiResidual = 1, kEpiGlu = 2;

// ------------------------------------------------------------------- host --
struct DeviceInfo {
    int cus;  // compute units of the current device
};
// Properties of the current HIP device, queried once per device.
hipError_t device_info(DeviceInfo *out);

// Launchers.  Arguments are already validated by the C-ABI layer; these only
// pick a kernel variant and grid and enqueue it on `s`.
// GEMV epilogue epi: kEpiNone, kEpiResidual (c[n] += the dot product) or
// kEpiGlu (n outputs from 2n weight rows: c[j] = silu(row j) * row n + j).
hipError_t launch_gemv_f16(const float *a, const uint16_t *b, float *c, int64_t n, int64_t k,
                           hipStream_t s, int epi = kEpiNone);
hipError_t launch_gemv_q4_0(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k,
                            hipStream_t s, int epi = kEpiNone);
hipError_t launch_gemv_q8_0(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k,
                            hipStream_t s, int epi = kEpiNone);
// n = output columns; with kEpiGlu the weights have 2n rows.
hipError_t launch_gemm(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n,
                       int64_t k, hipStream_t s, int epi = kEpiNone);
// Small-M weight-streaming product (M <= 16 rows of A per launch).
hipError_t launch_skinny(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t s, int epi = kEpiNone);
// C [m, no] from split partial sums [splits][m][nw] summed in split order,
// then the epilogue (nw = no, or 2 * no for kEpiGlu: gate then up columns).
hipError_t launch_reduce_splits(const float *partial, float *c, int64_t m, int64_t no, int64_t nw, int splits,
                                int epi, hipStream_t s);
// Tile shape and K-split count the GEMM picks for a problem on `cus` CUs.
void gemm_plan(int64_t m, int64_t n, int64_t k, int fmt, int cus, int *bm, int *bn, int *splits);
// Test hook: force the GEMM tiling (bm, bn from the compiled set; splits >= 1,
// capped at the number of k-tiles); (0, 0, 0) clears it.  False if unknown.
bool set_gemm_plan_override(int bm, int bn, int splits);
hipError_t launch_fill_zero(float *c, int64_t count, hipStream_t s);
hipError_t launch_pack_f16(const float *w, uint16_t *out, int64_t count, hipStream_t s);
hipError_t launch_quantize_q8_0(const float *w, uint8_t *out, int64_t count, hipStream_t s);

// Split-K scratch.  One buffer per device, grown on demand from the device's
// default memory pool (stream-ordered) and kept for reuse; a lease holds the
// device's lock from acquire() until the kernels that use the buffer are
// enqueued, then records an event on the stream, and the next lease waits on
// that event from its own stream, so uses on different streams never overlap.
// Requests above kScratchCacheBytes take a private stream-ordered allocation.
constexpr size_t kScratchCacheBytes = size_t(256) << 20;
class ScratchLease {
  public:
    ScratchLease() = default;
    ScratchLease(const ScratchLease &) = delete;
    ScratchLease &operator=(const ScratchLease &) = delete;
    ~ScratchLease();
    // Gives *ptr with at least `bytes` bytes usable by work enqueued on `s`.
    hipError_t acquire(size_t bytes, hipStream_t s, void **ptr);
    // After the last kernel using the buffer is enqueued on `s`.
    hipError_t release();

  private:
    int dev_ = -1;
    hipStream_t s_ = nullptr;
    void *priv_ = nullptr;  // private allocation (large requests)
    bool held_ = false;     // device lock held
};

// Set by WQ_TRACE=1: one line per launch on stderr.
bool trace_enabled();

}  // namespace wq
