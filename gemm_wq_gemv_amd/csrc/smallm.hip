// Small-M product for Q8_0 / Q4_0 weights (1 <= M <= 16): C[M,N] = A[M,K] . B[N,K]^T
// with every weight streamed from HBM once, through the fp32 matrix cores.
//
// Operation: the M > 1 branch of dispatch_gemm_q8 / dispatch_gemm_q4
// (lattice-inference 0.9.0, dispatch.rs); its prior art on the pages is the
// multi-row kernel gemm_q8 (lattice-inference 0.1.2, metal_qwen35.rs).  For
// M <= 16 the product is a weight stream: a few activation rows meet every
// weight once, so the design copies the decode GEMV's byte stream and puts the
// few rows of A on the matrix cores.
//
// CDNA4 design:
//  * A workgroup owns R = 4 * NT weight rows; its W waves take the K steps
//    (16 quantized blocks, 512 columns each) round-robin.  For one step a wave
//    copies the R row pieces -- R * 16 blocks, contiguous 16-byte aligned byte
//    ranges when K % 256 == 0 -- into its own LDS region with coalesced
//    128-bit loads (the next step's loads are in flight while this one is
//    decoded), as the staged GEMV does.
//  * Matrix op: v_mfma_f32_4x4x1_16b_f32, sixteen independent 4x4 blocks.
//    Lane (b, c) = (lane / 4, lane % 4) takes whole quantized block b of the
//    step in weight row 4 t + c of tile t (read from LDS as its dword-aligned
//    window, realigned by a byte permute) and the 32 activations of that block
//    in row 4 mb + c of A: the 32 codes of one block are 32 rank-1 steps with
//    one scale, so the matrix core accumulates sum_i q_i a_i with the raw codes
//    and the lane applies d once per block (acc += d * T), the order the pages
//    use (d * sum q a).  Every lane's accumulator column is its own weight row,
//    so the scale is the lane's own.
//  * At the end the 16 blocks are summed (DPP row rotations, cross-row
//    swizzles), the W waves through LDS in wave order, and, when K is split
//    across workgroups as well, partial tiles go to scratch and reduce_splits
//    sums them in split order.  Deterministic.
// Requires K % 256 == 0 and 16-byte aligned a and b.
#include "wq_internal.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>

namespace wq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

enum { SM_Q8_0 = 1, SM_Q4_0 = 2 };

template <int FMT>
struct SmFmt {
    static constexpr int kBytes = FMT == SM_Q8_0 ? 34 : 18;  // block bytes
    static constexpr int kCodeDw = FMT == SM_Q8_0 ? 8 : 4;   // code dwords of a block
    static constexpr int kStepBytes = 16 * kBytes;           // one row's bytes per step
    static constexpr int kStepChunks = kStepBytes / 16;      // 34 or 18
};

// Code e (0..31) of a block as f32: Q8_0 the int8 code, Q4_0 the nibble
// value u - 8 (byte e / 2, low nibble for even e).
template <int FMT>
__device__ __forceinline__ float code_value(const uint32_t (&cw)[SmFmt<FMT>::kCodeDw], int e) {
    if constexpr (FMT == SM_Q8_0) {
        return static_cast<float>(static_cast<int8_t>((cw[e >> 2] >> (8 * (e & 3))) & 0xffu));
    } else {
        const uint32_t byte = (cw[e >> 3] >> (8 * ((e >> 1) & 3))) & 0xffu;
        return static_cast<float>(static_cast<int>((e & 1) ? (byte >> 4) : (byte & 0xfu)) - 8);
    }
}

// Raw, untyped buffer resource over [p, p + bytes) (bytes capped at 4 GiB - 1).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t sm_rsrc(const void *p, uint64_t bytes) {
    const uint32_t n = (bytes >> 32) != 0 ? 0xffffffffu : static_cast<uint32_t>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(n), 0x00020000);
}
constexpr int kSmStream = 2;  // non-temporal: every weight is read once

// Sum over the 16 blocks (lanes with equal lane % 4): rotations by 4 and 8
// inside each 16-lane row, then across rows.
__device__ __forceinline__ float block_sum16(float v) {
    v += dpp_f32<0x124>(v);  // row_ror:4
    v += dpp_f32<0x128>(v);  // row_ror:8
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    return v;
}

// Workgroup (grp, split) = (blockIdx.x % groups, blockIdx.x / groups) owns
// weight rows [R * grp, R * grp + R) and steps [split * sps, min(nsteps,
// (split + 1) * sps)); wave w takes steps w, w + W, ... of that range.  With
// mode kStore the sums go to C [M, N], kAdd adds them to C (residual), kPartial
// writes them raw to out + split * M * N for reduce_splits.
enum { kStore = 0, kAdd = 1, kPartial = 2 };

template <int FMT, int MB, int NT, int W>
__global__ __launch_bounds__(W * 64) void gemm_smallm(const float *__restrict__ a, const uint8_t *__restrict__ b,
                                                      float *__restrict__ out, int64_t M, int64_t N, int64_t K,
                                                      int groups, int sps, int mode) {
    using F = SmFmt<FMT>;
    constexpr int R = 4 * NT;
    constexpr int SBY = F::kStepBytes, CPR = F::kStepChunks;
    constexpr int CH = R * CPR;                  // chunks of a full step
    constexpr int LPL = (CH + kWave - 1) / kWave;  // loads per lane and step
    constexpr int NV = MB * NT * 4;              // accumulator values per lane
    extern __shared__ uint4 smem4[];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int bl = lane >> 2, c = lane & 3;
    const int grp = static_cast<int>(blockIdx.x % groups), sp = static_cast<int>(blockIdx.x / groups);
    const int64_t row0 = static_cast<int64_t>(grp) * R;
    const int64_t rows_left = N - row0;
    const int nb = static_cast<int>(K >> 5);
    const int nsteps = (nb + 15) >> 4;
    const int s0 = sp * sps, s1 = min(nsteps, s0 + sps);
    const int64_t row_bytes = static_cast<int64_t>(nb) * F::kBytes;
    const uint8_t *wrows = b + row0 * row_bytes;
    uint8_t *stage = reinterpret_cast<uint8_t *>(smem4) + w * (R * SBY);

    v4f acc[MB][NT];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mb][t] = v4f{0.f, 0.f, 0.f, 0.f};

    // Chunk ci = u * 64 + lane of a step is chunk cc = ci % CPR of stage row
    // r = ci / CPR.  Lanes past the last chunk, chunks past a partial step's
    // end and rows past N re-read an in-bounds chunk (their LDS bytes are
    // never used for a stored output).
    // Per-lane byte offsets of the chunk loads inside a full step (fixed for the
    // whole K loop; only the step base moves, in scalar registers), and of the
    // LDS slots they go to.  A partial last step (8 blocks) uses the offsets of
    // its first half: chunk cc is re-read as cc - cpr when past the step's end.
    uint32_t goff[LPL], soff[LPL];
    int ccol[LPL];
#pragma unroll
    for (int u = 0; u < LPL; ++u) {
        const int ci = min(u * kWave + lane, CH - 1);
        const int r = ci / CPR, cc = ci % CPR;
        const int64_t row = min<int64_t>(r, rows_left - 1);
        goff[u] = static_cast<uint32_t>(row * row_bytes + 16 * cc);
        soff[u] = static_cast<uint32_t>(r * SBY + 16 * cc);
        ccol[u] = cc;
    }
    // Loads go through a buffer resource over the rest of the tile's rows from
    // the step on; `real == false` gives a resource of size 0, so every load is
    // out of range and returns zeros without touching memory (the last
    // iteration's stand-in prefetch, see below).
    uint4 nxt[LPL];
    const uint64_t tile_bytes = static_cast<uint64_t>(min<int64_t>(R, rows_left)) * row_bytes;
    auto fetch = [&](int s, bool real) {
        const int cpr = min(16, nb - 16 * s) * F::kBytes / 16;  // chunks per row in this step
        const uint64_t start = static_cast<uint64_t>(s) * SBY;
        const __amdgpu_buffer_rsrc_t rs = sm_rsrc(wrows + start, real ? tile_bytes - start : 0);
#pragma unroll
        for (int u = 0; u < LPL; ++u) {
            const uint32_t o = ccol[u] < cpr ? goff[u] : goff[u] - 16 * cpr;
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(o), 0, kSmStream);
            nxt[u] = make_uint4(v.x, v.y, v.z, v.w);
        }
    };

    const int first = s0 + w;
    const int cnt = first < s1 ? (s1 - 1 - first) / W + 1 : 0;
    const int last = first + (cnt - 1) * W;
    if (cnt > 0) fetch(first, true);
    for (int i = 0; i < cnt; ++i) {
        const int s = first + i * W;
        const int nbs = min(16, nb - 16 * s);  // blocks in this step (a multiple of 8)
        const int blk = min(bl, nbs - 1);      // lanes past the step decode its last block, masked
        // The stage is this wave's own: its LDS operations execute in program
        // order, so the previous step's reads are done before these stores and
        // the stores before the reads below.
#pragma unroll
        for (int u = 0; u < LPL; ++u) smem4[(w * (R * SBY) + soff[u]) / 16] = nxt[u];
        // This lane's activations: block blk of the step in rows 4 mb + c (rows
        // past M repeat row M - 1; their outputs are never stored).  Issued
        // before the next step's weight loads, so the decode below waits for
        // them only, not for the prefetch (vmcnt counts loads in issue order).
        float av[MB][32];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            const float4 *ar = reinterpret_cast<const float4 *>(
                a + min<int64_t>(4 * mb + c, M - 1) * K + 32 * (16 * static_cast<int64_t>(s) + blk));
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 x = ar[q];
                av[mb][4 * q + 0] = x.x;
                av[mb][4 * q + 1] = x.y;
                av[mb][4 * q + 2] = x.z;
                av[mb][4 * q + 3] = x.w;
            }
        }
        // The next step's weights, in flight during the decode.  Issued on every
        // iteration (the last one through an empty resource): a conditional
        // prefetch makes the compiler's wait counts pessimistic at the join,
        // which serialises the prefetch with the decode.
        fetch(min(s + W, last), i + 1 < cnt);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            uint32_t cw[F::kCodeDw];
            const uint32_t hb = block_window<F::kCodeDw>(stage, (4 * t + c) * SBY + F::kBytes * blk, cw);
            const float d = bl < nbs ? half_bits_to_float(hb) : 0.f;
            v4f tsum[MB];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) tsum[mb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 32; ++e) {
                const float x = code_value<FMT>(cw, e);  // one code feeds every row group
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    tsum[mb] = __builtin_amdgcn_mfma_f32_4x4x1f32(av[mb][e], x, tsum[mb], 0, 0, 0);
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[mb][t][q] = fmaf(d, tsum[mb][q], acc[mb][t][q]);
        }
        __builtin_amdgcn_wave_barrier();
    }

    // Sum the 16 blocks; lane (b, c) keeps value v of its (mb, t, q) list when
    // v % 16 == b, so the 64 lanes write each wave's NV x 4 sums exactly once.
    __syncthreads();  // every wave is done with its stage: the LDS is reused below
    float *red = reinterpret_cast<float *>(smem4);  // [W][NV][4]
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int v = (mb * NT + t) * 4 + q;
                const float sum = block_sum16(acc[mb][t][q]);
                if ((v & 15) == bl) red[(w * NV + v) * 4 + c] = sum;
            }
    __syncthreads();
    float *dst = out + (mode == kPartial ? static_cast<int64_t>(sp) * M * N : 0);
    const bool add = mode == kAdd;
    for (int e = threadIdx.x; e < NV * 4; e += W * kWave) {
        const int v = e >> 2, j = e & 3;
        const int mb = v / (NT * 4), t = (v >> 2) % NT, q = v & 3;
        const int64_t row = 4 * mb + q, col = row0 + 4 * t + j;
        if (row >= M || col >= N) continue;
        float sum = red[v * 4 + j];
#pragma unroll
        for (int ww = 1; ww < W; ++ww) sum += red[(ww * NV + v) * 4 + j];
        float *p = dst + row * N + col;
        *p = add ? *p + sum : sum;
    }
}

// Tuning hook: WQ_SMALLM_SHAPE = 1..4 forces (NT, W) = (4, 4), (8, 2), (4, 2)
// or (8, 1); unset or 0 = the default.
int smallm_shape() {
    static const int v = [] {
        const char *e = std::getenv("WQ_SMALLM_SHAPE");
        return e ? std::atoi(e) : 0;
    }();
    return v;
}

int smallm_splits() {
    static const int v = [] {
        const char *e = std::getenv("WQ_SMALLM_SPLITS");
        return e ? std::atoi(e) : 0;
    }();
    return v;
}

// Waves per CU the plan aims for before it splits K across workgroups.
constexpr int kSmWavesPerCU = 8;

struct SmPlan {
    int groups, splits, sps;
};

template <int FMT, int NT, int W>
SmPlan sm_plan(int64_t n, int64_t k, int cus) {
    const int64_t nb = k / 32, nsteps = (nb + 15) / 16;
    const int64_t groups = (n + 4 * NT - 1) / (4 * NT);
    // Workgroups for about kSmWavesPerCU waves per CU, K split across them only
    // as far as that needs and never below one step per wave.
    int64_t want = (static_cast<int64_t>(kSmWavesPerCU) * cus + groups * W - 1) / (groups * W);
    want = std::max<int64_t>(1, std::min<int64_t>(want, (nsteps + W - 1) / W));
    if (smallm_splits() > 0) want = std::min<int64_t>(smallm_splits(), nsteps);
    const int64_t sps = (nsteps + want - 1) / want;
    return SmPlan{static_cast<int>(groups), static_cast<int>((nsteps + sps - 1) / sps), static_cast<int>(sps)};
}

template <int FMT, int MB, int NT, int W>
hipError_t run_sm(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k, int cus, hipStream_t s,
                  int epi) {
    using F = SmFmt<FMT>;
    const SmPlan p = sm_plan<FMT, NT, W>(n, k, cus);
    const bool glu = epi == kEpiGlu;          // n counts the 2 no weight rows here
    const int64_t no = glu ? n / 2 : n;
    ScratchLease lease;
    float *out = c;
    const bool partial = p.splits > 1 || glu;  // raw sums to scratch, then reduce_splits
    if (partial) {
        void *scratch = nullptr;
        const hipError_t e =
            lease.acquire(static_cast<size_t>(p.splits) * static_cast<size_t>(m) * static_cast<size_t>(n) * 4, s,
                          &scratch);
        if (e != hipSuccess) return e;
        out = static_cast<float *>(scratch);
    }
    const size_t lds = std::max<size_t>(static_cast<size_t>(W) * 4 * NT * F::kStepBytes,
                                        static_cast<size_t>(W) * MB * NT * 16 * 4);
    if (trace_enabled())
        fprintf(stderr,
                "[wqmm] gemm_smallm<fmt=%d,MB=%d,NT=%d,W=%d> m=%lld n=%lld k=%lld groups=%d splits=%d sps=%d lds=%zu "
                "epi=%d\n",
                FMT, MB, NT, W, (long long)m, (long long)n, (long long)k, p.groups, p.splits, p.sps, lds, epi);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.groups) * p.splits));
    const int mode = partial ? kPartial : epi == kEpiResidual ? kAdd : kStore;
    hipLaunchKernelGGL((gemm_smallm<FMT, MB, NT, W>), grid, dim3(W * kWave), lds, s, a, b, out, m, n, k, p.groups,
                       p.sps, mode);
    hipError_t e = hipGetLastError();
    if (partial) {
        if (e == hipSuccess)
            e = launch_reduce_splits(out, c, m, no, n, p.splits, glu ? kEpiGlu : epi, s);
        const hipError_t er = lease.release();
        if (e == hipSuccess) e = er;
    }
    return e;
}

template <int FMT, int MB>
hipError_t run_sm_mb(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k, int cus,
                     hipStream_t s, int epi) {
    switch (smallm_shape()) {
        case 1: return run_sm<FMT, MB, 4, 4>(a, b, c, m, n, k, cus, s, epi);
        case 2: return run_sm<FMT, MB, 8, 2>(a, b, c, m, n, k, cus, s, epi);
        case 3: return run_sm<FMT, MB, 4, 2>(a, b, c, m, n, k, cus, s, epi);
        case 4: return run_sm<FMT, MB, 8, 1>(a, b, c, m, n, k, cus, s, epi);
        default: return run_sm<FMT, MB, 4, 4>(a, b, c, m, n, k, cus, s, epi);
    }
}

template <int FMT>
hipError_t run_sm_fmt(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k, int cus,
                      hipStream_t s, int epi) {
    switch ((m + 3) / 4) {
        case 1: return run_sm_mb<FMT, 1>(a, b, c, m, n, k, cus, s, epi);
        case 2: return run_sm_mb<FMT, 2>(a, b, c, m, n, k, cus, s, epi);
        case 3: return run_sm_mb<FMT, 3>(a, b, c, m, n, k, cus, s, epi);
        default: return run_sm_mb<FMT, 4>(a, b, c, m, n, k, cus, s, epi);
    }
}

}  // namespace

bool smallm_ok(const float *a, const void *b, int fmt, int64_t m, int64_t k) {
    return (fmt == SM_Q8_0 || fmt == SM_Q4_0) && m >= 1 && m <= 16 && k % 256 == 0 && k > 0 &&
           (reinterpret_cast<uintptr_t>(a) & 15) == 0 && (reinterpret_cast<uintptr_t>(b) & 15) == 0;
}

// n = output columns; with kEpiGlu the weights have 2n rows.
hipError_t launch_smallm(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t s, int epi) {
    if (!smallm_ok(a, b, fmt, m, k)) return hipErrorInvalidValue;
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    const int64_t nw = epi == kEpiGlu ? 2 * n : n;
    const uint8_t *b8 = static_cast<const uint8_t *>(b);
    if (fmt == SM_Q8_0) return run_sm_fmt<SM_Q8_0>(a, b8, c, m, nw, k, di.cus, s, epi);
    return run_sm_fmt<SM_Q4_0>(a, b8, c, m, nw, k, di.cus, s, epi);
}

}  // namespace wq
