// Small-M product (2 <= M <= 16): C[M,N] = A[M,K] . B[N,K]^T with f16, Q8_0
// or Q4_0 weights, streamed once from HBM through the fp32 matrix cores.
//
// Operation: the M > 1 branch of dispatch_gemm_q8 (lattice-inference 0.9.0,
// dispatch.rs); its multi-row GEMV prior art is the kernel gemm_q8 (a few
// weight rows times a few activation rows per threadgroup, lattice-inference
// 0.1.2, metal_qwen35.rs).  For M <= 16 the product is a weight stream, so
// the tiled GEMM's LDS staging and per-tile barriers are pure overhead here.
//
// CDNA4 design:
//  * Matrix op: v_mfma_f32_4x4x1_16b_f32, sixteen independent 4x4 blocks of
//    rank-1 updates.  Block b = lane / 4 works on its own chunk of E
//    consecutive k; lane c = lane % 4 of the block supplies row c of a group of
//    4 rows of A and row c of a tile of 4 weight rows.  A and the weights
//    share the lane -> (block, row) map, so every block accumulates
//    D_b[i][j] = sum over its k of A[i][k] * W[j][k], and the 16 blocks are
//    summed once at the end.  Rows of A are padded to a multiple of 4 (not of
//    16), so M = 2 wastes half the matrix-core work, not seven eighths.
//  * A wave owns NT tiles of 4 weight rows and MB = ceil(M/4) groups of A
//    rows.  One step covers KS = 16*E columns: per row of a tile that is
//    16*E contiguous weights (coalesced), per lane NT weight chunks and MB
//    activation chunks, then E * NT * MB matrix ops.
//  * Loads are buffer loads: the wave-uniform resource moves by one step's
//    bytes per step (scalar arithmetic) and each lane's offset into it is fixed
//    for the whole loop, so the main loop spends no vector instructions on
//    addresses.  Reads past the end of a matrix return zero in hardware.
//  * Loads run P steps ahead in a ring of P+1 register sets, so each wave
//    keeps P steps of weights in flight.  The main loop covers full steps only;
//    the one partial step of K (if any) is done after it, with the columns past
//    K zeroed in both operands.  No LDS and no barrier in the main loop.
//  * A workgroup of W waves shares its tiles and takes a K range; its waves
//    take the range's steps round-robin.  At the end each wave sums its 16
//    blocks with DPP row rotations and cross-row swizzles, the W waves are
//    summed through LDS in wave order, and, when K is also split across
//    workgroups, partial tiles (only the M real rows) go to scratch and
//    reduce_splits sums them in split order: results are deterministic.
//  * The scalar variant (VEC = false) loads activations (and f16 weights)
//    element by element with guards; it serves f16 rows that are not 16-byte
//    aligned (K % 8 != 0 or a misaligned pointer) and activations that are not
//    16-byte aligned.
#include "wq_internal.h"

#include <algorithm>
#include <cstdio>

namespace wq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQ8BlockBytes = 34;
constexpr int kQ4BlockBytes = 18;
enum { FMT_F16 = 0, FMT_Q8_0 = 1, FMT_Q4_0 = 2 };

// Buffer resource over [p, p + bytes) (bytes capped at 4 GiB - 1): raw,
// untyped (stride 0), third dword as for every gfx9 target.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint64_t bytes) {
    const uint32_t n = (bytes >> 32) != 0 ? 0xffffffffu : static_cast<uint32_t>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(n), 0x00020000);
}
constexpr int kStream = 2;  // non-temporal: every weight is read once

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, kStream);
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, kStream);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, kStream));
}
__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, kStream));
}

template <int FMT, int MB, int NT, int E, bool VEC>
struct Skinny {
    static constexpr int KS = 16 * E;  // columns per step
    static constexpr int WD = FMT == FMT_F16 ? E / 2 : FMT == FMT_Q8_0 ? E / 4 : E / 8;  // weight dwords
    static_assert(E == 8 || E == 16 || E == 32, "chunk");
    static constexpr int QBB = FMT == FMT_Q4_0 ? kQ4BlockBytes : kQ8BlockBytes;
    // Bytes one step advances along a weight row / an activation row.
    static constexpr uint32_t kWStep = FMT == FMT_F16 ? 2 * KS : KS / 32 * QBB;
    static constexpr uint32_t kAStep = 4 * KS;

    struct Regs {
        float a[MB][E];
        uint32_t w[NT][WD];
        uint32_t d[FMT != FMT_F16 ? NT : 1];
    };

    // Per-lane byte offsets, fixed for the whole K loop.  Lane (b, c) reads
    // columns E*b .. E*b+E-1 of each step, in weight row 4*t + c of the
    // workgroup's tiles and in A row min(4*mb + c, M-1) (rows past M repeat
    // row M-1 and feed outputs that are never stored).
    struct Lane {
        uint32_t a[MB];  // into A
        uint32_t w[NT];  // into the tiles: f16 chunk, or Q8_0 codes
        uint32_t d[NT];  // offset of the scale of the lane's block (Q8_0, Q4_0)
        int b, c;
    };

    // glu: tiles t < NT/2 are gate rows and t >= NT/2 the matching up rows,
    // each half addressed from its own base (row 4 * (t % (NT/2)) + c).
    static __device__ __forceinline__ Lane lane_offsets(int lane, int64_t M, int64_t K, bool glu) {
        Lane L;
        L.b = lane >> 2;
        L.c = lane & 3;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            L.a[mb] = static_cast<uint32_t>((min<int64_t>(4 * mb + L.c, M - 1) * K + E * L.b) * 4);
        const uint64_t row_bytes = FMT == FMT_F16 ? 2ull * K : static_cast<uint64_t>(K >> 5) * QBB;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int tt = glu ? t % (NT / 2) : t;
            const uint64_t rb = static_cast<uint64_t>(4 * tt + L.c) * row_bytes;
            if constexpr (FMT == FMT_F16) {
                L.w[t] = static_cast<uint32_t>(rb + 2 * E * L.b);
                L.d[t] = 0;
            } else {
                // The lane's E columns start at code index off of block blk:
                // byte 2 + off (Q8_0) or 2 + off / 2 (Q4_0, two codes a byte).
                const int blk = (E * L.b) >> 5, off = (E * L.b) & 31;
                L.d[t] = static_cast<uint32_t>(rb + blk * QBB);
                L.w[t] = L.d[t] + 2 + (FMT == FMT_Q8_0 ? off : off / 2);
            }
        }
        return L;
    }

    // Loads one step.  ra / rw / ru: resources whose base is the step's first
    // column in A / in the workgroup's first weight row / in its first up row
    // (ru serves tiles t >= NT/2 when glu).  For the scalar variant: k0 = the
    // lane's first column, a the matrix, wrows / urows the f16 rows at those
    // bases and rows_left the rows from a base to the end of its half.
    static __device__ __forceinline__ void load(Regs &r, const Lane &L, __amdgpu_buffer_rsrc_t ra,
                                                __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t ru, bool glu,
                                                const float *__restrict__ a, const uint16_t *__restrict__ wrows,
                                                const uint16_t *__restrict__ urows, int64_t M, int64_t K,
                                                int64_t rows_left, int64_t k0) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if constexpr (VEC) {
#pragma unroll
                for (int q = 0; q < E / 4; ++q) {
                    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, static_cast<int>(L.a[mb] + 16 * q), 0, 0);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        // Through a scalar: bit-casting the vector element
                        // expression itself reads element 0 in this compiler.
                        const uint32_t x = v[u];
                        r.a[mb][4 * q + u] = __builtin_bit_cast(float, x);
                    }
                }
            } else {
                const float *arow = a + min<int64_t>(4 * mb + L.c, M - 1) * K;
#pragma unroll
                for (int e = 0; e < E; ++e) r.a[mb][e] = (k0 + e < K) ? arow[k0 + e] : 0.f;
            }
        }
        if constexpr (FMT == FMT_F16) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const bool up = glu && t >= NT / 2;
                if constexpr (VEC) {
                    const __amdgpu_buffer_rsrc_t rt = up ? ru : rw;
#pragma unroll
                    for (int q = 0; q < E / 8; ++q) {
                        const u32x4 v = bload16(rt, L.w[t] + 16 * q);
#pragma unroll
                        for (int u = 0; u < 4; ++u) r.w[t][4 * q + u] = v[u];
                    }
                } else {
                    // Rows past the end repeat the last row (outputs never stored).
                    const int tt = glu ? t % (NT / 2) : t;
                    const uint16_t *row = (up ? urows : wrows) + min<int64_t>(4 * tt + L.c, rows_left - 1) * K;
#pragma unroll
                    for (int e = 0; e < E; e += 2) {
                        const uint32_t lo = (k0 + e < K) ? row[k0 + e] : 0u;
                        const uint32_t hi = (k0 + e + 1 < K) ? row[k0 + e + 1] : 0u;
                        r.w[t][e / 2] = lo | (hi << 16);
                    }
                }
            }
        } else {
            // WD dwords of codes: 4 (Q8_0) or 8 (Q4_0) weights per dword.
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const __amdgpu_buffer_rsrc_t rt = (glu && t >= NT / 2) ? ru : rw;
                r.d[t] = bload2(rt, L.d[t]);
                if constexpr (WD == 1) {
                    r.w[t][0] = bload4(rt, L.w[t]);
                } else if constexpr (WD == 2) {
                    const u32x2 v = bload8(rt, L.w[t]);
                    r.w[t][0] = v[0], r.w[t][1] = v[1];
                } else {
#pragma unroll
                    for (int q = 0; q < WD / 4; ++q) {
                        const u32x4 v = bload16(rt, L.w[t] + 16 * q);
#pragma unroll
                        for (int u = 0; u < 4; ++u) r.w[t][4 * q + u] = v[u];
                    }
                }
            }
        }
    }

    // Weight e of tile t as f32 (exact decode).
    static __device__ __forceinline__ float weight(const Regs &r, int t, int e) {
        if constexpr (FMT == FMT_F16) {
            const uint32_t w = r.w[t][e / 2];
            return half_bits_to_float((e & 1) ? (w >> 16) : (w & 0xffffu));
        } else if constexpr (FMT == FMT_Q8_0) {
            const uint32_t w = r.w[t][e / 4];
            const int8_t q = static_cast<int8_t>((w >> (8 * (e & 3))) & 0xffu);
            return half_bits_to_float(r.d[t]) * static_cast<float>(q);
        } else {
            // Code byte j holds column 2j (low nibble) and 2j + 1 (high).
            const uint32_t w = r.w[t][e / 8];
            const int u = static_cast<int>((w >> (4 * (e & 7))) & 0xfu);
            return half_bits_to_float(r.d[t]) * static_cast<float>(u - 8);
        }
    }

    // One step's matrix ops.  TAIL (the partial step only): chunks of 8
    // columns at or past K are zeroed in both operands, so bytes read past a
    // row's end (the next row's blocks, whose scale may be anything) cannot
    // leak in -- for every format and load variant except scalar f16, whose
    // loads already return zeros past K (K need not be a multiple of 8 there).
    template <bool TAIL>
    static __device__ __forceinline__ void compute(v4f (&acc)[MB][NT], const Regs &r, int64_t k0, int64_t K) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            bool in = true;
            if constexpr (TAIL && (VEC || FMT != FMT_F16)) in = k0 + (e & ~7) + 8 <= K;
            float wv[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) wv[t] = in ? weight(r, t, e) : 0.f;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const float av = in ? r.a[mb][e] : 0.f;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[mb][t] = __builtin_amdgcn_mfma_f32_4x4x1f32(av, wv[t], acc[mb][t], 0, 0, 0);
            }
        }
    }
};

// Sum over the 16 blocks (lanes with equal lane % 4): rotations by 4 and 8
// inside each 16-lane row, then across rows.  Every lane gets the total of its
// lane % 4.
__device__ __forceinline__ float block_sum(float v) {
    v += dpp_f32<0x124>(v);  // row_ror:4
    v += dpp_f32<0x128>(v);  // row_ror:8
    v += __shfl_xor(v, 16, kWave);
    v += __shfl_xor(v, 32, kWave);
    return v;
}

// Workgroup (grp, split) = (blockIdx.x % groups, blockIdx.x / groups) owns
// weight rows [4*NT*grp, 4*NT*(grp+1)) -- with the GLU epilogue, output
// columns [2*NT*grp, 2*NT*(grp+1)): their gate rows and (NO later) their up
// rows -- and steps [split*sps, min(nsteps, (split+1)*sps)); wave w takes
// steps w, w+W, ... of that range.  N = weight rows, NO = output columns.
// With one split the sums go to C [M, NO] through the epilogue, otherwise the
// raw sums go to out + split*M*N with column = weight row.
template <int FMT, int MB, int NT, int E, int P, int W, bool VEC>
__global__ __launch_bounds__(W * 64) void gemm_skinny(const float *__restrict__ a, const void *__restrict__ bw,
                                                      float *__restrict__ out, int64_t M, int64_t N, int64_t K,
                                                      int groups, int sps, int splits, int64_t NO, int epi) {
    using S = Skinny<FMT, MB, NT, E, VEC>;
    constexpr int KS = S::KS;
    constexpr int NV = MB * NT * 4;  // accumulator values per lane
    __shared__ float red[W][NV][4];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int grp = static_cast<int>(blockIdx.x % groups), sp = static_cast<int>(blockIdx.x / groups);
    const bool glu = epi == kEpiGlu;
    // n0: first weight row (plain) or first output column (glu) of the group;
    // g0 / u0: first gate / up weight row; rows_left: rows from g0 (or u0) to
    // the end of its half of the matrix.
    const int64_t n0 = static_cast<int64_t>(grp) * (glu ? 2 : 4) * NT;
    const int64_t g0 = n0, u0 = glu ? NO + n0 : n0;
    const int64_t rows_left = (glu ? NO : N) - n0;
    const int nsteps = static_cast<int>((K + KS - 1) / KS);
    const int nfull = static_cast<int>(K / KS);
    const int s0 = sp * sps, s1 = min(nsteps, s0 + sps);

    const typename S::Lane L = S::lane_offsets(lane, M, K, glu);
    const uint64_t row_bytes = FMT == FMT_F16 ? 2ull * K : static_cast<uint64_t>(K >> 5) * S::QBB;
    const uint8_t *wbase = static_cast<const uint8_t *>(bw) + g0 * row_bytes;
    const uint8_t *ubase = static_cast<const uint8_t *>(bw) + u0 * row_bytes;
    const uint64_t wbytes = (N - g0) * row_bytes, ubytes = (N - u0) * row_bytes;  // to the matrix end
    const uint64_t abytes = static_cast<uint64_t>(M) * K * 4;
    const uint16_t *wrows = static_cast<const uint16_t *>(bw) + g0 * K;  // scalar f16 path
    const uint16_t *urows = static_cast<const uint16_t *>(bw) + u0 * K;

    v4f acc[MB][NT];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[mb][t] = v4f{0.f, 0.f, 0.f, 0.f};

    typename S::Regs r[P + 1];
    auto load_step = [&](typename S::Regs &dst, int st) {
        const uint64_t wo = static_cast<uint64_t>(st) * S::kWStep, ao = static_cast<uint64_t>(st) * S::kAStep;
        S::load(dst, L, make_rsrc(reinterpret_cast<const uint8_t *>(a) + ao, abytes - ao),
                make_rsrc(wbase + wo, wbytes - wo), make_rsrc(ubase + wo, ubytes - wo), glu, a, wrows, urows, M, K,
                rows_left, static_cast<int64_t>(st) * KS + E * L.b);
    };

    // Full steps of this wave: first, first + W, ... below min(s1, nfull).
    const int first = s0 + wv;
    const int fend = min(s1, nfull);
    const int cnt = first < fend ? (fend - 1 - first) / W + 1 : 0;
    if (cnt > 0) {
        const int lastst = first + (cnt - 1) * W;
        // Ring slot q of the group starting at step index i holds step i + q;
        // position q loads step i + q + P into slot (q + P) % (P + 1).  Loads
        // past the last step re-read it, so every position issues the same loads.
#pragma unroll
        for (int p = 0; p < P; ++p) load_step(r[p], min(first + p * W, lastst));
        int i = 0;
        for (; i + P + 1 <= cnt; i += P + 1) {
#pragma unroll
            for (int q = 0; q <= P; ++q) {
                load_step(r[(q + P) % (P + 1)], min(first + (i + q + P) * W, lastst));
                __builtin_amdgcn_sched_barrier(0);  // loads stay ahead of this step's decode
                S::template compute<false>(acc, r[q], 0, K);
            }
        }
        // The last cnt - i (< P + 1) steps are already in slots 0 .. cnt-i-1.
#pragma unroll
        for (int q = 0; q < P; ++q)
            if (i + q < cnt) S::template compute<false>(acc, r[q], 0, K);
    }
    // The partial step of K, if any, by the wave of this split that owns it.
    if (nfull < nsteps && nfull >= s0 && nfull < s1 && (nfull - s0) % W == wv) {
        load_step(r[0], nfull);
        S::template compute<true>(acc, r[0], static_cast<int64_t>(nfull) * KS + E * L.b, K);
    }

    // Sum the 16 blocks; lane (b, c) keeps value v of its (mb, t, i) list when
    // v % 16 == b, so the 64 lanes write each wave's NV x 4 sums exactly once.
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = (mb * NT + t) * 4 + i;
                const float s = block_sum(acc[mb][t][i]);
                if ((v & 15) == L.b) red[wv][v][L.c] = s;
            }
    __syncthreads();
    if (splits == 1 && glu) {
        // SwiGLU: gate tile t pairs with up tile t + NT/2 of the same columns.
        for (int e = threadIdx.x; e < NV * 2; e += W * kWave) {
            const int vg = e >> 2, j = e & 3;  // vg over (mb, t < NT/2, i)
            const int mb = vg / (NT * 2), t = (vg >> 2) % (NT / 2), i = vg & 3;
            const int v = (mb * NT + t) * 4 + i, vu = v + 2 * NT;
            const int64_t row = 4 * mb + i, col = n0 + 4 * t + j;
            if (row >= M || col >= NO) continue;
            float g = red[0][v][j], u = red[0][vu][j];
#pragma unroll
            for (int w = 1; w < W; ++w) g += red[w][v][j], u += red[w][vu][j];
            out[row * NO + col] = silu(g) * u;
        }
        return;
    }
    const bool resid = splits == 1 && epi == kEpiResidual;
    float *dst = out + static_cast<int64_t>(sp) * M * N;
    for (int e = threadIdx.x; e < NV * 4; e += W * kWave) {
        const int v = e >> 2, j = e & 3;
        const int mb = v / (NT * 4), t = (v >> 2) % NT, i = v & 3;
        const int64_t row = 4 * mb + i;
        // Column of C (plain) or weight row (glu partial sums).
        int64_t col = n0 + 4 * t + j;
        bool ok = col < N;
        if (glu) {
            const int64_t oc = n0 + 4 * (t % (NT / 2)) + j;
            ok = oc < NO;
            col = t < NT / 2 ? oc : NO + oc;
        }
        if (row >= M || !ok) continue;
        float sum = red[0][v][j];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += red[w][v][j];
        float *p = dst + row * N + col;
        *p = resid ? *p + sum : sum;
    }
}

// Variant per format and row-group count MB (measured on MI355X at N, K in
// {4096, 11008}, M = 2..16): NT tiles of 4 rows per wave, E columns per lane
// and step, P steps of prefetch.  Workgroups have W = 4 waves.
template <int FMT, int MB>
struct SkCfg {
    static constexpr int NT = 4, E = 8, P = MB <= 2 ? 2 : 1;
};
template <>
struct SkCfg<FMT_Q8_0, 1> {
    static constexpr int NT = 2, E = 16, P = 2;
};
template <>
struct SkCfg<FMT_Q4_0, 1> {
    static constexpr int NT = 2, E = 16, P = 2;
};
constexpr int kSkW = 4;
constexpr int kSkWavesPerCU = 8;

struct SkPlan {
    int groups, splits, sps;
};

// Workgroups for about kSkWavesPerCU waves per CU; K is split across
// workgroups only as far as that needs, and every split keeps at least P+1
// steps per wave.  n = output columns (glu: 2*NT per group, else 4*NT).
template <int FMT, int MB>
SkPlan plan_for(int64_t n, int64_t k, int cus, bool glu) {
    using C = SkCfg<FMT, MB>;
    const int64_t nsteps = (k + 16LL * C::E - 1) / (16LL * C::E);
    const int64_t per = (glu ? 2LL : 4LL) * C::NT;
    const int64_t groups = (n + per - 1) / per;
    int64_t want = (static_cast<int64_t>(kSkWavesPerCU) * cus + groups * kSkW - 1) / (groups * kSkW);
    want = std::max<int64_t>(1, std::min<int64_t>(want, nsteps / (static_cast<int64_t>(kSkW) * (C::P + 1))));
    const int64_t sps = (nsteps + want - 1) / want;
    return SkPlan{static_cast<int>(groups), static_cast<int>((nsteps + sps - 1) / sps), static_cast<int>(sps)};
}

// n = output columns; the weights have nw = n (or 2n with the GLU epilogue) rows.
template <int FMT, int MB>
hipError_t run_skinny(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, bool vec, int cus,
                      hipStream_t s, int epi) {
    using C = SkCfg<FMT, MB>;
    static_assert(C::NT % 2 == 0, "the GLU epilogue pairs tile halves");
    const bool glu = epi == kEpiGlu;
    const int64_t nw = glu ? 2 * n : n;
    const SkPlan p = plan_for<FMT, MB>(n, k, cus, glu);
    ScratchLease lease;
    float *out = c;
    if (p.splits > 1) {
        void *scratch = nullptr;
        hipError_t e = lease.acquire(
            static_cast<size_t>(p.splits) * static_cast<size_t>(m) * static_cast<size_t>(nw) * 4, s, &scratch);
        if (e != hipSuccess) return e;
        out = static_cast<float *>(scratch);
    }
    if (trace_enabled())
        fprintf(stderr,
                "[wqmm] gemm_skinny<fmt=%d,MB=%d,NT=%d,E=%d,P=%d,W=%d,vec=%d> m=%lld n=%lld k=%lld groups=%d "
                "splits=%d sps=%d epi=%d\n",
                FMT, MB, C::NT, C::E, C::P, kSkW, vec, (long long)m, (long long)n, (long long)k, p.groups,
                p.splits, p.sps, epi);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(p.groups) * p.splits));
    if (vec)
        hipLaunchKernelGGL((gemm_skinny<FMT, MB, C::NT, C::E, C::P, kSkW, true>), grid, dim3(kSkW * 64), 0, s, a,
                           b, out, m, nw, k, p.groups, p.sps, p.splits, n, epi);
    else
        hipLaunchKernelGGL((gemm_skinny<FMT, MB, C::NT, C::E, C::P, kSkW, false>), grid, dim3(kSkW * 64), 0, s, a,
                           b, out, m, nw, k, p.groups, p.sps, p.splits, n, epi);
    hipError_t e = hipGetLastError();
    if (p.splits > 1) {
        if (e == hipSuccess) e = launch_reduce_splits(out, c, m, n, nw, p.splits, epi, s);
        const hipError_t er = lease.release();
        if (e == hipSuccess) e = er;
    }
    return e;
}

template <int FMT>
hipError_t run_fmt(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, bool vec, int cus,
                   hipStream_t s, int epi) {
    switch ((m + 3) / 4) {
        case 1: return run_skinny<FMT, 1>(a, b, c, m, n, k, vec, cus, s, epi);
        case 2: return run_skinny<FMT, 2>(a, b, c, m, n, k, vec, cus, s, epi);
        case 3: return run_skinny<FMT, 3>(a, b, c, m, n, k, vec, cus, s, epi);
        default: return run_skinny<FMT, 4>(a, b, c, m, n, k, vec, cus, s, epi);
    }
}

}  // namespace

hipError_t launch_skinny(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t s, int epi) {
    if (m < 1 || m > 16) return hipErrorInvalidValue;
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    const bool a16 = (reinterpret_cast<uintptr_t>(a) & 15) == 0;
    if (fmt == FMT_F16) {
        const bool vec = a16 && (reinterpret_cast<uintptr_t>(b) & 15) == 0 && k % 8 == 0;
        return run_fmt<FMT_F16>(a, b, c, m, n, k, vec, di.cus, s, epi);
    }
    if (fmt == FMT_Q4_0) return run_fmt<FMT_Q4_0>(a, b, c, m, n, k, a16, di.cus, s, epi);
    return run_fmt<FMT_Q8_0>(a, b, c, m, n, k, a16, di.cus, s, epi);
}

}  // namespace wq
