// Prefill GEMM (M > 1): C[M,N] = A[M,K] . B[N,K]^T with f16, Q8_0 or Q4_0 weights,
// fp32 matrix-core accumulation.
//
// Operation: dispatch_gemm_q8 / dispatch_gemm (lattice-inference 0.9.0,
// dispatch.rs) for M > 1; tiling prior art: matmul_bt (16x16 threadgroup
// tiles), gemm_q8 (multi-row GEMV) and gemm_q4_tiled (BM=64 x BN=32, one
// quant block per k-step, the weight tile dequantised into threadgroup memory,
// 8x8 simdgroup matrices) in lattice-inference 0.1.2, metal_qwen35.rs.
//
// CDNA4 design:
//  * A workgroup of 4 waves computes a BM x BN tile of C; waves are arranged
//    WM x WN and each owns a (BM/WM) x (BN/WN) sub-tile made of 32x32 blocks,
//    each accumulated by v_mfma_f32_32x32x2_f32 in 16 AGPRs, where the
//    sub-tile is a multiple of 32 both ways; otherwise of 16x16 blocks,
//    accumulated by v_mfma_f32_16x16x4_f32 in four AGPRs.  The 32x32 block
//    needs fewer independent accumulator chains to keep the matrix core busy
//    (measured on MI355X: 2-6 % faster on every 64/128-row tile and split).
//  * The K loop steps by BK = 32, exactly one Q8_0 block per weight row.  Each
//    step stages the A tile (f32) and the weight tile, widened (f16) or
//    dequantised (d*q, exact in f32), in LDS.  Three-stage pipeline with one
//    barrier per step: tile i is read from LDS buffer i&1 by the matrix cores,
//    tile i+1 (already in registers) is written to the other buffer between
//    the two halves of step i's MFMAs, and tile i+2 is loading from memory.
//  * The reduction index inside a 32-wide step is permuted so that every lane
//    reads consecutive k with 128-bit LDS reads: with 16x16 blocks, in MFMA
//    step t the lane group g = lane/16 supplies k = 8g + t (8 k per lane);
//    with 32x32 blocks g = lane/32 supplies k = 16g + t (16 k per lane).  The
//    sum over k is unchanged; only its order differs.
//  * Rows of the LDS tiles are padded by 16 bytes to spread LDS banks.
//  * Split K: when the (M, N) tiles alone cannot fill 256 CUs (small M, long
//    K), the K range is cut into equal splits whose partial tiles go to a
//    scratch buffer and are summed in split order by a second pass, so the
//    result is deterministic.  A cost model picks the tile shape and split
//    count per call.
//  * Workgroup -> tile mapping is XCD-aware: workgroups are dealt round-robin
//    to the 8 XCDs, so consecutive workgroup ids on one XCD are given tiles
//    that share weight columns (M-fastest tile order) and hit the same L2.
#include "wq_internal.h"

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace wq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BK = 32;
constexpr int PAD = 4;            // floats of padding per LDS row
constexpr int LDP = BK + PAD;     // LDS row pitch in floats
constexpr int kQ8BlockBytes = 34;
constexpr int kQ4BlockBytes = 18;

enum { FMT_F16 = 0, FMT_Q8_0 = 1, FMT_Q4_0 = 2 };

typedef float v16f __attribute__((ext_vector_type(16)));

// MF: the matrix-core block, 16 (v_mfma_f32_16x16x4_f32, 4 accumulators per
// lane) or 32 (v_mfma_f32_32x32x2_f32, 16 accumulators per lane).
template <int BM, int BN, int WM, int WN, int FMT, bool VEC, int MF>
struct Gemm {
    static_assert(WM * WN == 4, "four waves");
    static_assert(MF == 16 || MF == 32, "matrix block");
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / MF, FN = WTN / MF;
    static_assert(FM >= 1 && FN >= 1 && WTM % MF == 0 && WTN % MF == 0, "wave tile");
    // Per lane and k-tile: 64 / MF lane groups share the BK = 32 reduction
    // indices, KQ float4 (KQ * 4 consecutive k) each.
    static constexpr int LG = 64 / MF, KQ = BK / LG / 4;
    static constexpr int NV = MF == 16 ? 4 : 16;  // accumulators per lane and block
    typedef typename std::conditional<MF == 16, v4f, v16f>::type acc_t;
    static constexpr int A_ITERS = (BM * 8 + 255) / 256;    // float4 chunks of A per thread
    static constexpr int B16_ITERS = (BN * 4 + 255) / 256;  // uint4 chunks of f16 B per thread
    static constexpr int B8_ITERS = (BN * 2 + 255) / 256;   // half blocks of Q8_0 / Q4_0 B per thread
    static constexpr bool QUANT = FMT != FMT_F16;
    static constexpr int QBB = FMT == FMT_Q4_0 ? kQ4BlockBytes : kQ8BlockBytes;  // block bytes
    static constexpr int QW = FMT == FMT_Q4_0 ? 4 : 8;  // 16-bit code words per half block

    struct Regs {
        float4 a[A_ITERS];
        uint4 b16[FMT == FMT_F16 ? B16_ITERS : 1];
        uint32_t d8[QUANT ? B8_ITERS : 1];
        uint32_t q8[QUANT ? B8_ITERS : 1][QW];
    };

    // Weight row feeding row `row` of the LDS weight tile.  Plain: n0 + row
    // (clamped: rows past N only feed outputs that are never stored).  GLU
    // (gate/up pairs for the SwiGLU epilogue; N = 2*NO weight rows, n0 = the
    // tile's first output column): each wave's WTN tile rows are WTN/2 gate
    // rows followed by the up rows of the same output columns, so fragment fj
    // and fj + FN/2 of a wave hold a gate and its up at the same lane.
    static __device__ __forceinline__ int64_t brow(int64_t n0, int row, int64_t N, int64_t NO, bool glu) {
        if (!glu) return min<int64_t>(n0 + row, N - 1);
        const int wn = row / WTN, within = row % WTN;
        const int64_t oc = min<int64_t>(n0 + wn * (WTN / 2) + within % (WTN / 2), NO - 1);
        return within < WTN / 2 ? oc : NO + oc;
    }

    // Global -> registers for the k-tile starting at k0.  On the vector path
    // every thread issues the same number of loads on every call (addresses
    // are clamped into the matrices and out-of-range values zeroed after the
    // load), so the compiler can count outstanding loads across the software
    // pipeline instead of draining them all.  VEC requires K % 8 == 0 (f16)
    // or K % 32 == 0 (Q8_0) and 16-byte aligned rows of A (and of f16 B).
    static __device__ __forceinline__ void load(Regs &r, const float *__restrict__ a,
                                                const void *__restrict__ bw, int64_t M, int64_t N,
                                                int64_t K, int64_t m0, int64_t n0, int64_t k0,
                                                int tid, int64_t NO, bool glu) {
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int row = (tid >> 3) + 32 * i;
            const int c4 = tid & 7;
            const int64_t gm = m0 + row, gk = k0 + 4 * c4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (VEC) {
                // Rows past M only feed outputs that are never stored; the
                // K tail is zeroed when the tile is written to LDS.
                const int64_t gmc = min<int64_t>(gm, M - 1), gkc = min<int64_t>(gk, K - 4);
                v = *reinterpret_cast<const float4 *>(a + gmc * K + gkc);
            } else if (row < BM && gm < M) {
                const float *p = a + gm * K + gk;
                if (gk + 0 < K) v.x = p[0];
                if (gk + 1 < K) v.y = p[1];
                if (gk + 2 < K) v.z = p[2];
                if (gk + 3 < K) v.w = p[3];
            }
            r.a[i] = v;
        }
        if constexpr (FMT == FMT_F16) {
            const uint16_t *b = static_cast<const uint16_t *>(bw);
#pragma unroll
            for (int i = 0; i < B16_ITERS; ++i) {
                const int row = (tid >> 2) + 64 * i;
                const int c8 = tid & 3;
                const int64_t gn = brow(n0, row, N, NO, glu), gk = k0 + 8 * c8;
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (VEC) {
                    const int64_t gkc = min<int64_t>(gk, K - 8);
                    v = *reinterpret_cast<const uint4 *>(b + gn * K + gkc);
                } else if (row < BN) {
                    const uint16_t *p = b + gn * K + gk;
                    uint32_t h[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) h[u] = (gk + u < K) ? p[u] : 0u;
                    v = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                   h[6] | (h[7] << 16));
                }
                r.b16[i] = v;
            }
        } else {
            // Thread half h of a block row reads the scale and the code bytes
            // of weights 16h .. 16h+15: 16 bytes (Q8_0) or 8 bytes (Q4_0).
            const uint8_t *b = static_cast<const uint8_t *>(bw);
            const int64_t row_bytes = (K >> 5) * QBB;
            const int64_t kb = k0 >> 5;
#pragma unroll
            for (int i = 0; i < B8_ITERS; ++i) {
                const int row = (tid >> 1) + 128 * i;
                const int h = tid & 1;
                // Rows past N only feed outputs that are never stored.
                const int64_t gnc = brow(n0, row, N, NO, glu);
                const uint16_t *blk = reinterpret_cast<const uint16_t *>(b + gnc * row_bytes + kb * QBB);
                r.d8[i] = blk[0];
#pragma unroll
                for (int u = 0; u < QW; ++u) r.q8[i][u] = blk[1 + QW * h + u];
            }
        }
    }

    // Registers -> LDS (A as is; weights widened or dequantised to f32).
    // k0/K: the tile's first k and the reduction length; on the vector path the
    // chunks at or past K (f16 with K % 32 != 0) are written as zeros here.
    static __device__ __forceinline__ void store(const Regs &r, float (*As)[LDP], float (*Bs)[LDP],
                                                 int tid, int64_t k0, int64_t K) {
        const bool a_in = !VEC || k0 + 4 * (tid & 7) + 4 <= K;
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int row = (tid >> 3) + 32 * i;
            if (row < BM)
                *reinterpret_cast<float4 *>(&As[row][4 * (tid & 7)]) = a_in ? r.a[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if constexpr (FMT == FMT_F16) {
            const bool b_in = !VEC || k0 + 8 * (tid & 3) + 8 <= K;
#pragma unroll
            for (int i = 0; i < B16_ITERS; ++i) {
                const int row = (tid >> 2) + 64 * i;
                if (row < BN) {
                    const uint4 v = b_in ? r.b16[i] : make_uint4(0u, 0u, 0u, 0u);
                    float4 lo = make_float4(half_bits_to_float(v.x & 0xffffu), half_bits_to_float(v.x >> 16),
                                            half_bits_to_float(v.y & 0xffffu), half_bits_to_float(v.y >> 16));
                    float4 hi = make_float4(half_bits_to_float(v.z & 0xffffu), half_bits_to_float(v.z >> 16),
                                            half_bits_to_float(v.w & 0xffffu), half_bits_to_float(v.w >> 16));
                    float *dst = &Bs[row][8 * (tid & 3)];
                    *reinterpret_cast<float4 *>(dst) = lo;
                    *reinterpret_cast<float4 *>(dst + 4) = hi;
                }
            }
        } else if constexpr (FMT == FMT_Q4_0) {
            // Code word u holds weights 4u .. 4u+3 of the half block, one per
            // nibble from the least significant: (nibble - 8) * d.
#pragma unroll
            for (int i = 0; i < B8_ITERS; ++i) {
                const int row = (tid >> 1) + 128 * i;
                if (row < BN) {
                    const float d = half_bits_to_float(r.d8[i]);
                    float *dst = &Bs[row][16 * (tid & 1)];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint32_t w = r.q8[i][u];
                        float4 v = make_float4(d * static_cast<float>(static_cast<int>(w & 0xfu) - 8),
                                               d * static_cast<float>(static_cast<int>((w >> 4) & 0xfu) - 8),
                                               d * static_cast<float>(static_cast<int>((w >> 8) & 0xfu) - 8),
                                               d * static_cast<float>(static_cast<int>((w >> 12) & 0xfu) - 8));
                        *reinterpret_cast<float4 *>(dst + 4 * u) = v;
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < B8_ITERS; ++i) {
                const int row = (tid >> 1) + 128 * i;
                if (row < BN) {
                    const float d = half_bits_to_float(r.d8[i]);
                    float *dst = &Bs[row][16 * (tid & 1)];
#pragma unroll
                    for (int u = 0; u < 8; u += 2) {
                        const uint32_t p0 = r.q8[i][u], p1 = r.q8[i][u + 1];
                        float4 v = make_float4(d * static_cast<float>(static_cast<int8_t>(p0 & 0xffu)),
                                               d * static_cast<float>(static_cast<int8_t>(p0 >> 8)),
                                               d * static_cast<float>(static_cast<int8_t>(p1 & 0xffu)),
                                               d * static_cast<float>(static_cast<int8_t>(p1 >> 8)));
                        *reinterpret_cast<float4 *>(dst + 2 * u) = v;
                    }
                }
            }
        }
    }

    // Fragments of one k-tile: lane (i = lane % MF, g = lane / MF) holds, for
    // fragment f, the 4 KQ consecutive k = 4 KQ g .. 4 KQ g + 4 KQ - 1 of its
    // row (8 for MF = 16, 16 for MF = 32); MFMA step t takes component t.
    struct Frags {
        float4 a[FM][KQ], b[FN][KQ];
    };

    static __device__ __forceinline__ void read_frags(Frags &fr, const float (*As)[LDP],
                                                      const float (*Bs)[LDP], int wm, int wn,
                                                      int lane) {
        const int li = lane % MF, lg = lane / MF;
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
#pragma unroll
            for (int f = 0; f < FM; ++f)
                fr.a[f][q] = *reinterpret_cast<const float4 *>(&As[wm * WTM + MF * f + li][4 * KQ * lg + 4 * q]);
#pragma unroll
            for (int f = 0; f < FN; ++f)
                fr.b[f][q] = *reinterpret_cast<const float4 *>(&Bs[wn * WTN + MF * f + li][4 * KQ * lg + 4 * q]);
        }
    }

    static __device__ __forceinline__ float comp(const float4 &v, int t) {
        return t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w;
    }

    // MFMA steps t = H * 4 KQ / 2 .. (H + 1) * 4 KQ / 2 - 1 on every block
    // (k = 4 KQ g + t in lane group g): half of the k-tile.
    template <int H>
    static __device__ __forceinline__ void mfma_half(acc_t (&acc)[FM][FN], const Frags &fr) {
        constexpr int T = 4 * KQ / 2;
#pragma unroll
        for (int t = H * T; t < (H + 1) * T; ++t)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (MF == 16)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(comp(fr.a[i][t / 4], t % 4),
                                                                         comp(fr.b[j][t / 4], t % 4), acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(comp(fr.a[i][t / 4], t % 4),
                                                                         comp(fr.b[j][t / 4], t % 4), acc[i][j], 0, 0, 0);
                }
    }

    // Row (within the block) of accumulator v of a lane: 16x16 blocks hold
    // row 4 (lane / 16) + v, 32x32 blocks row 8 (v / 4) + 4 (lane / 32) + v % 4;
    // the column is lane % MF.
    static __device__ __forceinline__ int acc_row(int lane, int v) {
        return MF == 16 ? 4 * (lane / 16) + v : 8 * (v / 4) + 4 * (lane / 32) + v % 4;
    }
};

// Grid: tiles * splits workgroups.  Split s covers k-tiles [s*kts, min(kt, (s+1)*kts)).
// N = weight rows; NO = output columns (N, or N / 2 for the GLU epilogue).
// With one split the tile goes to C [M, NO] through the epilogue; otherwise the
// raw sums go to out = partial + s*M*N, column = weight row, and
// reduce_splits sums them in split order and applies the epilogue.
template <int BM, int BN, int WM, int WN, int FMT, bool VEC, int MF>
__global__ __launch_bounds__(256) void gemm_mfma(const float *__restrict__ a, const void *__restrict__ bw,
                                                 float *__restrict__ c, int64_t M, int64_t N, int64_t K,
                                                 int mtiles, int tiles, int splits, int kts, int64_t NO,
                                                 int epi) {
    using G = Gemm<BM, BN, WM, WN, FMT, VEC, MF>;
    __shared__ float As[2][BM][LDP];
    __shared__ float Bs[2][BN][LDP];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int idx = xcd_tile(blockIdx.x, tiles * splits);
    const int tile = idx % tiles, split = idx / tiles;
    const bool glu = epi == kEpiGlu;
    const int64_t m0 = static_cast<int64_t>(tile % mtiles) * BM;
    const int64_t n0 = static_cast<int64_t>(tile / mtiles) * (glu ? BN / 2 : BN);  // first output column
    const int64_t ktiles = (K + BK - 1) / BK;
    const int64_t kt0 = static_cast<int64_t>(split) * kts;
    const int64_t nkt = min<int64_t>(ktiles, kt0 + kts) - kt0;  // >= 1 by construction
    float *out = c + static_cast<int64_t>(split) * M * N;

    typename G::acc_t acc[G::FM][G::FN];
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int j = 0; j < G::FN; ++j)
#pragma unroll
            for (int v = 0; v < G::NV; ++v) acc[i][j][v] = 0.f;

    // Software pipeline: tile i is in LDS buffer i & 1; tile i+1 sits in
    // registers and is written to the other buffer between the two MFMA
    // halves of step i; tile i+2 is being loaded from global memory.
    typename G::Regs r0, r1;
    G::load(r0, a, bw, M, N, K, m0, n0, kt0 * BK, tid, NO, glu);
    G::store(r0, As[0], Bs[0], tid, kt0 * BK, K);
    G::load(r1, a, bw, M, N, K, m0, n0, (kt0 + min<int64_t>(1, nkt - 1)) * BK, tid, NO, glu);
    __syncthreads();

    auto step = [&](int64_t i, typename G::Regs &rnext, typename G::Regs &rfut) {
        // Always load (the last tile again near the end): a fixed load count.
        G::load(rfut, a, bw, M, N, K, m0, n0, (kt0 + min<int64_t>(i + 2, nkt - 1)) * BK, tid, NO, glu);
        const int cur = static_cast<int>(i & 1);
        typename G::Frags fr;
        G::read_frags(fr, As[cur], Bs[cur], wm, wn, lane);
        G::template mfma_half<0>(acc, fr);
        if (i + 1 < nkt) G::store(rnext, As[cur ^ 1], Bs[cur ^ 1], tid, (kt0 + i + 1) * BK, K);
        G::template mfma_half<1>(acc, fr);
        __syncthreads();
    };
    int64_t i = 0;
    for (; i + 1 < nkt; i += 2) {
        step(i, r1, r0);
        step(i + 1, r0, r1);
    }
    if (i < nkt) step(i, r1, r0);

    // Accumulator v of block (fi, fj): row G::acc_row(lane, v), column lane % MF.
    const int li = lane % MF;
    const int64_t rwave = m0 + wm * G::WTM;
    if (splits == 1 && glu) {
        // SwiGLU: gate fragment fj pairs with up fragment fj + FN/2.
        if constexpr (G::FN % 2 == 0) {
#pragma unroll
            for (int fi = 0; fi < G::FM; ++fi) {
#pragma unroll
                for (int fj = 0; fj < G::FN / 2; ++fj) {
                    const int64_t col = n0 + wn * (G::WTN / 2) + MF * fj + li;
                    if (col >= NO) continue;
#pragma unroll
                    for (int v = 0; v < G::NV; ++v) {
                        const int64_t row = rwave + MF * fi + G::acc_row(lane, v);
                        if (row < M) c[row * NO + col] = silu(acc[fi][fj][v]) * acc[fi][fj + G::FN / 2][v];
                    }
                }
            }
        }
        return;
    }
    const bool resid = splits == 1 && epi == kEpiResidual;
#pragma unroll
    for (int fi = 0; fi < G::FM; ++fi) {
#pragma unroll
        for (int fj = 0; fj < G::FN; ++fj) {
            // Column of C (one split) or of the partial buffer (weight row).
            int64_t col = n0 + wn * G::WTN + MF * fj + li;
            bool ok = col < N;
            if (glu) {
                const int within = MF * fj + li;
                const int64_t oc = n0 + wn * (G::WTN / 2) + within % (G::WTN / 2);
                ok = oc < NO;
                col = within < G::WTN / 2 ? oc : NO + oc;
            }
            if (!ok) continue;
#pragma unroll
            for (int v = 0; v < G::NV; ++v) {
                const int64_t row = rwave + MF * fi + G::acc_row(lane, v);
                if (row < M) {
                    float *dst = out + row * N + col;
                    *dst = resid ? *dst + acc[fi][fj][v] : acc[fi][fj][v];
                }
            }
        }
    }
}

// C[r, j] (r < m, j < no) from the split partial sums partial[s][r][.] (row
// length nw), summed in split order (deterministic): plain, added to C
// (residual), or silu(gate) * up with gate at column j and up at no + j (GLU,
// nw = 2 * no).  With splits == 1 it is the GLU epilogue alone.  A thread
// takes W adjacent columns of one row (W = 4: 16-byte loads and stores, when
// no is a multiple of 4 and C is 16-byte aligned); blockIdx.y strides rows.
template <int W>
__global__ __launch_bounds__(256) void reduce_splits(const float *__restrict__ partial, float *__restrict__ c,
                                                     int64_t m, int64_t no, int64_t nw, int splits, int epi) {
    typedef float vec __attribute__((ext_vector_type(W)));
    const int64_t j = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * W;
    if (j >= no) return;
    const int64_t plane = m * nw;
    for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
        const float *p = partial + r * nw + j;
        vec v = *reinterpret_cast<const vec *>(p);
#pragma unroll 4
        for (int s = 1; s < splits; ++s) v += *reinterpret_cast<const vec *>(p + s * plane);
        vec *out = reinterpret_cast<vec *>(c + r * no + j);
        if (epi == kEpiGlu) {
            vec u = *reinterpret_cast<const vec *>(p + no);
#pragma unroll 4
            for (int s = 1; s < splits; ++s) u += *reinterpret_cast<const vec *>(p + s * plane + no);
            vec o;
#pragma unroll
            for (int i = 0; i < W; ++i) o[i] = silu(v[i]) * u[i];
            *out = o;
        } else {
            *out = epi == kEpiResidual ? *out + v : v;
        }
    }
}

struct TileCfg {
    int bm, bn;
    int occ;     // workgroups that fit on one CU at once (LDS and VGPR limits)
    double eff;  // fraction of the fp32 matrix-core rate one CU sustains on
                 // this tile when enough workgroups are co-resident
};

struct Plan {
    TileCfg t;
    int splits;
    int kts;  // k-tiles per split
};

template <int BM, int BN, int WM, int WN, int FMT>
hipError_t run(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, bool vec, int splits,
               int kts, hipStream_t s, int64_t no, int epi) {
    const bool glu = epi == kEpiGlu;
    const int64_t mt = (m + BM - 1) / BM, nt = glu ? (no + BN / 2 - 1) / (BN / 2) : (n + BN - 1) / BN;
    const int64_t tiles = mt * nt;
    if (tiles * splits > 0x7fffffffLL) return hipErrorInvalidValue;
    const int64_t grid = tiles * splits;
    if (trace_enabled())
        fprintf(stderr,
                "[wqmm] gemm_mfma<BM=%d,BN=%d,WM=%d,WN=%d,fmt=%d,vec=%d> m=%lld n=%lld k=%lld splits=%d kts=%d "
                "epi=%d grid=%lld\n",
                BM, BN, WM, WN, FMT, vec ? 1 : 0, (long long)m, (long long)n, (long long)k, splits, kts, epi,
                (long long)grid);
    // 32x32 blocks where the wave tile is a multiple of 32 both ways (and, for
    // the fused SwiGLU, has an even number of 32-column fragments); else 16x16.
    constexpr bool mf32_tile = (BM / WM) % 32 == 0 && (BN / WN) % 32 == 0;
    constexpr bool mf32_glu = mf32_tile && ((BN / WN) / 32) % 2 == 0;
    const bool mf32 = vec && mf32_tile && (!glu || splits > 1 || mf32_glu);
    if (mf32) {
        if constexpr (mf32_tile)
            hipLaunchKernelGGL((gemm_mfma<BM, BN, WM, WN, FMT, true, 32>), dim3(grid), dim3(256), 0, s, a, b, c, m, n,
                               k, static_cast<int>(mt), static_cast<int>(tiles), splits, kts, no, epi);
    } else if (vec) {
        hipLaunchKernelGGL((gemm_mfma<BM, BN, WM, WN, FMT, true, 16>), dim3(grid), dim3(256), 0, s, a, b, c, m, n, k,
                           static_cast<int>(mt), static_cast<int>(tiles), splits, kts, no, epi);
    } else {
        hipLaunchKernelGGL((gemm_mfma<BM, BN, WM, WN, FMT, false, 16>), dim3(grid), dim3(256), 0, s, a, b, c, m, n,
                           k, static_cast<int>(mt), static_cast<int>(tiles), splits, kts, no, epi);
    }
    return hipGetLastError();
}

// Tile shapes compiled in, with their occupancy and sustained efficiency.
// The efficiencies and the co-residency factors in choose_plan were fitted
// to measured run times of every (tile, split) choice on MI355X for the
// M = 512 prefill shapes and the Q8_0 M sweep (M = 2 .. 64).
constexpr TileCfg kCfgs[] = {
    {128, 128, 2, 0.90}, {128, 96, 2, 0.873}, {128, 64, 2, 0.837}, {64, 128, 2, 0.837},
    {64, 64, 4, 0.76},   {32, 128, 3, 0.70},  {16, 128, 3, 0.35},  {16, 64, 6, 0.30},
};

// Cost model over tile shapes and K splits, in CU clock cycles.  The busiest
// CU runs per_cu workgroups, co = min(per_cu, occ) of them at once; a CU with
// a single workgroup (one wave per SIMD) loses latency hiding (factor 0.6),
// two recover most of it (0.92).  Weight streaming bounds the time from
// below; a split adds the partial-sum pass.
// The GLU epilogue pairs fragment fj with fj + FN/2 inside a wave: it needs an
// even number of 16-column fragments per wave (WN = 4 for BM = 16, else 2).
bool glu_ok(const TileCfg &t) { return (t.bn / (t.bm == 16 ? 4 : 2) / 16) % 2 == 0; }

Plan choose_plan(int64_t m, int64_t n, int64_t k, int fmt, int cus, bool glu = false) {
    const int64_t ktiles = (k + BK - 1) / BK;
    const double wbytes = fmt == FMT_F16 ? 2.0 * n * k
                          : static_cast<double>(n) * (k / 32) * (fmt == FMT_Q4_0 ? kQ4BlockBytes : kQ8BlockBytes);
    const double hbm_bytes_per_cycle = 6.0e12 / 2.4e9;  // sustained, whole chip
    Plan best{kCfgs[0], 1, static_cast<int>(ktiles)};
    double best_t = 1e300;
    for (const TileCfg &t : kCfgs) {
        if (t.bm > 16 && t.bm >= 2 * m) continue;  // mostly padding rows
        if (glu && !glu_ok(t)) continue;
        const int64_t tiles = ((m + t.bm - 1) / t.bm) * ((n + t.bn - 1) / t.bn);
        for (int sp : {1, 2, 3, 4, 6, 8, 12, 16}) {
            const int64_t kts = (ktiles + sp - 1) / sp;
            const int64_t splits = (ktiles + kts - 1) / kts;  // no empty split
            if (splits != sp && sp != 1) continue;
            if (sp > 1 && kts < 4) continue;
            const int64_t wgs = tiles * splits;
            if (wgs > 0x7fffffffLL) continue;
            const int64_t per_cu = (wgs + cus - 1) / cus;
            const int64_t co = std::min<int64_t>(per_cu, t.occ);
            const double f = co <= 1 ? 0.6 : co == 2 ? 0.92 : 1.0;
            double est = per_cu * (2.0 * t.bm * t.bn * BK * kts) / (256.0 * t.eff * f) +
                         2000.0 * static_cast<double>((per_cu + co - 1) / co);
            const double mt = static_cast<double>((m + t.bm - 1) / t.bm);
            est = std::max(est, wbytes * std::min(mt, 4.0) / hbm_bytes_per_cycle);
            if (splits > 1) est += 2.0 * splits * m * n * 4.0 / hbm_bytes_per_cycle + 1000.0;
            if (est < best_t * 0.98) {
                best_t = est;
                best = Plan{t, static_cast<int>(splits), static_cast<int>(kts)};
            }
        }
    }
    return best;
}

// n = weight rows, no = output columns.
template <int FMT>
hipError_t dispatch_tile(const Plan &p, const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k,
                         bool vec, hipStream_t s, int64_t no, int epi) {
    const int sp = p.splits, kts = p.kts;
    const TileCfg t = p.t;
    if (t.bm == 128 && t.bn == 128) return run<128, 128, 2, 2, FMT>(a, b, c, m, n, k, vec, sp, kts, s, no, epi);
    if (t.bm == 128 && t.bn == 96) return run<128, 96, 2, 2, FMT>(a, b, c, m, n, k, vec, sp, kts, s, no, epi);
    if (t.bm == 128 && t.bn == 64) return run<128, 64, 2, 2, FMT>(a, b, c, m, n, k, vec, sp, kts, s, no, epi);
    if (t.bm == 64 && t.bn == 128) return run<64, 128, 2, 2, FMT>(a, b, c, m, n, k, vec, sp, kts, s, no, epi);
    if (t.bm == 64 && t.bn == 64) return run<64, 64, 2, 2, FMT>(a, b, c, m, n, k, vec, sp, kts, s, no, epi);
    if (t.bm == 32 && t.bn == 128) return run<32, 128, 2, 2, FMT>(a, b, c, m, n, k, vec, sp, kts, s, no, epi);
    if (t.bm == 16 && t.bn == 128) return run<16, 128, 1, 4, FMT>(a, b, c, m, n, k, vec, sp, kts, s, no, epi);
    return run<16, 64, 1, 4, FMT>(a, b, c, m, n, k, vec, sp, kts, s, no, epi);
}

std::atomic<uint64_t> g_plan_override{0};  // bm | bn << 16 | splits << 32; 0 = none

bool known_tile(int bm, int bn) {
    for (const TileCfg &t : kCfgs)
        if (t.bm == bm && t.bn == bn) return true;
    return false;
}

// A forced tile that cannot take the GLU epilogue falls back to the model.
Plan planned(int64_t m, int64_t n, int64_t k, int fmt, int cus, bool glu = false) {
    const uint64_t o = g_plan_override.load(std::memory_order_relaxed);
    if (o == 0) return choose_plan(m, n, k, fmt, cus, glu);
    const int bm = static_cast<int>(o & 0xffff), bn = static_cast<int>((o >> 16) & 0xffff);
    if (glu && !glu_ok(TileCfg{bm, bn, 1, 1.0})) return choose_plan(m, n, k, fmt, cus, glu);
    const int64_t ktiles = (k + BK - 1) / BK;
    const int64_t want = std::max<int64_t>(1, std::min<int64_t>(static_cast<int64_t>(o >> 32), ktiles));
    const int64_t kts = (ktiles + want - 1) / want;
    TileCfg t = kCfgs[0];
    for (const TileCfg &c : kCfgs)
        if (c.bm == bm && c.bn == bn) t = c;
    return Plan{t, static_cast<int>((ktiles + kts - 1) / kts), static_cast<int>(kts)};
}

// n = output columns; the weights have nw = n (or 2n for the GLU epilogue) rows.
template <int FMT>
hipError_t dispatch(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, bool vec,
                    hipStream_t s, int cus, int epi) {
    const int64_t nw = epi == kEpiGlu ? 2 * n : n;
    Plan p = planned(m, nw, k, FMT, cus, epi == kEpiGlu);
    if (p.splits == 1) return dispatch_tile<FMT>(p, a, b, c, m, nw, k, vec, s, n, epi);
    // Split K: partial tiles go to the device's scratch buffer, then one pass
    // sums them in split order and applies the epilogue.
    ScratchLease lease;
    void *scratch = nullptr;
    const size_t bytes = static_cast<size_t>(p.splits) * static_cast<size_t>(m) * static_cast<size_t>(nw) * 4;
    hipError_t e = lease.acquire(bytes, s, &scratch);
    if (e != hipSuccess) return e;
    float *partial = static_cast<float *>(scratch);
    e = dispatch_tile<FMT>(p, a, b, partial, m, nw, k, vec, s, n, epi);
    if (e == hipSuccess) e = launch_reduce_splits(partial, c, m, n, nw, p.splits, epi, s);
    const hipError_t er = lease.release();
    return e != hipSuccess ? e : er;
}

}  // namespace

hipError_t launch_reduce_splits(const float *partial, float *c, int64_t m, int64_t no, int64_t nw, int splits,
                                int epi, hipStream_t s) {
    if (m <= 0 || no <= 0) return hipSuccess;
    const bool vec = no % 4 == 0 && reinterpret_cast<uintptr_t>(c) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(partial) % 16 == 0;
    const int w = vec ? 4 : 1;
    const int64_t gx = (no + 256 * w - 1) / (256 * w);
    if (gx > 0x7fffffffLL) return hipErrorInvalidValue;
    // Enough rows per launch for about 2048 workgroups; the rest are strided.
    const int64_t gy = std::max<int64_t>(1, std::min<int64_t>({m, 65535, (2048 + gx - 1) / gx}));
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
    if (vec)
        hipLaunchKernelGGL(reduce_splits<4>, grid, dim3(256), 0, s, partial, c, m, no, nw, splits, epi);
    else
        hipLaunchKernelGGL(reduce_splits<1>, grid, dim3(256), 0, s, partial, c, m, no, nw, splits, epi);
    return hipGetLastError();
}

void gemm_plan(int64_t m, int64_t n, int64_t k, int fmt, int cus, int *bm, int *bn, int *splits) {
    const Plan p = planned(m, n, k, fmt, cus);
    *bm = p.t.bm;
    *bn = p.t.bn;
    *splits = p.splits;
}

bool set_gemm_plan_override(int bm, int bn, int splits) {
    if (bm == 0 && bn == 0 && splits == 0) {
        g_plan_override.store(0, std::memory_order_relaxed);
        return true;
    }
    if (!known_tile(bm, bn) || splits < 1 || splits > 64) return false;
    g_plan_override.store(static_cast<uint64_t>(bm) | (static_cast<uint64_t>(bn) << 16) |
                              (static_cast<uint64_t>(splits) << 32),
                          std::memory_order_relaxed);
    return true;
}

hipError_t launch_gemm(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                       hipStream_t s, int epi) {
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    const bool a16 = (reinterpret_cast<uintptr_t>(a) & 15u) == 0;
    const bool b16 = (reinterpret_cast<uintptr_t>(b) & 15u) == 0;
    if (fmt == FMT_F16) {
        const bool vec = a16 && b16 && (k % 8 == 0);
        return dispatch<FMT_F16>(a, b, c, m, n, k, vec, s, di.cus, epi);
    }
    const bool vec = a16;  // K % 32 == 0 always holds for Q8_0 and Q4_0
    if (fmt == FMT_Q4_0) return dispatch<FMT_Q4_0>(a, b, c, m, n, k, vec, s, di.cus, epi);
    return dispatch<FMT_Q8_0>(a, b, c, m, n, k, vec, s, di.cus, epi);
}

}  // namespace wq
