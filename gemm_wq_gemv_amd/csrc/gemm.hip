// Prefill GEMM (M > 1): C[M,N] = A[M,K] . B[N,K]^T with f16 or Q8_0 weights,
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
//    WM x WN and each owns a (BM/WM) x (BN/WN) sub-tile made of 16x16 blocks,
//    each block accumulated by v_mfma_f32_16x16x4_f32 in four AGPR/VGPRs.
//  * The K loop steps by BK = 32, exactly one Q8_0 block per weight row.  Each
//    step stages the A tile (f32) and the weight tile, widened (f16) or
//    dequantised (d*q, exact in f32), into LDS, double-buffered: the global
//    loads of step k+1 are in flight while the matrix cores work on step k,
//    with one barrier per step.
//  * The reduction index inside a 32-wide step is permuted so that every lane
//    reads 8 consecutive k (two 128-bit LDS reads) per 16-row fragment: in MFMA
//    step t the lane group g = lane/16 supplies k = 8g + t.  The sum over k is
//    unchanged; only its order differs.
//  * Rows of the LDS tiles are padded by 16 bytes to spread LDS banks.
//  * Workgroup -> tile mapping is XCD-aware: workgroups are dealt round-robin
//    to the 8 XCDs, so consecutive workgroup ids on one XCD are given tiles
//    that share weight columns (M-fastest tile order) and hit the same L2.
#include "wq_internal.h"

namespace wq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int BK = 32;
constexpr int PAD = 4;            // floats of padding per LDS row
constexpr int LDP = BK + PAD;     // LDS row pitch in floats
constexpr int kXcds = 8;
constexpr int kQ8BlockBytes = 34;

enum { FMT_F16 = 0, FMT_Q8_0 = 1 };

// Tile id for workgroup `bid` of `tiles`, so that XCD x (= bid % 8) receives a
// contiguous range of tile ids.
__device__ __forceinline__ int xcd_tile(int bid, int tiles) {
    const int q = tiles / kXcds, r = tiles % kXcds;
    const int x = bid % kXcds, local = bid / kXcds;
    return x < r ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

template <int BM, int BN, int WM, int WN, int FMT, bool VEC>
struct Gemm {
    static_assert(WM * WN == 4, "four waves");
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static_assert(FM >= 1 && FN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
    static constexpr int A_ITERS = (BM * 8 + 255) / 256;    // float4 chunks of A per thread
    static constexpr int B16_ITERS = (BN * 4 + 255) / 256;  // uint4 chunks of f16 B per thread
    static constexpr int B8_ITERS = (BN * 2 + 255) / 256;   // half blocks of Q8_0 B per thread

    struct Regs {
        float4 a[A_ITERS];
        uint4 b16[FMT == FMT_F16 ? B16_ITERS : 1];
        uint32_t d8[FMT == FMT_Q8_0 ? B8_ITERS : 1];
        uint32_t q8[FMT == FMT_Q8_0 ? B8_ITERS : 1][8];
    };

    // Global -> registers for the k-tile starting at k0.
    static __device__ __forceinline__ void load(Regs &r, const float *__restrict__ a,
                                                const void *__restrict__ bw, int64_t M, int64_t N,
                                                int64_t K, int64_t m0, int64_t n0, int64_t k0,
                                                int tid) {
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int row = (tid >> 3) + 32 * i;
            const int c4 = tid & 7;
            const int64_t gm = m0 + row, gk = k0 + 4 * c4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (row < BM && gm < M) {
                const float *p = a + gm * K + gk;
                if (VEC) {
                    if (gk + 4 <= K) v = *reinterpret_cast<const float4 *>(p);
                } else {
                    if (gk + 0 < K) v.x = p[0];
                    if (gk + 1 < K) v.y = p[1];
                    if (gk + 2 < K) v.z = p[2];
                    if (gk + 3 < K) v.w = p[3];
                }
            }
            r.a[i] = v;
        }
        if constexpr (FMT == FMT_F16) {
            const uint16_t *b = static_cast<const uint16_t *>(bw);
#pragma unroll
            for (int i = 0; i < B16_ITERS; ++i) {
                const int row = (tid >> 2) + 64 * i;
                const int c8 = tid & 3;
                const int64_t gn = n0 + row, gk = k0 + 8 * c8;
                uint4 v = make_uint4(0u, 0u, 0u, 0u);
                if (row < BN && gn < N) {
                    const uint16_t *p = b + gn * K + gk;
                    if (VEC) {
                        if (gk + 8 <= K) v = *reinterpret_cast<const uint4 *>(p);
                    } else {
                        uint32_t h[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) h[u] = (gk + u < K) ? p[u] : 0u;
                        v = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                       h[6] | (h[7] << 16));
                    }
                }
                r.b16[i] = v;
            }
        } else {
            const uint8_t *b = static_cast<const uint8_t *>(bw);
            const int64_t row_bytes = (K >> 5) * kQ8BlockBytes;
            const int64_t kb = k0 >> 5;
#pragma unroll
            for (int i = 0; i < B8_ITERS; ++i) {
                const int row = (tid >> 1) + 128 * i;
                const int h = tid & 1;
                const int64_t gn = n0 + row;
                r.d8[i] = 0u;
#pragma unroll
                for (int u = 0; u < 8; ++u) r.q8[i][u] = 0u;
                if (row < BN && gn < N) {
                    const uint16_t *blk =
                        reinterpret_cast<const uint16_t *>(b + gn * row_bytes + kb * kQ8BlockBytes);
                    r.d8[i] = blk[0];
#pragma unroll
                    for (int u = 0; u < 8; ++u) r.q8[i][u] = blk[1 + 8 * h + u];
                }
            }
        }
    }

    // Registers -> LDS (A as is; weights widened or dequantised to f32).
    static __device__ __forceinline__ void store(const Regs &r, float (*As)[LDP], float (*Bs)[LDP],
                                                 int tid) {
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int row = (tid >> 3) + 32 * i;
            if (row < BM) *reinterpret_cast<float4 *>(&As[row][4 * (tid & 7)]) = r.a[i];
        }
        if constexpr (FMT == FMT_F16) {
#pragma unroll
            for (int i = 0; i < B16_ITERS; ++i) {
                const int row = (tid >> 2) + 64 * i;
                if (row < BN) {
                    const uint4 v = r.b16[i];
                    float4 lo = make_float4(half_bits_to_float(v.x & 0xffffu), half_bits_to_float(v.x >> 16),
                                            half_bits_to_float(v.y & 0xffffu), half_bits_to_float(v.y >> 16));
                    float4 hi = make_float4(half_bits_to_float(v.z & 0xffffu), half_bits_to_float(v.z >> 16),
                                            half_bits_to_float(v.w & 0xffffu), half_bits_to_float(v.w >> 16));
                    float *dst = &Bs[row][8 * (tid & 3)];
                    *reinterpret_cast<float4 *>(dst) = lo;
                    *reinterpret_cast<float4 *>(dst + 4) = hi;
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

    static __device__ __forceinline__ void compute(v4f (&acc)[FM][FN], const float (*As)[LDP],
                                                   const float (*Bs)[LDP], int wm, int wn, int lane) {
        const int li = lane & 15, lg = lane >> 4;
        float af[FM][8], bf[FN][8];
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            const float *src = &As[wm * WTM + 16 * f + li][8 * lg];
            const float4 x = *reinterpret_cast<const float4 *>(src);
            const float4 y = *reinterpret_cast<const float4 *>(src + 4);
            af[f][0] = x.x; af[f][1] = x.y; af[f][2] = x.z; af[f][3] = x.w;
            af[f][4] = y.x; af[f][5] = y.y; af[f][6] = y.z; af[f][7] = y.w;
        }
#pragma unroll
        for (int f = 0; f < FN; ++f) {
            const float *src = &Bs[wn * WTN + 16 * f + li][8 * lg];
            const float4 x = *reinterpret_cast<const float4 *>(src);
            const float4 y = *reinterpret_cast<const float4 *>(src + 4);
            bf[f][0] = x.x; bf[f][1] = x.y; bf[f][2] = x.z; bf[f][3] = x.w;
            bf[f][4] = y.x; bf[f][5] = y.y; bf[f][6] = y.z; bf[f][7] = y.w;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][t], bf[j][t], acc[i][j], 0, 0, 0);
    }
};

template <int BM, int BN, int WM, int WN, int FMT, bool VEC>
__global__ __launch_bounds__(256) void gemm_mfma(const float *__restrict__ a, const void *__restrict__ bw,
                                                 float *__restrict__ c, int64_t M, int64_t N, int64_t K,
                                                 int mtiles, int tiles) {
    using G = Gemm<BM, BN, WM, WN, FMT, VEC>;
    __shared__ float As[2][BM][LDP];
    __shared__ float Bs[2][BN][LDP];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int tile = xcd_tile(blockIdx.x, tiles);
    const int64_t m0 = static_cast<int64_t>(tile % mtiles) * BM;
    const int64_t n0 = static_cast<int64_t>(tile / mtiles) * BN;

    v4f acc[G::FM][G::FN];
#pragma unroll
    for (int i = 0; i < G::FM; ++i)
#pragma unroll
        for (int j = 0; j < G::FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int64_t ktiles = (K + BK - 1) / BK;
    typename G::Regs r;
    G::load(r, a, bw, M, N, K, m0, n0, 0, tid);
    G::store(r, As[0], Bs[0], tid);
    __syncthreads();
    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int cur = static_cast<int>(kt & 1);
        const bool more = kt + 1 < ktiles;
        if (more) G::load(r, a, bw, M, N, K, m0, n0, (kt + 1) * BK, tid);
        G::compute(acc, As[cur], Bs[cur], wm, wn, lane);
        if (more) G::store(r, As[cur ^ 1], Bs[cur ^ 1], tid);
        __syncthreads();
    }

    // D[i][j] of a 16x16 block: lane l, register v holds row 4*(l/16) + v, column l%16.
    const int li = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int i = 0; i < G::FM; ++i) {
#pragma unroll
        for (int j = 0; j < G::FN; ++j) {
            const int64_t col = n0 + wn * G::WTN + 16 * j + li;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = m0 + wm * G::WTM + 16 * i + 4 * lg + v;
                if (row < M && col < N) c[row * N + col] = acc[i][j][v];
            }
        }
    }
}

struct TileCfg {
    int bm, bn;
};

template <int BM, int BN, int WM, int WN, int FMT>
hipError_t run(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, bool vec,
               hipStream_t s) {
    const int64_t mt = (m + BM - 1) / BM, nt = (n + BN - 1) / BN;
    const int64_t tiles = mt * nt;
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    if (trace_enabled())
        fprintf(stderr, "[wqmm] gemm_mfma<BM=%d,BN=%d,WM=%d,WN=%d,fmt=%d,vec=%d> m=%lld n=%lld k=%lld grid=%lld\n",
                BM, BN, WM, WN, FMT, vec ? 1 : 0, (long long)m, (long long)n, (long long)k, (long long)tiles);
    if (vec)
        hipLaunchKernelGGL((gemm_mfma<BM, BN, WM, WN, FMT, true>), dim3(tiles), dim3(256), 0, s, a, b, c, m, n,
                           k, static_cast<int>(mt), static_cast<int>(tiles));
    else
        hipLaunchKernelGGL((gemm_mfma<BM, BN, WM, WN, FMT, false>), dim3(tiles), dim3(256), 0, s, a, b, c, m, n,
                           k, static_cast<int>(mt), static_cast<int>(tiles));
    return hipGetLastError();
}

// Candidate tiles: (BM, BN).  The estimate prefers configurations that fill
// every CU evenly and, among those, larger tiles (fewer re-reads of A and B).
constexpr TileCfg kCfgs[] = {{128, 128}, {128, 96}, {128, 64}, {64, 128}, {64, 64}, {32, 128}, {16, 256}, {16, 128}};

double tile_efficiency(const TileCfg &t) {
    // Relative throughput per CU of one tile shape when every CU is busy
    // (bigger wave tiles amortise LDS traffic and barriers better).
    const double area = static_cast<double>(t.bm) * t.bn;
    return area / (area + 2048.0);
}

TileCfg choose_tile(int64_t m, int64_t n, int cus) {
    TileCfg best = kCfgs[0];
    double best_t = 1e300;
    for (const TileCfg &t : kCfgs) {
        const int64_t mt = (m + t.bm - 1) / t.bm, nt = (n + t.bn - 1) / t.bn;
        const int64_t tiles = mt * nt;
        const int per_cu = 1;
        const int64_t rounds = (tiles + static_cast<int64_t>(cus) * per_cu - 1) / (static_cast<int64_t>(cus) * per_cu);
        // time ~ rounds * tile area (padded M included) / efficiency
        const double est = static_cast<double>(rounds) * t.bm * t.bn / tile_efficiency(t);
        if (est < best_t * 0.999) {
            best_t = est;
            best = t;
        }
    }
    return best;
}

template <int FMT>
hipError_t dispatch(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, bool vec,
                    hipStream_t s, int cus) {
    const TileCfg t = choose_tile(m, n, cus);
    if (t.bm == 128 && t.bn == 128) return run<128, 128, 2, 2, FMT>(a, b, c, m, n, k, vec, s);
    if (t.bm == 128 && t.bn == 96) return run<128, 96, 2, 2, FMT>(a, b, c, m, n, k, vec, s);
    if (t.bm == 128 && t.bn == 64) return run<128, 64, 2, 2, FMT>(a, b, c, m, n, k, vec, s);
    if (t.bm == 64 && t.bn == 128) return run<64, 128, 2, 2, FMT>(a, b, c, m, n, k, vec, s);
    if (t.bm == 64 && t.bn == 64) return run<64, 64, 2, 2, FMT>(a, b, c, m, n, k, vec, s);
    if (t.bm == 32 && t.bn == 128) return run<32, 128, 2, 2, FMT>(a, b, c, m, n, k, vec, s);
    if (t.bm == 16 && t.bn == 256) return run<16, 256, 1, 4, FMT>(a, b, c, m, n, k, vec, s);
    return run<16, 128, 1, 4, FMT>(a, b, c, m, n, k, vec, s);
}

}  // namespace

hipError_t launch_gemm(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                       hipStream_t s) {
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    const bool a16 = (reinterpret_cast<uintptr_t>(a) & 15u) == 0;
    const bool b16 = (reinterpret_cast<uintptr_t>(b) & 15u) == 0;
    if (fmt == FMT_F16) {
        const bool vec = a16 && b16 && (k % 8 == 0);
        return dispatch<FMT_F16>(a, b, c, m, n, k, vec, s, di.cus);
    }
    const bool vec = a16;  // K % 32 == 0 always holds for Q8_0
    return dispatch<FMT_Q8_0>(a, b, c, m, n, k, vec, s, di.cus);
}

}  // namespace wq
