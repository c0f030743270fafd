// Prefill GEMM on the f16 matrix cores with f32 results: C[M,N] = A[M,K] . B[N,K]^T
// for f32 A and f16, Q8_0 or Q4_0 weights, M > 1.
//
// Operation: dispatch_gemm / dispatch_gemm_q8 (lattice-inference 0.9.0,
// dispatch.rs) for M > 1; the kernels matmul_bt, gemm_q8 and gemm_q4_tiled
// (lattice-inference 0.1.2, metal_qwen35.rs) are the tiling prior art.  Within
// a quantized block the codes are summed against the activations and the block
// scale applied once, c = sum_j d_j sum_i q_i a_i, as in those kernels.
//
// Arithmetic.  The f16 matrix rate of CDNA4 is sixteen times its f32 rate, so
// the f32 operand is carried as two f16 numbers: for row r of A a power of two
// s_r is chosen so that max_k |a[r,k]| s_r lies in [2^14, 2^15), and
// hi = f16(a s_r), lo = f16(a s_r - hi).  hi + lo equals a s_r to at least 22
// significant bits (f32 has 24).  Weights are exact in f16: f16 weights as
// they are, quantized codes (-128..127, -8..7) as small integers.  Every
// product of two f16 numbers is exact in f32, so one 16x16x32 matrix step over
// hi and one over lo give sum_k (hi + lo) w in f32 accumulation; the row scale
// 1 / s_r (and a quantized block's d) is applied in f32 by the lane.  The
// representation error of A is at most 2^-22 |a| per element, far inside the
// product's f32 rounding over K terms.
//
// CDNA4 layout:
//  * One pass over A (hl_split) writes the hi and lo halves of every row to
//    scratch, per 32-column tile as 32 hi then 32 lo numbers (128 bytes), and
//    the row's 1 / s_r.
//  * The product runs in workgroups of 4 waves (2 x 2) over BM x BN tiles of C;
//    the wave tile is made of 16x16 blocks, each accumulated by
//    v_mfma_f32_16x16x32_f16.  The K loop steps by 32 = one quantized block =
//    one matrix step.  Per step the A tile (hi and lo) and the weight tile
//    (f16, or codes turned into f16 integers with the scales beside them) are
//    staged in LDS, double-buffered, with the next tile loading from memory
//    meanwhile (one barrier per step).
//  * Lane l of a matrix step holds 8 consecutive k (8 (l / 16) .. + 7) of
//    row l % 16 of both operands: 16-byte LDS reads; rows padded to 144 / 80
//    bytes so 8 consecutive rows fall on distinct banks.
//  * Quantized weights: per block and output block the two matrix steps start
//    from zero and the lane adds d times the result to its accumulators.
//  * K split across workgroups where the tiles alone cannot fill the chip;
//    partial tiles are summed in split order by a second pass (deterministic).
//    Workgroup -> tile mapping as in the fp32 GEMM (XCD-aware).
// Requires K % 32 == 0, 16-byte aligned a and b.
#include "wq_internal.h"

#include <algorithm>
#include <atomic>
#include <cfloat>
#include <cstdio>
#include <type_traits>

namespace wq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { HL_F16 = 0, HL_Q8_0 = 1, HL_Q4_0 = 2 };
constexpr int kBK = 32;      // k per step: one quantized block, one matrix step
constexpr int kAPitch = 72;  // f16 per LDS row of the A tile: hi 32, lo 32, padding 8
constexpr int kBPitch = 40;  // f16 per LDS row of the weight tile: 32, padding 8
constexpr int kStages = 2;   // register sets of tiles in flight between global memory and LDS

// ------------------------------------------------------------------ split --
// Split of 8 consecutive elements (x * s) into their hi and lo halves.
__device__ __forceinline__ void hl_pair(const float4 &v0, const float4 &v1, float s, h8 &hi, h8 &lo) {
    const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const float y = x[u] * s;
        const _Float16 h = static_cast<_Float16>(y);
        const float hf = static_cast<float>(h);
        hi[u] = h;
        lo[u] = __builtin_isfinite(hf) ? static_cast<_Float16>(y - hf) : static_cast<_Float16>(0.f);
    }
}

__device__ __forceinline__ float amax8(const float4 &v0, const float4 &v1) {
    return fmaxf(fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))),
                 fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
}

// Exponent e of s_r = 2^e for a row maximum mx (hl_split).
__device__ __forceinline__ int hl_exponent(float mx) {
    if (!(mx > 0.f && mx <= FLT_MAX)) return 0;
    int ex;
    frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
    return min(max(15 - ex, -113), 126);
}

// Row r of A (grid: one workgroup per row): hi / lo halves into
// ahl[r][t][0..31] (hi) and ahl[r][t][32..63] (lo) for 32-column tile t, and
// rs[r] = 1 / s_r.  An all-zero or non-finite row keeps s_r = 1; s_r is held
// to [2^-113, 2^126] so that both it and 1 / s_r are normal f32 numbers.  A
// non-finite hi gets lo = 0, so infinities and NaN reach the sums as in f32.
// Thread t takes the 8-element chunks t, t + 256, ...: up to kSplitRegs of them
// stay in registers between the maximum and the split (one read of the row);
// longer rows are read twice.
constexpr int kSplitRegs = 8;
__global__ __launch_bounds__(256) void hl_split(const float *__restrict__ a, uint16_t *__restrict__ ahl,
                                                float *__restrict__ rs, int64_t K) {
    __shared__ float wave_max[4];
    const int64_t row = blockIdx.x;
    const float *ar = a + row * K;
    uint16_t *out = ahl + row * 2 * K;
    const int tid = threadIdx.x;
    const bool in_regs = K <= 256 * 8 * kSplitRegs;
    float4 v[kSplitRegs][2];
    float mx = 0.f;
    if (in_regs) {
#pragma unroll
        for (int u = 0; u < kSplitRegs; ++u) {
            const int64_t j = (static_cast<int64_t>(tid) + 256 * u) * 8;
            v[u][0] = v[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < K) {
                v[u][0] = *reinterpret_cast<const float4 *>(ar + j);
                v[u][1] = *reinterpret_cast<const float4 *>(ar + j + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < kSplitRegs; ++u) mx = fmaxf(mx, amax8(v[u][0], v[u][1]));
    } else {
        for (int64_t j = static_cast<int64_t>(tid) * 8; j < K; j += 256 * 8)
            mx = fmaxf(mx, amax8(*reinterpret_cast<const float4 *>(ar + j), *reinterpret_cast<const float4 *>(ar + j + 4)));
    }
    mx = group_max<64>(mx);
    if ((tid & 63) == 0) wave_max[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    const int e = hl_exponent(mx);
    const float s = ldexpf(1.f, e);
    if (tid == 0) rs[row] = ldexpf(1.f, -e);
    auto put = [&](int64_t j, const float4 &v0, const float4 &v1) {
        h8 hi, lo;
        hl_pair(v0, v1, s, hi, lo);
        uint16_t *dst = out + (j >> 5) * 64 + (j & 31);
        *reinterpret_cast<h8 *>(dst) = hi;
        *reinterpret_cast<h8 *>(dst + 32) = lo;
    };
    if (in_regs) {
#pragma unroll
        for (int u = 0; u < kSplitRegs; ++u) {
            const int64_t j = (static_cast<int64_t>(tid) + 256 * u) * 8;
            if (j < K) put(j, v[u][0], v[u][1]);
        }
    } else {
        for (int64_t j = static_cast<int64_t>(tid) * 8; j < K; j += 256 * 8)
            put(j, *reinterpret_cast<const float4 *>(ar + j), *reinterpret_cast<const float4 *>(ar + j + 4));
    }
}

// ---------------------------------------------------------------- product --
template <int BM, int BN, int FMT>
struct HTile {
    static constexpr int WTM = BM / 2, WTN = BN / 2;  // wave tile (2 x 2 waves)
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static_assert(FM >= 1 && FN >= 2 && FN % 2 == 0, "wave tile");
    static constexpr bool QUANT = FMT != HL_F16;
    static constexpr int A_IT = BM / 32;             // 16-byte chunks of the A tile per thread
    static constexpr int B_IT = BN / 64;             // 16-byte chunks of an f16 weight tile per thread
    static constexpr int Q_IT = (BN + 127) / 128;    // half blocks per thread (quantized)
    static constexpr int QBB = FMT == HL_Q4_0 ? 18 : 34;

    // Tile row that thread tid stages in pass i (A: 16-byte chunk tid % 8 of
    // 32 rows per pass; f16 weights: chunk tid % 4 of 64 rows; quantized: half
    // tid % 2 of 128 rows).  The rows a group of 16 lanes writes are chosen so
    // that its 16-byte LDS stores fall on distinct banks (row pitches of 9 and
    // 5 sixteen-byte units): A rows q and q + 8; f16 weight rows q, q + 4,
    // q + 8, q + 12; quantized rows {0, 1, 4, 5, 8, 9, 12, 13} + 2 (group & 1).
    static __device__ __forceinline__ int a_row(int tid, int i) {
        const int g16 = tid >> 4;
        return 32 * i + (g16 & 7) + 16 * (g16 >> 3) + 8 * ((tid >> 3) & 1);
    }
    static __device__ __forceinline__ int b_row(int tid, int i) {
        const int g16 = tid >> 4;
        return 64 * i + 16 * (g16 >> 2) + (g16 & 3) + 4 * ((tid >> 2) & 3);
    }
    static __device__ __forceinline__ int q_row(int tid, int i) {
        const int g16 = tid >> 4, idx = (tid & 15) >> 1;
        return 128 * i + 16 * (g16 >> 1) + 2 * (g16 & 1) + (idx & 1) + 4 * (idx >> 1);
    }

    // Quantized half rows: the dwords holding bytes [start, start + 18)
    // (Q8_0: scale and codes 0..15, or codes 16..31) or [start, start + 10)
    // (Q4_0), read from the dword boundary at or below start; sh = start % 4.
    static constexpr int QD = FMT == HL_Q4_0 ? 3 : 5;  // dwords per half row
    struct Regs {
        u32x4 a[A_IT];
        u32x4 b[QUANT ? 1 : B_IT];
        uint32_t w[QUANT ? Q_IT : 1][QD];
        uint32_t sh[QUANT ? Q_IT : 1];
    };

    // Weight row feeding row `row` of the weight tile (clamped: rows past N
    // feed outputs that are never stored).  GLU (N = 2 NO weight rows, gate
    // then up; n0 = the tile's first output column): the first half of each
    // wave's WTN rows are gate rows, the second half the up rows of the same
    // output columns, so fragment fj and fj + FN / 2 pair up in a lane.
    static __device__ __forceinline__ int64_t brow(int64_t n0, int row, int64_t N, int64_t NO, bool glu) {
        if (!glu) return min<int64_t>(n0 + row, N - 1);
        const int wn = row / WTN, within = row % WTN;
        const int64_t oc = min<int64_t>(n0 + wn * (WTN / 2) + within % (WTN / 2), NO - 1);
        return within < WTN / 2 ? oc : NO + oc;
    }

    // Global -> registers for k-tile kt.  Every thread issues the same loads
    // on every call (rows clamped), so the pipeline's load counts are fixed.
    static __device__ __forceinline__ void load(Regs &r, const uint16_t *__restrict__ ahl,
                                                const void *__restrict__ bw, __amdgpu_buffer_rsrc_t rb, int64_t M,
                                                int64_t N, int64_t K,
                                                int64_t m0, int64_t n0, int64_t kt, int tid, int64_t NO,
                                                bool glu) {
#pragma unroll
        for (int i = 0; i < A_IT; ++i) {
            const int row = a_row(tid, i);
            const int64_t gm = min<int64_t>(m0 + row, M - 1);
            r.a[i] = *reinterpret_cast<const u32x4 *>(ahl + gm * 2 * K + kt * 64 + 8 * (tid & 7));
        }
        if constexpr (!QUANT) {
            const uint16_t *b = static_cast<const uint16_t *>(bw);
#pragma unroll
            for (int i = 0; i < B_IT; ++i) {
                const int row = b_row(tid, i);
                const int64_t gn = brow(n0, row, N, NO, glu);
                r.b[i] = *reinterpret_cast<const u32x4 *>(b + gn * K + kt * kBK + 8 * (tid & 3));
            }
        } else {
            // Thread half h of a block row (block at byte b0, even): Q8_0 h = 0
            // reads the scale and codes 0..15 from b0, h = 1 codes 16..31 from
            // b0 + 18; Q4_0 the scale and code bytes 0..7 from b0, bytes 8..15
            // from b0 + 10.  Whole dwords through the buffer resource (its
            // size rounded up to a dword; dwords past it read as zero).
            const int64_t row_bytes = (K >> 5) * QBB;
#pragma unroll
            for (int i = 0; i < Q_IT; ++i) {
                const int row = q_row(tid, i);
                if (row < BN) {
                    const int h = tid & 1;
                    const int64_t gn = brow(n0, row, N, NO, glu);
                    const uint32_t start = static_cast<uint32_t>(gn * row_bytes + kt * QBB) +
                                           static_cast<uint32_t>(h) * (FMT == HL_Q4_0 ? 10u : 18u);
                    const int base = static_cast<int>(start & ~3u);
                    r.sh[i] = start & 3u;
                    if constexpr (FMT == HL_Q8_0) {
                        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, base, 0, 0));
                        r.w[i][0] = v.x;
                        r.w[i][1] = v.y;
                        r.w[i][2] = v.z;
                        r.w[i][3] = v.w;
                        r.w[i][4] = __builtin_amdgcn_raw_buffer_load_b32(rb, base + 16, 0, 0);
                    } else {
                        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rb, base, 0, 0));
                        r.w[i][0] = v.x;
                        r.w[i][1] = v.y;
                        r.w[i][2] = __builtin_amdgcn_raw_buffer_load_b32(rb, base + 8, 0, 0);
                    }
                }
            }
        }
    }

    // Registers -> LDS.  Codes become f16 integers: a Q8_0 byte (xor 0x80)
    // becomes the low mantissa byte of 1024 (v_perm_b32), a Q4_0 nibble the
    // low mantissa bits, then 1152 (1032) is subtracted, exactly.
    static __device__ __forceinline__ void store(const Regs &r, uint16_t (*As)[kAPitch], uint16_t (*Bs)[kBPitch],
                                                 float *Ds, int tid) {
#pragma unroll
        for (int i = 0; i < A_IT; ++i) {
            *reinterpret_cast<u32x4 *>(&As[a_row(tid, i)][8 * (tid & 7)]) = r.a[i];
        }
        if constexpr (!QUANT) {
#pragma unroll
            for (int i = 0; i < B_IT; ++i) {
                *reinterpret_cast<u32x4 *>(&Bs[b_row(tid, i)][8 * (tid & 3)]) = r.b[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < Q_IT; ++i) {
                const int row = q_row(tid, i);
                if (row < BN) {
                    const int h = tid & 1;
                    // Code dwords start at byte cs of the loaded dwords (the
                    // scale comes first in half 0).
                    const uint32_t sh = r.sh[i], cs = sh + 2u * static_cast<uint32_t>(1 - h);
                    constexpr int NX = FMT == HL_Q8_0 ? 4 : 2;
                    uint32_t x[NX];
#pragma unroll
                    for (int j = 0; j < NX; ++j)
                        x[j] = cs == 2u ? __builtin_amdgcn_alignbyte(r.w[i][j + 1], r.w[i][j], 2)
                                        : (cs == 4u ? r.w[i][j + 1] : r.w[i][j]);
                    uint32_t o[8];
                    if constexpr (FMT == HL_Q8_0) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t v = x[j] ^ 0x80808080u;
                            o[2 * j] = __builtin_amdgcn_perm(0x64646464u, v, 0x04010400u);
                            o[2 * j + 1] = __builtin_amdgcn_perm(0x64646464u, v, 0x04030402u);
                        }
                    } else {
                        // Byte k of a code dword holds columns 2k (low nibble) and 2k + 1.
#pragma unroll
                        for (int j = 0; j < 2; ++j)
#pragma unroll
                            for (int k = 0; k < 4; ++k)
                                o[4 * j + k] = ((x[j] >> (8 * k)) & 0xFu) | (((x[j] >> (8 * k + 4)) & 0xFu) << 16) |
                                               0x64006400u;
                    }
                    const _Float16 bias = FMT == HL_Q8_0 ? static_cast<_Float16>(1152.f) : static_cast<_Float16>(1032.f);
                    const hh2 b2 = {bias, bias};
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        o[u] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(hh2, o[u]) - b2);
                    *reinterpret_cast<u32x4 *>(&Bs[row][16 * h]) = u32x4{o[0], o[1], o[2], o[3]};
                    *reinterpret_cast<u32x4 *>(&Bs[row][16 * h + 8]) = u32x4{o[4], o[5], o[6], o[7]};
                    if (h == 0) Ds[row] = half_bits_to_float(sh != 0u ? r.w[i][0] >> 16 : r.w[i][0] & 0xFFFFu);
                }
            }
        }
    }

    struct Frags {
        h8 hi[FM], lo[FM], b[FN];
    };

    static __device__ __forceinline__ void read_frags(Frags &f, float (&dcol)[FN], const uint16_t (*As)[kAPitch],
                                                      const uint16_t (*Bs)[kBPitch], const float *Ds, int wm, int wn,
                                                      int lane) {
        const int li = lane & 15, g = lane >> 4;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            f.hi[i] = *reinterpret_cast<const h8 *>(&As[wm * WTM + 16 * i + li][8 * g]);
            f.lo[i] = *reinterpret_cast<const h8 *>(&As[wm * WTM + 16 * i + li][32 + 8 * g]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            f.b[j] = *reinterpret_cast<const h8 *>(&Bs[wn * WTN + 16 * j + li][8 * g]);
            if constexpr (QUANT) dcol[j] = Ds[wn * WTN + 16 * j + li];
        }
    }

    // Output blocks j in [J0, J1) of one k-tile (dcol: the block scales of
    // the lane's weight row, quantized formats).
    template <int J0, int J1>
    static __device__ __forceinline__ void mma(f4 (&acc)[FM][FN], const Frags &f, const float (&dcol)[FN]) {
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            if constexpr (!QUANT) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.hi[i], f.b[j], acc[i][j], 0, 0, 0);
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.lo[i], f.b[j], acc[i][j], 0, 0, 0);
            } else {
                const f4 zero = {0.f, 0.f, 0.f, 0.f};
                f4 t[FM];
#pragma unroll
                for (int i = 0; i < FM; ++i) t[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.hi[i], f.b[j], zero, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < FM; ++i) t[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.lo[i], f.b[j], t[i], 0, 0, 0);
#pragma unroll
                for (int i = 0; i < FM; ++i) acc[i][j] += dcol[j] * t[i];
            }
        }
    }
};

template <int N>
using Int = std::integral_constant<int, N>;

// f(i + s, Int<s>) for s = S .. NS - 1.
template <int S, int NS, typename F>
__device__ __forceinline__ void unrolled_steps(F &f, int64_t i) {
    if constexpr (S < NS) {
        f(i + S, Int<S>{});
        unrolled_steps<S + 1, NS>(f, i);
    }
}

// The same for the last n - i < NS steps.
template <int S, int NS, typename F>
__device__ __forceinline__ void tail_steps(F &f, int64_t i, int64_t n) {
    if constexpr (S < NS - 1) {
        if (i + S < n) {
            f(i + S, Int<S>{});
            tail_steps<S + 1, NS>(f, i, n);
        }
    }
}

// Grid: tiles * splits workgroups.  Split s covers k-tiles [s kts, min(K / 32,
// (s + 1) kts)).  N = weight rows; NO = output columns (N, or N / 2 for GLU).
// One split: the tile goes to C [M, NO] through the epilogue.  Otherwise the
// scaled raw sums go to c + s M N (column = weight row) and reduce_splits sums
// them in split order and applies the epilogue.
template <int BM, int BN, int FMT, int NS>
__global__ __launch_bounds__(256) void gemm_hl(const uint16_t *__restrict__ ahl, const float *__restrict__ rs,
                                               const void *__restrict__ bw, float *__restrict__ c, int64_t M,
                                               int64_t N, int64_t K, int mtiles, int tiles, int kts, int splits,
                                               int64_t NO, int epi) {
    using T = HTile<BM, BN, FMT>;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][kAPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][kBPitch];
    __shared__ float Ds[2][T::QUANT ? BN : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int idx = xcd_tile(blockIdx.x, tiles * splits);
    const int tile = idx % tiles, split = idx / tiles;
    const bool glu = epi == kEpiGlu;
    const int64_t m0 = static_cast<int64_t>(tile % mtiles) * BM;
    const int64_t n0 = static_cast<int64_t>(tile / mtiles) * (glu ? BN / 2 : BN);
    const int64_t ktiles = K / kBK;
    const int64_t kt0 = static_cast<int64_t>(split) * kts;
    const int64_t nkt = min<int64_t>(ktiles, kt0 + kts) - kt0;  // >= 1 by construction
    // Quantized weights: N (K / 32) block bytes < 2^31 (checked by the host),
    // the resource's size rounded up to a dword.
    const uint32_t wbytes = T::QUANT ? static_cast<uint32_t>(N * (K >> 5) * T::QBB) : 0u;
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(bw), 0, static_cast<int>((wbytes + 3u) & ~3u), 0x00020000);

    f4 acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    // Tile i sits in LDS buffer i & 1.  NS register sets hold the tiles
    // i + 1 .. i + NS: at step i, set i % NS (its tile went to LDS during
    // step i - 1) starts loading tile i + NS, and set (i + 1) % NS, issued
    // NS - 1 steps earlier, goes to the other LDS buffer halfway through the
    // step's matrix work.  Tile indices past the end are clamped (the same
    // load count every step).
    auto ktile = [&](int64_t t) { return kt0 + min<int64_t>(t, nkt - 1); };
    typename T::Regs r[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) T::load(r[s], ahl, bw, rb, M, N, K, m0, n0, ktile(s), tid, NO, glu);
    T::store(r[0], As[0], Bs[0], Ds[0], tid);
    __syncthreads();

    auto step = [&](int64_t i, auto set) __attribute__((always_inline)) {
        constexpr int S = decltype(set)::value;
        T::load(r[S], ahl, bw, rb, M, N, K, m0, n0, ktile(i + NS), tid, NO, glu);
        // Keep these loads at the top of the step, so that the store below
        // waits only for loads issued NS - 1 steps earlier.
        __builtin_amdgcn_sched_barrier(0);
        const int cur = static_cast<int>(i & 1);
        typename T::Frags f;
        float dcol[T::FN];
        T::read_frags(f, dcol, As[cur], Bs[cur], Ds[cur], wm, wn, lane);
        T::template mma<0, T::FN / 2>(acc, f, dcol);
        // Unconditional (after the last step it writes a buffer nobody reads):
        // a conditional store would let the compiler sink the loads feeding
        // it to just before it, exposing their whole latency.
        T::store(r[(S + 1) % NS], As[cur ^ 1], Bs[cur ^ 1], Ds[cur ^ 1], tid);
        T::template mma<T::FN / 2, T::FN>(acc, f, dcol);
        __syncthreads();
    };
    int64_t i = 0;
    for (; i + NS <= nkt; i += NS) unrolled_steps<0, NS>(step, i);
    tail_steps<0, NS>(step, i, nkt);

    // Accumulator v of block (fi, fj): row 16 fi + 4 (lane / 16) + v of the
    // wave tile, column lane % 16.
    const int li = lane & 15, g = lane >> 4;
    const int64_t rwave = m0 + wm * T::WTM;
    float scale[T::FM][4];
#pragma unroll
    for (int fi = 0; fi < T::FM; ++fi)
#pragma unroll
        for (int v = 0; v < 4; ++v) scale[fi][v] = rs[min<int64_t>(rwave + 16 * fi + 4 * g + v, M - 1)];
    float *out = c + static_cast<int64_t>(split) * M * N;
    if (splits == 1 && glu) {
#pragma unroll
        for (int fi = 0; fi < T::FM; ++fi)
#pragma unroll
            for (int fj = 0; fj < T::FN / 2; ++fj) {
                const int64_t col = n0 + wn * (T::WTN / 2) + 16 * fj + li;
                if (col >= NO) continue;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t row = rwave + 16 * fi + 4 * g + v;
                    if (row < M)
                        c[row * NO + col] =
                            silu(acc[fi][fj][v] * scale[fi][v]) * (acc[fi][fj + T::FN / 2][v] * scale[fi][v]);
                }
            }
        return;
    }
    const bool resid = splits == 1 && epi == kEpiResidual;
#pragma unroll
    for (int fi = 0; fi < T::FM; ++fi)
#pragma unroll
        for (int fj = 0; fj < T::FN; ++fj) {
            int64_t col = n0 + wn * T::WTN + 16 * fj + li;
            bool ok = col < N;
            if (glu) {
                const int within = 16 * fj + li;
                const int64_t oc = n0 + wn * (T::WTN / 2) + within % (T::WTN / 2);
                ok = oc < NO;
                col = within < T::WTN / 2 ? oc : NO + oc;
            }
            if (!ok) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = rwave + 16 * fi + 4 * g + v;
                if (row < M) {
                    float *dst = out + row * N + col;
                    const float val = acc[fi][fj][v] * scale[fi][v];
                    *dst = resid ? *dst + val : val;
                }
            }
        }
}

// ------------------------------------------------------------------- plan --
struct HlTile {
    int bm, bn;
};
// Tiles compiled in (all reachable through the plan override); the planner
// chooses between 64x128 and 64x64 (the 128-row tiles measured slower on
// every shape below M = 1024).
constexpr HlTile kHlTiles[] = {{128, 128}, {128, 64}, {64, 128}, {64, 64}};

struct HlPlan {
    HlTile t;
    int splits, kts;
};

std::atomic<uint64_t> g_hl_override{0};  // bm | bn << 16 | splits << 32; 0 = none

// Cost model, in units of one 32-column step of a 64x128 f16 tile.  The
// busiest CU runs per_cu workgroups, co = min(per_cu, occ) of them at once
// (occ: workgroups that fit on a CU by registers and LDS); one or two
// resident workgroups hide less latency (factors f1, f2).  Each round of
// co-resident workgroups adds a fixed cost; a K split adds the partial-sum
// pass (a fixed part and one proportional to splits x M x N).  Step costs,
// factors and pass costs were fitted to measured run times of every (tile,
// split) choice on MI355X (f16 M = 17 .. 1024 at N, K in {2048, 4096, 6144};
// Q8_0 M = 17 .. 512 and Q4_0 M = 64, 512 at (11008, 4096) and (4096, 11008));
// the chosen plan is within 5 % of the best measured one on all of them.
struct HlCost {
    int bm, bn, occ;
    double step;
};
constexpr HlCost kHlF16[] = {{64, 128, 4, 1.0}, {64, 64, 5, 0.813}};
constexpr HlCost kHlQ8[] = {{64, 128, 2, 5.82}, {64, 64, 3, 3.88}};
constexpr HlCost kHlQ4[] = {{64, 128, 2, 4.92}, {64, 64, 3, 3.15}};
constexpr double kHlF1 = 0.30, kHlF2 = 0.783, kHlRound = 11.3, kHlSplit0 = 7.43, kHlSplit = 8.0e-6;

HlPlan hl_choose(int64_t m, int64_t n, int64_t k, int fmt, int cus, bool glu) {
    (void)glu;  // every tile pairs gate and up columns (an even number of 16-column blocks per wave)
    const int64_t ktiles = k / kBK;
    HlPlan best{HlTile{64, 128}, 1, static_cast<int>(ktiles)};
    double best_t = 1e300;
    auto consider = [&](const HlCost &c) {
        const int64_t tiles = ((m + c.bm - 1) / c.bm) * ((n + c.bn - 1) / c.bn);
        for (int sp : {1, 2, 4, 8, 16}) {
            const int64_t kts = (ktiles + sp - 1) / sp;
            const int64_t splits = (ktiles + kts - 1) / kts;
            if (splits != sp) continue;  // no empty split
            const int64_t wgs = tiles * splits;
            if (wgs > 0x7fffffffLL) continue;
            const int64_t per_cu = (wgs + cus - 1) / cus;
            const int64_t co = std::min<int64_t>(per_cu, c.occ);
            const double f = co == 1 ? kHlF1 : co == 2 ? kHlF2 : 1.0;
            double est = static_cast<double>(per_cu) * kts * c.step / f + kHlRound * ((per_cu + co - 1) / co);
            if (splits > 1) est += kHlSplit0 + kHlSplit * static_cast<double>(splits) * m * n;
            if (est < best_t) {
                best_t = est;
                best = HlPlan{HlTile{c.bm, c.bn}, static_cast<int>(splits), static_cast<int>(kts)};
            }
        }
    };
    for (const HlCost &c : fmt == HL_F16 ? kHlF16 : fmt == HL_Q8_0 ? kHlQ8 : kHlQ4) consider(c);
    return best;
}

HlPlan hl_planned(int64_t m, int64_t n, int64_t k, int fmt, int cus, bool glu) {
    const uint64_t o = g_hl_override.load(std::memory_order_relaxed);
    if (o == 0) return hl_choose(m, n, k, fmt, cus, glu);
    const int bm = static_cast<int>(o & 0xffff), bn = static_cast<int>((o >> 16) & 0xffff);
    if (glu && ((bn / 2 / 16) % 2 != 0)) return hl_choose(m, n, k, fmt, cus, glu);
    const int64_t ktiles = k / kBK;
    const int64_t want = std::max<int64_t>(1, std::min<int64_t>(static_cast<int64_t>(o >> 32), ktiles));
    const int64_t kts = (ktiles + want - 1) / want;
    return HlPlan{HlTile{bm, bn}, static_cast<int>((ktiles + kts - 1) / kts), static_cast<int>(kts)};
}

template <int BM, int BN, int FMT>
hipError_t hl_run(const uint16_t *ahl, const float *rs, const void *b, float *out, int64_t m, int64_t nw, int64_t k,
                  int64_t no, int splits, int kts, int epi, hipStream_t s) {
    const bool glu = epi == kEpiGlu;
    const int64_t mt = (m + BM - 1) / BM, nt = glu ? (no + BN / 2 - 1) / (BN / 2) : (nw + BN - 1) / BN;
    const int64_t tiles = mt * nt;
    if (tiles * splits > 0x7fffffffLL) return hipErrorInvalidValue;
    if (trace_enabled())
        fprintf(stderr, "[wqmm] gemm_hl<BM=%d,BN=%d,fmt=%d> m=%lld n=%lld k=%lld splits=%d kts=%d epi=%d grid=%lld\n",
                BM, BN, FMT, (long long)m, (long long)nw, (long long)k, splits, kts, epi,
                (long long)(tiles * splits));
    hipLaunchKernelGGL((gemm_hl<BM, BN, FMT, kStages>), dim3(static_cast<unsigned>(tiles * splits)), dim3(256), 0, s, ahl, rs,
                       b, out, m, nw, k, static_cast<int>(mt), static_cast<int>(tiles), kts, splits, no, epi);
    return hipGetLastError();
}

template <int FMT>
hipError_t hl_dispatch(const HlPlan &p, const uint16_t *ahl, const float *rs, const void *b, float *out, int64_t m,
                       int64_t nw, int64_t k, int64_t no, int epi, hipStream_t s) {
    const int sp = p.splits, kts = p.kts;
    if (p.t.bm == 128 && p.t.bn == 128) return hl_run<128, 128, FMT>(ahl, rs, b, out, m, nw, k, no, sp, kts, epi, s);
    if (p.t.bm == 128 && p.t.bn == 64) return hl_run<128, 64, FMT>(ahl, rs, b, out, m, nw, k, no, sp, kts, epi, s);
    if (p.t.bm == 64 && p.t.bn == 128) return hl_run<64, 128, FMT>(ahl, rs, b, out, m, nw, k, no, sp, kts, epi, s);
    return hl_run<64, 64, FMT>(ahl, rs, b, out, m, nw, k, no, sp, kts, epi, s);
}

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

bool hgemm_ok(const float *a, const void *b, int fmt, int64_t m, int64_t nw, int64_t k) {
    if (m < 1 || nw < 1 || k <= 0 || k % kBK != 0 || m > 0x7fffffffLL) return false;
    if ((reinterpret_cast<uintptr_t>(a) & 15u) != 0 || (reinterpret_cast<uintptr_t>(b) & 15u) != 0) return false;
    // Quantized weights are read through a buffer resource with 32-bit offsets.
    if (fmt != HL_F16 && static_cast<double>(nw) * (k / 32) * (fmt == HL_Q4_0 ? 18 : 34) >= 2147483648.0) return false;
    return true;
}

hipError_t launch_hgemm(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                        hipStream_t s, int epi) {
    if (m <= 0 || n <= 0) return hipSuccess;
    const int64_t nw = epi == kEpiGlu ? 2 * n : n;
    if (!hgemm_ok(a, b, fmt, m, nw, k)) return hipErrorInvalidValue;
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    const HlPlan p = hl_planned(m, nw, k, fmt, di.cus, epi == kEpiGlu);
    const size_t ahl_bytes = round256(static_cast<size_t>(m) * static_cast<size_t>(k) * 4);
    const size_t rs_bytes = round256(static_cast<size_t>(m) * 4);
    const size_t part_bytes =
        p.splits > 1 ? static_cast<size_t>(p.splits) * static_cast<size_t>(m) * static_cast<size_t>(nw) * 4 : 0;
    ScratchLease lease;
    void *scratch = nullptr;
    e = lease.acquire(ahl_bytes + rs_bytes + part_bytes, s, &scratch);
    if (e != hipSuccess) return e;
    uint16_t *ahl = static_cast<uint16_t *>(scratch);
    float *rs = reinterpret_cast<float *>(static_cast<char *>(scratch) + ahl_bytes);
    float *part = p.splits > 1 ? reinterpret_cast<float *>(static_cast<char *>(scratch) + ahl_bytes + rs_bytes) : c;
    hipLaunchKernelGGL(hl_split, dim3(static_cast<unsigned>(m)), dim3(256), 0, s, a, ahl, rs, k);
    e = hipGetLastError();
    if (e == hipSuccess) {
        e = fmt == HL_F16    ? hl_dispatch<HL_F16>(p, ahl, rs, b, part, m, nw, k, n, epi, s)
            : fmt == HL_Q8_0 ? hl_dispatch<HL_Q8_0>(p, ahl, rs, b, part, m, nw, k, n, epi, s)
                             : hl_dispatch<HL_Q4_0>(p, ahl, rs, b, part, m, nw, k, n, epi, s);
    }
    if (e == hipSuccess && p.splits > 1) e = launch_reduce_splits(part, c, m, n, nw, p.splits, epi, s);
    const hipError_t er = lease.release();
    return e != hipSuccess ? e : er;
}

void hgemm_plan(int64_t m, int64_t n, int64_t k, int fmt, int cus, int *bm, int *bn, int *splits) {
    const HlPlan p = hl_planned(m, n, k, fmt, cus, false);
    *bm = p.t.bm;
    *bn = p.t.bn;
    *splits = p.splits;
}

bool set_hgemm_plan_override(int bm, int bn, int splits) {
    if (bm == 0 && bn == 0 && splits == 0) {
        g_hl_override.store(0, std::memory_order_relaxed);
        return true;
    }
    bool known = false;
    for (const HlTile &t : kHlTiles) known = known || (t.bm == bm && t.bn == bn);
    if (!known || splits < 1 || splits > 64) return false;
    g_hl_override.store(static_cast<uint64_t>(bm) | (static_cast<uint64_t>(bn) << 16) |
                            (static_cast<uint64_t>(splits) << 32),
                        std::memory_order_relaxed);
    return true;
}

}  // namespace wq
