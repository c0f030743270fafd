// Weight-streaming product for Q8_0 / Q4_0 weights and 1 <= M <= 16 rows of A
// on the f16 matrix cores: C[M,N] = A[M,K] . B[N,K]^T, every weight read from
// HBM once.
//
// Operation: the M == 1 decode GEMV and the small-M branch of dispatch_gemm_q8
// / dispatch_gemm_q4 (lattice-inference 0.9.0, dispatch.rs; kernels
// gemv_q8_decode, gemv_q4_decode and gemm_q8, lattice-inference 0.1.2,
// metal_qwen35.rs): within a block the codes are summed against the
// activations and the block scale is applied once, c = sum_j d_j sum_i q_i a_i.
//
// Why f16 matrix cores with f32 results: a code is a small integer (-128..127
// for Q8_0, -8..7 for Q4_0), exact in f16.  An f32 activation x is carried as
// two f16 numbers, hi = f16(x s) and lo = f16(x s - hi) with s a power of two
// chosen per row of A and K range (so that |x s| < 2^15): hi + lo equals x s
// to 22 significant bits.  The matrix core multiplies f16 pairs exactly and
// accumulates in f32, so one K = 32 step over a quantized block computes
// sum_i q_i (hi_i + lo_i) in two instructions (v_mfma_f32_16x16x32_f16), the
// lane applies d (and 1/s) in f32.  The f16 rate is sixteen times the f32
// matrix rate, so the matrix work of 16 rows of A costs little next to the
// weight stream, and M = 1 .. 16 run in nearly the same time.
//
// CDNA4 layout:
//  * A 16x16x32 step takes, per lane l, 8 k slots of weight row l % 16 (the B
//    operand) and the same 8 k slots of activation row l % 16 (the A
//    operand); lane group g = l / 16 holds slots 8g .. 8g + 7.  Which k of the
//    block a slot holds is free as long as both operands agree, so the slots
//    follow the bytes: two consecutive blocks (68 bytes for Q8_0, 36 for
//    Q4_0; they start at a dword boundary because K % 256 == 0) are read by
//    each lane as whole dwords -- codes of the odd block are dword-aligned, the
//    even block's first two and last two codes share dwords with the scales
//    and are regrouped by one v_perm_b32 in lane group 3.
//  * Weights reach those dwords one of two ways.  Staged (the variants the
//    planner uses): a wave copies each 256-column superblock of its 16-row
//    tiles with contiguous 128-bit loads (17 or 9 per row, 5 or 3 per lane),
//    writes the chunks to its own LDS region and reads its operand dwords
//    back (in order within the wave, no barrier).  Direct: each lane loads its
//    operand dwords from global memory (12 or 20 bytes per lane and 16 rows in
//    2 or 3 loads); measured slower, because the texture path is bound by the
//    number of load instructions, not bytes.
//  * Codes become f16 by placing the byte (Q8_0: xor 0x80) or nibble in the
//    mantissa of 1024 and subtracting 1152 (1032) with one packed f16 op.
//  * Lane group 3 also holds both scales of the pair; one ds_bpermute hands
//    them to the other three lane groups of the same weight row.
//  * A workgroup owns TW groups of P tiles of 16 weight rows and a K range of
//    whole 256-column superblocks, split among KWV waves per tile group.  The
//    activations of the range are read first, the first two superblocks of
//    weights are issued next, then the activations are split into hi / lo
//    into LDS in operand order.  A wave streams its superblocks with the next
//    one's loads in flight while the current one is decoded; the KWV partial
//    tiles meet in LDS in wave order.
//  * When K is split across workgroups, each writes its partial tile to
//    scratch and one more launch sums the partials in split order.
//    Deterministic.
// Requires K % 256 == 0, 16-byte aligned a and b, N * K / 32 * 34 < 2^31,
// and M * K <= 196608 (at most 16 splits of at most 48 / M superblocks).
#include "wq_internal.h"

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>

namespace wq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { WS_Q8_0 = 1, WS_Q4_0 = 2 };

template <int FMT>
struct WsFmt {
    static constexpr int kBytes = FMT == WS_Q8_0 ? 34 : 18;  // block
    static constexpr int kPair = 2 * kBytes;                 // two blocks, dword-aligned
    static constexpr int kSb = 8 * kBytes;                   // superblock: 8 blocks, 256 columns
};

constexpr uint32_t kWsOut = 0x80000000u;  // out-of-range buffer offset: the load returns zeros
constexpr int kWsMaxSplits = 16;          // K splits across workgroups (partials summed by ws_reduce)

// Block column (0..31) that k slot t (0..7) of lane group g holds, for the even
// (first) or odd (second) block of a pair.
template <int FMT>
__device__ __forceinline__ int ws_kpos(int odd, int g, int t) {
    if constexpr (FMT == WS_Q8_0) {
        if (odd) return 8 * g + t;
        if (g < 3) return 2 + 8 * g + t;
        return t < 4 ? 26 + t : t < 6 ? t - 4 : 24 + t;  // codes 26..29, then 0, 1, 30, 31
    } else {
        // A code dword b0..b3 gives the pairs (lo b0, lo b2), (hi b0, hi b2),
        // (lo b1, lo b3), (hi b1, hi b3); byte i holds columns 2i (lo), 2i + 1.
        const int o = (t >> 1) + 4 * (t & 1);
        if (odd) return 8 * g + o;
        if (g < 3) return 4 + 8 * g + o;
        return (t >> 1) + 28 * (t & 1);  // bytes 0, 1, 14, 15
    }
}

// Byte offsets, inside a pair of blocks, of lane group g's loads: main (Q8_0
// two dwords, Q4_0 one), extra (lane group 3 only) and odd (the second block).
template <int FMT>
struct WsLaneOff {
    uint32_t main, extra, odd;
    __device__ __forceinline__ explicit WsLaneOff(int g) {
        if constexpr (FMT == WS_Q8_0) {
            main = g < 3 ? 4u + 8u * g : 28u;  // dwords 1+2g, 2+2g (group 3: dwords 7, 8)
            extra = g < 3 ? kWsOut : 0u;       // dword 0: the scale and codes 0, 1
            odd = 36u + 8u * g;
        } else {
            main = g < 3 ? 4u + 4u * g : 0u;  // dword 1+g (group 3: dword 0)
            extra = g < 3 ? kWsOut : 16u;      // dword 4: codes 14, 15 and the next scale
            odd = 20u + 4u * g;
        }
    }
};

// One pair of blocks of one weight row tile as loaded by a lane.
template <int FMT>
struct WsPair;
template <>
struct WsPair<WS_Q8_0> {
    u32x2 m, o;
    uint32_t e;
};
template <>
struct WsPair<WS_Q4_0> {
    uint32_t m, o, e;
};

template <int FMT, int AUX>
__device__ __forceinline__ void ws_load(WsPair<FMT> &p, __amdgpu_buffer_rsrc_t rb, uint32_t voff,
                                        const WsLaneOff<FMT> &lo, uint32_t soff) {
    const uint32_t ex = lo.extra == kWsOut ? kWsOut : voff + lo.extra;
    if constexpr (FMT == WS_Q8_0) {
        p.m = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rb, static_cast<int>(voff + lo.main),
                                                                          static_cast<int>(soff), AUX));
        p.e = __builtin_amdgcn_raw_buffer_load_b32(rb, static_cast<int>(ex), static_cast<int>(soff), AUX);
        p.o = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rb, static_cast<int>(voff + lo.odd),
                                                                          static_cast<int>(soff), AUX));
    } else {
        p.m = __builtin_amdgcn_raw_buffer_load_b32(rb, static_cast<int>(voff + lo.main), static_cast<int>(soff),
                                                   AUX);
        p.e = __builtin_amdgcn_raw_buffer_load_b32(rb, static_cast<int>(ex), static_cast<int>(soff), AUX);
        p.o = __builtin_amdgcn_raw_buffer_load_b32(rb, static_cast<int>(voff + lo.odd), static_cast<int>(soff),
                                                   AUX);
    }
}

__device__ __forceinline__ uint32_t f16x2_sub(uint32_t x, _Float16 v) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(hh2, x) - hh2{v, v});
}

// Four Q8_0 codes (int8 bytes of x) as two f16 pairs: byte u = q + 128 in the
// mantissa of 1024, minus 1152.
__device__ __forceinline__ void ws_q8_codes(uint32_t x, uint32_t &p0, uint32_t &p1) {
    const uint32_t u = x ^ 0x80808080u;
    p0 = f16x2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u), static_cast<_Float16>(1152.0f));
    p1 = f16x2_sub(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u), static_cast<_Float16>(1152.0f));
}

// Eight Q4_0 weights (nibbles of x) as four f16 pairs u - 8.
__device__ __forceinline__ h8 ws_q4_codes(uint32_t x) {
    const _Float16 bias = static_cast<_Float16>(1032.0f);
    const uint32_t v0 = f16x2_sub((x & 0x000F000Fu) | 0x64006400u, bias);
    const uint32_t v1 = f16x2_sub(((x >> 4) & 0x000F000Fu) | 0x64006400u, bias);
    const uint32_t v2 = f16x2_sub(((x >> 8) & 0x000F000Fu) | 0x64006400u, bias);
    const uint32_t v3 = f16x2_sub(((x >> 12) & 0x000F000Fu) | 0x64006400u, bias);
    return __builtin_bit_cast(h8, u32x4{v0, v1, v2, v3});
}

// The B operands of the even and odd block and the scale pair (lane group 3's
// view: scale of the even block in the low half, of the odd block in the high
// half; other lane groups get garbage and take lane group 3's).
template <int FMT>
__device__ __forceinline__ void ws_decode(const WsPair<FMT> &p, int g, h8 &be, h8 &bo, uint32_t &sc) {
    if constexpr (FMT == WS_Q8_0) {
        const uint32_t c1 = g == 3 ? __builtin_amdgcn_perm(p.m.y, p.e, 0x05040302u) : p.m.y;
        uint32_t e0, e1, e2, e3, o0, o1, o2, o3;
        ws_q8_codes(p.m.x, e0, e1);
        ws_q8_codes(c1, e2, e3);
        ws_q8_codes(p.o.x, o0, o1);
        ws_q8_codes(p.o.y, o2, o3);
        be = __builtin_bit_cast(h8, u32x4{e0, e1, e2, e3});
        bo = __builtin_bit_cast(h8, u32x4{o0, o1, o2, o3});
        sc = __builtin_amdgcn_perm(p.m.y, p.e, 0x07060100u);  // dword 0 low half, dword 8 high half
    } else {
        const uint32_t c = g == 3 ? __builtin_amdgcn_perm(p.e, p.m, 0x05040302u) : p.m;
        be = ws_q4_codes(c);
        bo = ws_q4_codes(p.o);
        sc = __builtin_amdgcn_perm(p.e, p.m, 0x07060100u);  // dword 0 low half, dword 4 high half
    }
}

// LDS layout of the activation operands: for local block jb and lane group g,
// the hi halves of rows 0..M-1 (16 bytes each), then the lo halves.
__device__ __forceinline__ uint32_t ws_frag_off(int jb, int g, int m, int M) {
    return static_cast<uint32_t>(((jb * 4 + g) * 2 * M + m) * 16);
}

constexpr int kWsIpt = 6;  // activation items (8 values) per thread in the single staging pass

// The power-of-two scale s of a row of activations with largest magnitude amax
// (amax * s in [2^14, 2^15), 1 for amax == 0), or 1 / s.
__device__ __forceinline__ float ws_scale(float amax, bool inverse) {
    int e = 0;
    if (amax > 0.f) {
        (void)frexpf(amax, &e);
        e -= 15;
    }
    e = e < -100 ? -100 : e > 100 ? 100 : e;
    return ldexpf(1.0f, inverse ? e : -e);
}

// Chunks of 16 bytes in one superblock of a 16-row tile, and per lane.
template <int FMT>
struct WsTile {
    static constexpr int kRowChunks = WsFmt<FMT>::kSb / 16;          // 17 (Q8_0) or 9 (Q4_0)
    static constexpr int kChunks = 16 * kRowChunks;                   // 272 or 144
    static constexpr int kLaneChunks = (kChunks + kWave - 1) / kWave;  // 5 or 3
    static constexpr int kBytes = 16 * kChunks;                       // 4352 or 2304
};

template <int FMT, int P, int KWV, int TW, bool STG>
__global__ __launch_bounds__(KWV *TW *kWave) void gemm_wstream(const float *__restrict__ a,
                                                              const uint8_t *__restrict__ b, float *__restrict__ c,
                                                              float *__restrict__ part, int M, int64_t n, int64_t k,
                                                              int nsb, int splits, int resid, int a_lds) {
    using F = WsFmt<FMT>;
    using T = WsTile<FMT>;
    constexpr int NW = KWV * TW;       // waves: TW row-tile groups x KWV K sub-ranges
    constexpr int R = TW * P * 16;     // weight rows per workgroup
    extern __shared__ __attribute__((aligned(16))) uint8_t ws_lds[];
    __shared__ uint32_t s_amax[16];

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform (scalar) from here on
    const int n16 = lane & 15, g = lane >> 4;
    const int tw = w / KWV, kw = w - tw * KWV;
    const int z = blockIdx.y;
    const int sb0 = static_cast<int>((static_cast<int64_t>(z) * nsb) / splits);
    const int sb1 = static_cast<int>((static_cast<int64_t>(z + 1) * nsb) / splits);
    const int ms0 = sb0 + ((sb1 - sb0) * kw) / KWV;        // this wave's superblocks
    const int ms1 = sb0 + ((sb1 - sb0) * (kw + 1)) / KWV;
    const int nbl = 8 * (sb1 - sb0);
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * R;
    const uint32_t row_bytes = static_cast<uint32_t>(k >> 5) * F::kBytes;
    if (tid < 16) s_amax[tid] = 0u;
    __syncthreads();

    // ---- 1. activations of the workgroup's K range into registers (first) ----
    const int items = nbl * 4 * M;  // (local block, lane group, row) triples, 8 values each
    float av[kWsIpt][8];
#pragma unroll
    for (int i = 0; i < kWsIpt; ++i) {
        const int it = tid + i * NW * kWave;
        if (it < items) {
            const int jb = it / (4 * M), rem = it - jb * 4 * M, gg = rem / M, m = rem - gg * M;
            const float *src = a + static_cast<int64_t>(m) * k + 32 * (8 * sb0 + jb);
#pragma unroll
            for (int t = 0; t < 8; ++t) av[i][t] = src[ws_kpos<FMT>(jb & 1, gg, t)];
        }
    }

    // ---- 2. the first two superblocks of weights (loads past the wave's range
    // go to an empty resource: zeros, no memory traffic) ----
    const int64_t rows_left = n - row0;
    const uint32_t nrec = static_cast<uint32_t>(rows_left < R ? rows_left : R) * row_bytes;  // integer min
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(b) + row0 * static_cast<int64_t>(row_bytes), 0, static_cast<int>(nrec), 0x00020000);
    const __amdgpu_buffer_rsrc_t rnull = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(b), 0, 0, 0x00020000);
    const WsLaneOff<FMT> lo(g);
    uint32_t voff[P];
#pragma unroll
    for (int p = 0; p < P; ++p) voff[p] = static_cast<uint32_t>(16 * (tw * P + p) + n16) * row_bytes;

    // Register stage of one superblock: STG, whole 16-byte chunks of the
    // tiles (copied to the wave's LDS region before decoding); otherwise the
    // lanes' operand dwords directly.
    struct Stage {
        WsPair<FMT> pr[STG ? 1 : P][4];
        u32x4 ch[STG ? P : 1][STG ? T::kLaneChunks : 1];
    };
    uint32_t coff[STG ? P : 1][STG ? T::kLaneChunks : 1];  // byte offset of each chunk of this lane
    if constexpr (STG) {
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int u = 0; u < T::kLaneChunks; ++u) {
                const int cc = lane + kWave * u;
                const int r = cc / T::kRowChunks, q = cc - r * T::kRowChunks;
                coff[p][u] = cc < T::kChunks ? static_cast<uint32_t>(16 * (tw * P + p) + r) * row_bytes + 16u * q
                                             : kWsOut;
            }
    }
    Stage cur, nxt;
    auto load_sb = [&](Stage &dst, int s) {
        // s is wave-uniform; readfirstlane keeps the offset in a scalar register
        // (without it the compiler may move the chain to vector registers and
        // wrap every load in a loop over distinct offsets).
        const int su = __builtin_amdgcn_readfirstlane(s);
        const bool live = su < ms1;
        const __amdgpu_buffer_rsrc_t r = live ? rb : rnull;
        const uint32_t sbase = static_cast<uint32_t>(live ? su : 0) * F::kSb;
        if constexpr (STG) {
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int u = 0; u < T::kLaneChunks; ++u)
                    dst.ch[p][u] = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(coff[p][u]),
                                                                         static_cast<int>(sbase), 0);
        } else {
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int pp = 0; pp < 4; ++pp)
                    ws_load<FMT, 0>(dst.pr[p][pp], r, voff[p], lo, sbase + pp * F::kPair);
        }
    };
    load_sb(cur, ms0);
    load_sb(nxt, ms0 + 1);

    // ---- 3. per-row scale (max over the K range), hi / lo into LDS ----
#pragma unroll
    for (int i = 0; i < kWsIpt; ++i) {
        const int it = tid + i * NW * kWave;
        if (it < items) {
            const int m = (it - (it / (4 * M)) * 4 * M) % M;
            float mx = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) mx = fmaxf(mx, fabsf(av[i][t]));
            atomicMax(&s_amax[m], __builtin_bit_cast(uint32_t, mx));
        }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWsIpt; ++i) {
        const int it = tid + i * NW * kWave;
        if (it < items) {
            const int jb = it / (4 * M), rem = it - jb * 4 * M, gg = rem / M, m = rem - gg * M;
            // s = 2^-e with amax * s in [2^14, 2^15): hi and lo stay normal f16 numbers.
            const float sc = ws_scale(__builtin_bit_cast(float, s_amax[m]), false);
            h8 hi, lo8;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float x = av[i][t] * sc;
                const _Float16 h = static_cast<_Float16>(x);
                hi[t] = h;
                lo8[t] = static_cast<_Float16>(x - static_cast<float>(h));
            }
            *reinterpret_cast<h8 *>(ws_lds + ws_frag_off(jb, gg, m, M)) = hi;
            *reinterpret_cast<h8 *>(ws_lds + ws_frag_off(jb, gg, m, M) + 16 * M) = lo8;
        }
    }
    __syncthreads();

    // ---- 4. weight stream ----
    const int m_mine = n16;  // activation row of this lane's A operand
    const bool a_live = m_mine < M;
    f4 acc[P];
#pragma unroll
    for (int p = 0; p < P; ++p) acc[p] = f4{0.f, 0.f, 0.f, 0.f};
    // Activation operands: lanes of rows m >= M keep zeros (set once here).
    h8 ahe = {}, ale = {}, aho = {}, alo = {};
    uint8_t *const stage_lds = ws_lds + a_lds + static_cast<size_t>(w) * P * T::kBytes;  // STG: this wave's tiles
    auto compute_sb = [&](const Stage &src, int s) {
        const int jb0 = 8 * (s - sb0);
        if constexpr (STG) {
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int u = 0; u < T::kLaneChunks; ++u)
                    if (lane + kWave * u < T::kChunks)
                        *reinterpret_cast<u32x4 *>(stage_lds + p * T::kBytes + 16 * (lane + kWave * u)) = src.ch[p][u];
        }
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            if (a_live) {
                const uint8_t *fe = ws_lds + ws_frag_off(jb0 + 2 * pp, g, m_mine, M);
                const uint8_t *fo = ws_lds + ws_frag_off(jb0 + 2 * pp + 1, g, m_mine, M);
                ahe = *reinterpret_cast<const h8 *>(fe);
                ale = *reinterpret_cast<const h8 *>(fe + 16 * M);
                aho = *reinterpret_cast<const h8 *>(fo);
                alo = *reinterpret_cast<const h8 *>(fo + 16 * M);
            }
#pragma unroll
            for (int p = 0; p < P; ++p) {
                WsPair<FMT> pr;
                if constexpr (STG) {
                    // The lane's operand dwords from the staged rows (LDS reads
                    // of one wave follow its writes in order).
                    const uint8_t *rowp = stage_lds + p * T::kBytes + n16 * F::kSb + pp * F::kPair;
                    const uint32_t *mp = reinterpret_cast<const uint32_t *>(rowp + lo.main);
                    const uint32_t *op = reinterpret_cast<const uint32_t *>(rowp + lo.odd);
                    const uint32_t *ep = reinterpret_cast<const uint32_t *>(rowp + (lo.extra == kWsOut ? 0u : lo.extra));
                    if constexpr (FMT == WS_Q8_0) {
                        pr.m = u32x2{mp[0], mp[1]};
                        pr.o = u32x2{op[0], op[1]};
                    } else {
                        pr.m = mp[0];
                        pr.o = op[0];
                    }
                    pr.e = ep[0];
                } else {
                    pr = src.pr[p][pp];
                }
                h8 be, bo;
                uint32_t scp;
                ws_decode<FMT>(pr, g, be, bo, scp);
                scp = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute((48 + n16) * 4, static_cast<int>(scp)));
                const float de = half_bits_to_float(scp & 0xffffu);
                const float dd = half_bits_to_float(scp >> 16);
                f4 te = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahe, be, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                f4 to = __builtin_amdgcn_mfma_f32_16x16x32_f16(aho, bo, f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                te = __builtin_amdgcn_mfma_f32_16x16x32_f16(ale, be, te, 0, 0, 0);
                to = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bo, to, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[p][r] = fmaf(dd, to[r], fmaf(de, te[r], acc[p][r]));
            }
        }
    };
    // Invariant at the loop head: cur (superblock s) and nxt (s + 1) are
    // issued, cur first; loads past the range read the empty resource.
    for (int s = ms0; s < ms1; s += 2) {
        compute_sb(cur, s);
        if (s + 1 >= ms1) break;
        load_sb(cur, s + 2);
        compute_sb(nxt, s + 1);
        load_sb(nxt, s + 3);
    }

    // ---- 5. epilogue: lane holds rows m = 4g + r of weight row n16 of each tile ----
    float us[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        us[r] = 4 * g + r < M ? ws_scale(__builtin_bit_cast(float, s_amax[4 * g + r]), true) : 0.f;
    if constexpr (KWV > 1) {
        // The K sub-ranges of a tile group meet in LDS (the activation operands
        // are no longer read), summed in wave order.
        __syncthreads();
        f4 *red = reinterpret_cast<f4 *>(ws_lds);
#pragma unroll
        for (int p = 0; p < P; ++p) red[(w * P + p) * kWave + lane] = acc[p];
        __syncthreads();
        if (kw != 0) return;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            f4 t = red[((tw * KWV) * P + p) * kWave + lane];
            for (int q = 1; q < KWV; ++q) t += red[((tw * KWV + q) * P + p) * kWave + lane];
            acc[p] = t;
        }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int64_t nn = row0 + 16 * (tw * P + p) + n16;
        if (nn >= n) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m >= M) continue;
            const float v = acc[p][r] * us[r];
            if (splits > 1) {
                part[(static_cast<int64_t>(z) * M + m) * n + nn] = v;
            } else {
                float *dst = c + static_cast<int64_t>(m) * n + nn;
                *dst = resid ? *dst + v : v;
            }
        }
    }
}

// Variants: (P tiles per wave, KWV K sub-ranges per workgroup, TW tile groups,
// weights staged through LDS).
struct WsShape {
    int p, kwv, tw, stg;
};
constexpr WsShape kWsShapes[] = {{1, 4, 1, 0}, {1, 8, 1, 0}, {2, 4, 1, 0}, {1, 2, 2, 0}, {2, 1, 4, 0},
                                 {1, 1, 4, 0}, {2, 8, 1, 0}, {1, 4, 1, 1}, {1, 1, 4, 1}, {2, 1, 4, 1},
                                 {1, 8, 1, 1}, {1, 2, 2, 1}, {1, 1, 8, 1}, {2, 1, 8, 1}};
constexpr int kWsNumShapes = sizeof(kWsShapes) / sizeof(kWsShapes[0]);

// Forced plan (wq_set_stream_plan): shape index + 1, splits; 0 = automatic.
std::atomic<int> g_ws_shape{0}, g_ws_splits{0};

struct WsPlan {
    int shape, groups, splits;
};

// Superblocks per split: at most 48 / M (the activations of a split are
// staged in one pass of at most 6 items per thread, and fit in 48 KiB of LDS).
int ws_min_splits(int64_t m, int nsb) {
    const int64_t per = std::max<int64_t>(1, 48 / m);
    return static_cast<int>((nsb + per - 1) / per);
}

// Automatic plan, from a sweep of every shape and 1 .. 8 splits on MI355X (Q8_0
// and Q4_0 at (N, K) = (11008, 4096) and (4096, 11008), M = 1, 4, 8, 16): the
// LDS-staged shapes win everywhere; 8 waves of one tile each (128 rows) up to
// M = 8, 8 waves of two tiles (256 rows, half the activation staging per
// weight byte) for larger M when N is small enough to leave the row groups
// busy.  K is split in a power of two (at most 8) of parts so that the grid
// has about two workgroups per CU: fewer, longer workgroups (or a count just
// above the CU count) left the last round of the grid underused (e.g. 3 splits
// of 16 superblocks at (11008, 4096): 21-22 us against 18-19 us for 4 or 8).
// Workgroup shape and K splits by M and the weight size, the rule that came
// closest to the best of every (shape, split) choice measured on MI355X for
// Q8_0 and Q4_0 at M = 2, 4, 8, 16 over (N, K) = (6144, 2048), (2048, 6144),
// (2048, 2048), (11008, 4096), (4096, 11008), (151936, 2048): within 2 % on
// average and 16 % at worst (the previous fixed choice: 11 % and 46 %).
// Shapes (0-based): 8 = one 16-row tile per wave, 4 tile groups per
// workgroup; 10 = 8 K sub-ranges per workgroup; 12 / 13 = 8 tile groups of
// one or two tiles.  splits = 0: about two workgroups per CU.
struct WsRule {
    int shape, splits;
};
WsRule ws_rule(int64_t m, int64_t n, int64_t k) {
    const int64_t nk = n * k;
    if (nk > (64LL << 20)) return WsRule{m >= 16 ? 13 : 12, 0};
    if (nk > (16LL << 20)) {
        if (m <= 4) return WsRule{8, 0};
        if (m <= 8) return WsRule{12, 8};
        return WsRule{n <= 6144 ? 13 : 12, 8};
    }
    if (m <= 2) return k > 4096 ? WsRule{8, 0} : WsRule{10, 1};
    if (m <= 4) return WsRule{8, 8};
    return WsRule{8, 0};
}

WsPlan ws_plan(int64_t m, int64_t n, int64_t k, int cus) {
    const int nsb = static_cast<int>(k / 256);
    const int smin = ws_min_splits(m, nsb);
    const WsRule rule = ws_rule(m, n, k);
    int shape = rule.shape;
    if (const int fs = g_ws_shape.load(std::memory_order_relaxed); fs > 0) shape = fs - 1;
    const WsShape &sh = kWsShapes[shape];
    const int64_t rows = 16LL * sh.p * sh.tw;
    const int64_t groups = (n + rows - 1) / rows;
    int64_t splits = 1;
    while (splits < 8 && splits * groups < 2LL * cus) splits *= 2;
    if (rule.splits > 0) splits = rule.splits;
    if (const int fsp = g_ws_splits.load(std::memory_order_relaxed); fsp > 0) splits = fsp;
    splits = std::min<int64_t>(std::min<int64_t>(std::max<int64_t>(splits, smin), nsb), kWsMaxSplits);
    return WsPlan{shape, static_cast<int>(groups), static_cast<int>(splits)};
}

// Split partials [splits][m][n] summed in split order (all loads of a thread
// issued before the first add), then the residual epilogue.
__global__ __launch_bounds__(256) void ws_reduce(const float *__restrict__ part, float *__restrict__ c, int64_t mn,
                                                 int splits, int resid) {
    const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
    if (i >= mn) return;
    f4 v[kWsMaxSplits];
    const bool full = i + 4 <= mn;
#pragma unroll
    for (int z = 0; z < kWsMaxSplits; ++z) {
        if (z < splits) {
            const float *p = part + z * mn + i;
            v[z] = full ? *reinterpret_cast<const f4 *>(p)
                        : f4{p[0], i + 1 < mn ? p[1] : 0.f, i + 2 < mn ? p[2] : 0.f, i + 3 < mn ? p[3] : 0.f};
        }
    }
    f4 t = v[0];
#pragma unroll
    for (int z = 1; z < kWsMaxSplits; ++z)
        if (z < splits) t += v[z];
    for (int e = 0; e < 4; ++e)
        if (i + e < mn) c[i + e] = resid ? c[i + e] + t[e] : t[e];
}

template <int FMT, int P, int KWV, int TW, bool STG>
hipError_t run_ws(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k, const WsPlan &pl,
                  hipStream_t s, int resid) {
    constexpr int NW = KWV * TW;
    const int nsb = static_cast<int>(k / 256);
    const int sb_max = (nsb + pl.splits - 1) / pl.splits;
    const size_t a_lds = static_cast<size_t>(sb_max) * 8 * 4 * 2 * static_cast<size_t>(m) * 16;
    const size_t lds = std::max<size_t>(a_lds + (STG ? static_cast<size_t>(NW) * P * WsTile<FMT>::kBytes : 0),
                                        static_cast<size_t>(NW) * P * kWave * 16);
    ScratchLease lease;
    float *part = nullptr;
    if (pl.splits > 1) {
        void *scratch = nullptr;
        const hipError_t e = lease.acquire(static_cast<size_t>(pl.splits) * m * n * 4, s, &scratch);
        if (e != hipSuccess) return e;
        part = static_cast<float *>(scratch);
    }
    if (trace_enabled())
        fprintf(stderr,
                "[wqmm] gemm_wstream<fmt=%d,P=%d,KWV=%d,TW=%d,STG=%d> m=%lld n=%lld k=%lld groups=%d splits=%d "
                "lds=%zu\n",
                FMT, P, KWV, TW, STG ? 1 : 0, (long long)m, (long long)n, (long long)k, pl.groups, pl.splits, lds);
    hipLaunchKernelGGL((gemm_wstream<FMT, P, KWV, TW, STG>), dim3(pl.groups, pl.splits), dim3(NW * kWave), lds, s,
                       a, b, c, part, static_cast<int>(m), n, k, nsb, pl.splits, resid, static_cast<int>(a_lds));
    hipError_t e = hipGetLastError();
    if (pl.splits > 1) {
        if (e == hipSuccess) {
            const int64_t mn = m * n;
            hipLaunchKernelGGL(ws_reduce, dim3(static_cast<unsigned>((mn / 4 + 255) / 256 + 1)), dim3(256), 0, s, part,
                               c, mn, pl.splits, resid);
            e = hipGetLastError();
        }
        const hipError_t er = lease.release();
        if (e == hipSuccess) e = er;
    }
    return e;
}

template <int FMT>
hipError_t run_ws_fmt(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k, const WsPlan &pl,
                      hipStream_t s, int resid) {
    switch (pl.shape) {
        case 0: return run_ws<FMT, 1, 4, 1, false>(a, b, c, m, n, k, pl, s, resid);
        case 1: return run_ws<FMT, 1, 8, 1, false>(a, b, c, m, n, k, pl, s, resid);
        case 2: return run_ws<FMT, 2, 4, 1, false>(a, b, c, m, n, k, pl, s, resid);
        case 3: return run_ws<FMT, 1, 2, 2, false>(a, b, c, m, n, k, pl, s, resid);
        case 4: return run_ws<FMT, 2, 1, 4, false>(a, b, c, m, n, k, pl, s, resid);
        case 5: return run_ws<FMT, 1, 1, 4, false>(a, b, c, m, n, k, pl, s, resid);
        case 6: return run_ws<FMT, 2, 8, 1, false>(a, b, c, m, n, k, pl, s, resid);
        case 7: return run_ws<FMT, 1, 4, 1, true>(a, b, c, m, n, k, pl, s, resid);
        case 8: return run_ws<FMT, 1, 1, 4, true>(a, b, c, m, n, k, pl, s, resid);
        case 9: return run_ws<FMT, 2, 1, 4, true>(a, b, c, m, n, k, pl, s, resid);
        case 10: return run_ws<FMT, 1, 8, 1, true>(a, b, c, m, n, k, pl, s, resid);
        case 11: return run_ws<FMT, 1, 2, 2, true>(a, b, c, m, n, k, pl, s, resid);
        case 12: return run_ws<FMT, 1, 1, 8, true>(a, b, c, m, n, k, pl, s, resid);
        default: return run_ws<FMT, 2, 1, 8, true>(a, b, c, m, n, k, pl, s, resid);
    }
}

}  // namespace

bool wstream_ok(const float *a, const void *b, int fmt, int64_t m, int64_t n, int64_t k) {
    const int64_t bytes = n * (k / 32) * (fmt == WS_Q8_0 ? 34 : 18);
    return (fmt == WS_Q8_0 || fmt == WS_Q4_0) && m >= 1 && m <= 16 && k > 0 && k % 256 == 0 && n >= 1 &&
           bytes < (int64_t(1) << 31) && 4 * k * m < (int64_t(1) << 31) &&
           ws_min_splits(m, static_cast<int>(k / 256)) <= kWsMaxSplits &&
           (reinterpret_cast<uintptr_t>(a) & 15) == 0 && (reinterpret_cast<uintptr_t>(b) & 15) == 0;
}

hipError_t launch_wstream(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                          hipStream_t s, int epi) {
    if (!wstream_ok(a, b, fmt, m, n, k) || (epi != kEpiNone && epi != kEpiResidual)) return hipErrorInvalidValue;
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    const WsPlan pl = ws_plan(m, n, k, di.cus);
    const uint8_t *b8 = static_cast<const uint8_t *>(b);
    const int resid = epi == kEpiResidual;
    if (fmt == WS_Q8_0) return run_ws_fmt<WS_Q8_0>(a, b8, c, m, n, k, pl, s, resid);
    return run_ws_fmt<WS_Q4_0>(a, b8, c, m, n, k, pl, s, resid);
}

bool set_wstream_plan_override(int shape, int splits) {
    if (shape < 0 || shape > kWsNumShapes || splits < 0) return false;
    g_ws_shape.store(shape, std::memory_order_relaxed);
    g_ws_splits.store(splits, std::memory_order_relaxed);
    return true;
}

}  // namespace wq
