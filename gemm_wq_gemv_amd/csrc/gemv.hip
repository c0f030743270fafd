// Decode GEMV (M = 1): c[n] = sum_k a[k] * w[n, k] for f16, Q8_0 and Q4_0 weights,
// with the epilogues: c[n] += that sum (residual), or c[j] = silu(g_j) * u_j
// for a fused gate||up weight of 2n rows (SwiGLU; gate row j and up row n + j).
//
// The operation is the M = 1 case of dispatch_matmul_half / dispatch_matmul_q8 /
// dispatch_matmul_q4 (lattice-inference 0.9.0, dispatch.rs) and of the kernels
// gemv_decode_m1, gemv_q8_decode and gemv_q4_decode (lattice-inference 0.1.2,
// metal_qwen35.rs).  Those kernels
// were written for 32-lane Apple SIMD groups (one threadgroup per output row
// for f16, two rows per threadgroup for Q8_0).  On CDNA4 the work is bound by
// HBM bandwidth, so the design here is about the byte stream:
//
//  * f16: a workgroup of KW waves owns a block of 4 rows and splits K among
//    its waves (KW = K / 512 for K <= 8192): each lane reads one 16-byte
//    chunk (8 weights) of each of the 4 rows with 128-bit non-temporal loads,
//    fully coalesced, plus the matching 8 activations; f16 -> f32 widening
//    happens in registers; the waves' partial sums meet in LDS.  One block
//    per workgroup: the hardware dispatcher starts a fresh workgroup as each
//    one retires, which streams HBM faster on MI355X than persistent waves
//    walking the rows (85 us against 93-97 us at N = 151936, K = 2048).
//  * Q8_0: a wave owns whole rows and holds the activation vector in VGPRs
//    (each lane keeps the slice of `a` that matches the blocks it decodes).
//    A 34-byte block is only 2-byte aligned, so the wave first copies S
//    whole rows (a contiguous, 16-byte aligned byte range when K % 256 == 0)
//    into its LDS slice with coalesced 128-bit loads, then each lane decodes
//    whole blocks from LDS (the block's dword-aligned 36-byte window, read
//    with 32-bit LDS loads and realigned by a byte permute) against its
//    register slice of `a`: sum_q = sum_i q_i a_i,
//    acc += d * sum_q, as the pages apply d after the block's int8 dot
//    product.  Q4_0 (18-byte blocks, 4-bit codes) is staged the same way; its
//    codes are turned into exact f16 values (u - 8) with one packed f16
//    subtraction per two codes and fed to mixed-precision FMAs.
//    The decode of a pass is branch-free so the rows' dependency
//    chains overlap, and the rows of a pass are reduced together by one
//    butterfly (each cross-lane step halves the values a lane carries).
//    The Q8_0 / Q4_0 grid is persistent: sized to fill the chip once, every
//    wave walks passes with a stride, balanced so all waves do equal work.
//  * Reductions: DPP within 16-lane rows, lane-xor across rows (64 lanes).
//  * SwiGLU: an f16 row block or a Q8_0 / Q4_0 pass holds gate rows and the
//    up rows of the same outputs, so after the reduction the gate and up
//    sums sit in two lanes of the same wave; one lane shuffle brings them
//    together and silu(g) * u is stored directly (no [2n] intermediate, no
//    second kernel).  Shapes those kernels cannot pair (unaligned or odd K,
//    very long K) take one GEMV over all 2n rows into scratch and one
//    element-wise pass.
#include "wq_internal.h"

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>

namespace wq {
namespace {

// What a GEMV kernel does with its row sums: store them (or add them: the
// residual flag), store silu(gate) * up (GLU), or keep a per-wave top-k list
// of (sum, row) and write it out at the end (TOPK: c is then a TopkCand array
// of one list of `aux` entries per wave, and the flag argument is that k).
enum { kModeStore = 0, kModeGlu = 1, kModeTopk = 2, kModeArgmax = 3 };

// Fused argmax of the f16 LM head (top-1): every workgroup folds its best row
// into one of kArgmaxSlots 64-bit slots with an atomic max of an order-keeping
// key, and argmax_finish reads the slots, writes the result and clears them.
// One set of slots per cached stream (kStreamSlots) plus one for the
// allocation-free entry point; zero (no candidate) between calls.
constexpr int kArgmaxSlots = 4096;  // about 9 f16 workgroups per slot at N = 151936 (1024 slots: 37, which measured 7 us slower)
__device__ unsigned long long g_argmax_slots[kStreamSlots + 1][kArgmaxSlots];

// Key of a candidate: the logit's bits made monotonic (negative values
// complemented, positive ones with the sign bit set; -0 counts as +0; NaN maps
// to the key 0, below every logit, so it is never taken) in the high word,
// 0xffffffff minus the id in the low word (equal logits: the lower id wins).
// Key 0: no candidate.
__device__ __forceinline__ unsigned long long argmax_key(float x, uint32_t id) {
    x = x + 0.0f;  // -0 -> +0
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    const unsigned long long key = (static_cast<unsigned long long>(k) << 32) | (0xffffffffu - id);
    return __builtin_isnan(x) ? 0ull : key;
}

// ------------------------------------------------------------------ f16 ----

// acc[r] += sum_e w[r] . (lo, hi) over the 8 f16 weights of each row's chunk,
// the rows' FMA chains advanced together (a mixed-precision FMA that depends
// on the one just before it costs a wait state).
template <int RB>
__device__ __forceinline__ void dot8_f16_rows(const uint4 (&w)[RB], float4 lo, float4 hi, float (&acc)[RB]) {
    const float x[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const uint32_t d = e < 2 ? w[r].x : e < 4 ? w[r].y : e < 6 ? w[r].z : w[r].w;
            acc[r] = fmaf(half_bits_to_float((e & 1) ? d >> 16 : d & 0xffffu), x[e], acc[r]);
        }
}

// K-split f16 GEMV (store and GLU modes): workgroup g (KW waves, KW =
// blockDim.x / 64) owns the g-th block of RB consecutive weight rows (GLU:
// RB/2 gate rows and the up rows of the same outputs) and wave w reads the
// w-th K slice of each row, T2 16-byte chunks per lane (chunk (w*T2 + t)*64 +
// lane of the row), against the matching activations.  Every wave has RB*T2
// loads in flight at once and the activations are read once per workgroup;
// the RB partial sums of a wave are reduced by one butterfly, then summed
// over the waves in wave order through LDS.  One block per workgroup and no
// grid stride: fresh workgroups from the hardware dispatcher keep every CU
// supplied until the last block (measured on MI355X, any per-workgroup loop
// over blocks, prefetched or not, costs 5-12 % at N = 151936).
// FULL: K == KW*T2*512 exactly.  Requires K % 8 == 0, 16-byte aligned a and b.
constexpr int kSplitMaxWaves = 16;

template <int T2, int RB, bool FULL, int MODE>
__global__ __launch_bounds__(kSplitMaxWaves * kWave) void gemv_f16_ksplit(const float *__restrict__ a,
                                                                          const uint16_t *__restrict__ b,
                                                                          float *__restrict__ c, int64_t n,
                                                                          int64_t k, int resid) {
    constexpr bool GLU = MODE == kModeGlu;
    static_assert(MODE == kModeStore || GLU || MODE == kModeArgmax, "store, GLU or argmax");
    static_assert(!GLU || RB % 2 == 0, "a GLU block pairs gate and up rows");
    constexpr int OC = GLU ? RB / 2 : RB;  // outputs per block
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int kw = blockDim.x / kWave;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * OC;  // first output of the block
    const int nch = static_cast<int>(k >> 3);

    uint4 wv[RB][T2];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        // Rows past the end are read clamped; their sums are never stored.
        const int64_t oc = min<int64_t>(r0 + r % OC, n - 1);
        const int64_t row = GLU && r >= OC ? n + oc : oc;
        const uint4 *brow = reinterpret_cast<const uint4 *>(b + row * k);
#pragma unroll
        for (int t = 0; t < T2; ++t) {
            const int idx = (w * T2 + t) * kWave + lane;
            wv[r][t] = (FULL || idx < nch) ? load_nt16(brow + idx) : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    float4 alo[T2], ahi[T2];
    const float4 *a4 = reinterpret_cast<const float4 *>(a);
#pragma unroll
    for (int t = 0; t < T2; ++t) {
        const int idx = (w * T2 + t) * kWave + lane;
        if (FULL || idx < nch) {
            alo[t] = a4[2 * idx];
            ahi[t] = a4[2 * idx + 1];
        } else {
            alo[t] = make_float4(0.f, 0.f, 0.f, 0.f);
            ahi[t] = alo[t];
        }
    }
    float acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = 0.f;
#pragma unroll
    for (int t = 0; t < T2; ++t) {
        uint4 wt[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) wt[r] = wv[r][t];
        dot8_f16_rows<RB>(wt, alo[t], ahi[t], acc);
    }
    // rows_sum leaves row j's sum in lanes j*(64/RB) ..; lane j (< RB) takes it.
    float v = __shfl(rows_sum<RB, kWave>(acc, lane), (lane % RB) * (kWave / RB), kWave);
    if (kw > 1) {
        __shared__ float part[kSplitMaxWaves][RB];
        if (lane < RB) part[w][lane] = v;
        __syncthreads();
        if (w != 0) return;
        v = part[0][lane % RB];
        for (int q = 1; q < kw; ++q) v += part[q][lane % RB];
    }
    if constexpr (GLU) {
        const float up = __shfl_down(v, OC, kWave);  // lane j + OC holds the up sum of output j
        if (lane < OC && r0 + lane < n) c[r0 + lane] = silu(v) * up;
    } else if constexpr (MODE == kModeArgmax) {
        // resid is the slot set; the block's best row goes to one slot.
        static_assert(RB <= 4, "the block's rows sit in one quad");
        unsigned long long key = (lane < RB && r0 + lane < n) ? argmax_key(v, static_cast<uint32_t>(r0 + lane)) : 0ull;
        key = max(key, static_cast<unsigned long long>(__shfl_xor(key, 1, kWave)));
        key = max(key, static_cast<unsigned long long>(__shfl_xor(key, 2, kWave)));
        if (lane == 0 && key != 0ull) atomicMax(&g_argmax_slots[resid][blockIdx.x % kArgmaxSlots], key);
    } else {
        if (lane < RB && r0 + lane < n) c[r0 + lane] = resid ? c[r0 + lane] + v : v;
    }
}

// Any K, any 2-byte alignment of b: one wave per row, lanes stride over K.
template <bool TOPK>
__global__ __launch_bounds__(256) void gemv_f16_any(const float *__restrict__ a,
                                                    const uint16_t *__restrict__ b,
                                                    float *__restrict__ c, int64_t n, int64_t k, int resid) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) / kWave;
    WaveTopk top;
    if constexpr (TOPK) top.init();
    for (int64_t row = wave; row < n; row += nwaves) {
        const uint16_t *brow = b + row * k;
        float acc = 0.f;
        for (int64_t kk = lane; kk < k; kk += kWave) acc = fmaf(half_bits_to_float(brow[kk]), a[kk], acc);
        acc = wave_sum(acc);
        if constexpr (TOPK)
            top.offer(resid, acc, static_cast<uint32_t>(row), lane == 0);
        else if (lane == 0)
            c[row] = resid ? c[row] + acc : acc;
    }
    if constexpr (TOPK) top.store(reinterpret_cast<TopkCand *>(c) + wave * resid, resid);
}

// The result of a fused argmax: the best slot of set `set` (the sentinel
// (-inf, no id) when every slot is empty), then every slot cleared for the
// next call.  One workgroup of 1024 lanes.
__global__ __launch_bounds__(1024) void argmax_finish(int set, float *__restrict__ vals, uint32_t *__restrict__ ids) {
    __shared__ unsigned long long wbest[16];
    unsigned long long best = 0ull;
#pragma unroll
    for (int i = threadIdx.x; i < kArgmaxSlots; i += 1024) {
        best = max(best, g_argmax_slots[set][i]);
        g_argmax_slots[set][i] = 0ull;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) best = max(best, static_cast<unsigned long long>(__shfl_xor(best, d, kWave)));
    if ((threadIdx.x & (kWave - 1)) == 0) wbest[threadIdx.x / kWave] = best;
    __syncthreads();
    if (threadIdx.x != 0) return;
    for (int w = 1; w < 16; ++w) best = max(best, wbest[w]);
    if (best == 0ull) {
        vals[0] = -__builtin_huge_valf();
        ids[0] = kTopkNoId;
        return;
    }
    const uint32_t k = static_cast<uint32_t>(best >> 32);
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    vals[0] = __builtin_bit_cast(float, u);
    ids[0] = 0xffffffffu - static_cast<uint32_t>(best & 0xffffffffu);
}

// ------------------------------------------------------- Q8_0 and Q4_0 ----

enum { QFMT_Q8_0 = 1, QFMT_Q4_0 = 2 };

// Block bytes, and 16-byte chunks each lane stages per pass (the stage holds
// whole rows: 8 rows of Q8_0 at K = 2048, 16 rows of Q4_0 at K = 2048).
template <int FMT>
struct QB {
    static constexpr int kBytes = FMT == QFMT_Q8_0 ? 34 : 18;
    static constexpr int kChunks = FMT == QFMT_Q8_0 ? 17 : 18;
    static constexpr int kStage = kChunks * 64 * 16;
};

// Dot product of one Q8_0 block held in LDS at byte offset pb with the 32
// activations av[0..31]: returns d * sum_i q_i * av[i].
__device__ __forceinline__ float q8_block_dot(const uint8_t *stage, int pb, const float *av) {
    uint32_t wd[8];
    const uint32_t hb = block_window<8>(stage, pb, wd);
    // Four independent partial sums (one per byte lane) keep four FMA chains
    // in flight instead of one 32-long dependent chain.
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t q = wd[i];
        part[0] = fmaf(static_cast<float>(static_cast<int8_t>(q & 0xffu)), av[4 * i + 0], part[0]);
        part[1] = fmaf(static_cast<float>(static_cast<int8_t>((q >> 8) & 0xffu)), av[4 * i + 1], part[1]);
        part[2] = fmaf(static_cast<float>(static_cast<int8_t>((q >> 16) & 0xffu)), av[4 * i + 2], part[2]);
        part[3] = fmaf(static_cast<float>(static_cast<int8_t>(q >> 24)), av[4 * i + 3], part[3]);
    }
    return half_bits_to_float(hb) * ((part[0] + part[1]) + (part[2] + part[3]));
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// (u - 8) for the 4-bit codes in bits 0..3 of both 16-bit halves of x, or
// 16 * (u - 8) for codes in bits 4..7 (HI): the code is placed in the
// mantissa of the f16 1024 (0x6400), which reads as 1024 + u (1024 + 16 u),
// and one packed subtraction removes 1032 (1152).  Every step is exact.
// The mask (in a VGPR) and 0x64006400 (in an SGPR) are register operands so
// that the and-or is one v_and_or_b32: a gfx9 VOP3 instruction takes no
// literal and at most one scalar operand.
struct Q4Consts {
    uint32_t lo, hi, magic;
};
__device__ __forceinline__ Q4Consts q4_consts() {
    Q4Consts k;
    asm("v_mov_b32 %0, 0x000f000f" : "=v"(k.lo));
    asm("v_mov_b32 %0, 0x00f000f0" : "=v"(k.hi));
    asm("s_mov_b32 %0, 0x64006400" : "=s"(k.magic));
    return k;
}
template <bool HI>
__device__ __forceinline__ h2 q4_pair(uint32_t x, const Q4Consts &k) {
    const uint32_t m = (x & (HI ? k.hi : k.lo)) | k.magic;
    const _Float16 bias = HI ? static_cast<_Float16>(1152.0f) : static_cast<_Float16>(1032.0f);
    return __builtin_bit_cast(h2, m) - h2{bias, bias};
}

// Dot product of one Q4_0 block in LDS at byte offset pb with av[0..31]:
// d * sum_i (u_i - 8) * av[i].  Byte j of the 16 code bytes (block bytes
// 2..17, read through block_window) holds weight 2j in its low nibble and
// 2j + 1 in its high nibble.  Codes from high nibbles come out scaled by 16
// and are summed apart; the exact power-of-two 1/16 is applied at the end.
// The f16 code values feed mixed-precision FMAs (f32 activation, f32 sum).
__device__ __forceinline__ float q4_block_dot(const uint8_t *stage, int pb, const float *av) {
    uint32_t wd[4];
    const uint32_t hb = block_window<4>(stage, pb, wd);
    const Q4Consts kc = q4_consts();
    float lo[2] = {0.f, 0.f}, hi[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // dword i = code bytes 4i .. 4i+3 = weights 8i .. 8i+7
        const uint32_t w = wd[i], w8 = wd[i] >> 8;
        const h2 p0 = q4_pair<false>(w, kc);   // weights 8i+0, 8i+4
        const h2 p1 = q4_pair<true>(w, kc);    // 8i+1, 8i+5 (x16)
        const h2 p2 = q4_pair<false>(w8, kc);  // 8i+2, 8i+6
        const h2 p3 = q4_pair<true>(w8, kc);   // 8i+3, 8i+7 (x16)
        const float *x = av + 8 * i;
        lo[0] = fmaf(static_cast<float>(p0.x), x[0], lo[0]);
        lo[1] = fmaf(static_cast<float>(p0.y), x[4], lo[1]);
        lo[0] = fmaf(static_cast<float>(p2.x), x[2], lo[0]);
        lo[1] = fmaf(static_cast<float>(p2.y), x[6], lo[1]);
        hi[0] = fmaf(static_cast<float>(p1.x), x[1], hi[0]);
        hi[1] = fmaf(static_cast<float>(p1.y), x[5], hi[1]);
        hi[0] = fmaf(static_cast<float>(p3.x), x[3], hi[0]);
        hi[1] = fmaf(static_cast<float>(p3.y), x[7], hi[1]);
    }
    return half_bits_to_float(hb) * ((lo[0] + lo[1]) + 0.0625f * (hi[0] + hi[1]));
}

template <int FMT>
__device__ __forceinline__ float block_dot(const uint8_t *stage, int pb, const float *av) {
    if constexpr (FMT == QFMT_Q8_0)
        return q8_block_dot(stage, pb, av);
    else
        return q4_block_dot(stage, pb, av);
}

// One wave per workgroup.  LPR lanes share a row; lane l covers blocks
// j = l % LPR + LPR * t (t < J) of that row and keeps a[32 j .. 32 j + 32) in
// VGPRs.  A pass covers S = SL * (64 / LPR) consecutive rows, i.e. S * row_bytes
// contiguous bytes (at most kChunks * 64 16-byte chunks).  The next pass is in
// flight in registers (kChunks independent 128-bit loads per lane) while the
// current pass, already copied to LDS, is decoded; the SL rows a lane group
// decodes are unrolled so their LDS reads and reductions interleave.
// Requires K % 256 == 0 (rows are whole 16-byte chunks), 16-byte aligned a, b.
// GLU: n is the output count and b has 2n rows; a pass stages HS = S/2 gate
// rows (stage rows 0 .. HS-1) and the up rows of the same outputs (stage rows
// HS .. S-1), two contiguous byte ranges.
template <int FMT, int J, int LPR, int SL, int MODE>
__global__ __launch_bounds__(64) void gemv_q_staged(const float *__restrict__ a,
                                                    const uint8_t *__restrict__ b,
                                                    float *__restrict__ c, int64_t n, int64_t k,
                                                    int64_t passes, int resid) {
    constexpr bool GLU = MODE == kModeGlu;
    extern __shared__ uint4 stage4[];
    constexpr int BB = QB<FMT>::kBytes;
    constexpr int CH = QB<FMT>::kChunks;
    constexpr int RPL = kWave / LPR;
    constexpr int S = SL * RPL;
    static_assert(!GLU || S % 2 == 0, "a GLU pass pairs gate and up rows");
    constexpr int HS = GLU ? S / 2 : S;  // outputs per pass
    const int lane = threadIdx.x;
    const int nb = static_cast<int>(k >> 5);
    const int row_bytes = nb * BB;
    const int jl = lane % LPR;
    const int rsub = lane / LPR;


    // Staging guards are wave-uniform: a whole 1 KiB load (or LDS write) is
    // skipped when the pass ends before it; inside the last one, lanes past
    // the end re-read the pass's last chunk (in bounds) and write it to LDS
    // slots nobody reads.  No per-lane exec masking in the streaming loop.
    uint4 next[CH];
    const int hc = HS * row_bytes / 16;  // stage chunks of one GLU half
    auto fetch = [&](int64_t p) {
        const int nch = static_cast<int>(min<int64_t>(HS, n - p * HS)) * row_bytes / 16;
        const uint4 *src = reinterpret_cast<const uint4 *>(b + p * HS * row_bytes);
        if constexpr (GLU) {
            // Stage chunk ci < hc: gate chunk ci; else up chunk ci - hc.  Chunks
            // past a half's end (last pass) re-read its last chunk, in bounds.
            const uint4 *usrc = reinterpret_cast<const uint4 *>(b + (n + p * HS) * row_bytes);
#pragma unroll
            for (int u = 0; u < CH; ++u)
                if (u * kWave < 2 * hc) {
                    const int ci = u * kWave + lane;
                    const bool up = ci >= hc;
                    next[u] = load_nt16((up ? usrc : src) + min(up ? ci - hc : ci, nch - 1));
                }
        } else {
#pragma unroll
            for (int u = 0; u < CH; ++u)
                if (u * kWave < nch) next[u] = load_nt16(src + min(u * kWave + lane, nch - 1));
        }
    };

    const uint8_t *stage = reinterpret_cast<const uint8_t *>(stage4);
    WaveTopk top;
    if constexpr (MODE == kModeTopk) top.init();
    int64_t p = blockIdx.x;
    // Waves that walk several passes issue their first pass's weights before
    // the activation slices (measured on MI355X: Q8_0 LM head 58.3 -> 56.9 us);
    // single-pass waves (small matrices) load the activations first (gate/up
    // 6144 x 2048: 6.7 -> 5.9 us).
    const bool weights_first = passes > static_cast<int64_t>(gridDim.x);
    if (weights_first && p < passes) fetch(p);
    float av[J][32];
#pragma unroll
    for (int t = 0; t < J; ++t) {
        const int j = jl + LPR * t;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < nb) v = reinterpret_cast<const float4 *>(a + 32 * j)[i];
            av[t][4 * i + 0] = v.x;
            av[t][4 * i + 1] = v.y;
            av[t][4 * i + 2] = v.z;
            av[t][4 * i + 3] = v.w;
        }
    }
    if (!weights_first) {
        wait_vmem_all();
        if (p < passes) fetch(p);
    }
    wait_vmem_all();
    for (; p < passes; p += gridDim.x) {
        const int64_t row0 = p * HS;  // first output of the pass
        const int rows = static_cast<int>(min<int64_t>(HS, n - row0));
        const int nch = GLU ? 2 * hc : rows * row_bytes / 16;
        __syncthreads();  // the previous pass is fully read from LDS
#pragma unroll
        for (int u = 0; u < CH; ++u)
            if (u * kWave < nch) stage4[u * kWave + lane] = next[u];
        __syncthreads();
        if (p + gridDim.x < passes) fetch(p + gridDim.x);  // in flight during the decode below
        // Branch-free decode: every (row, slot) reads an in-bounds block of the
        // stage (rows past `rows` hold stale bytes, slots past the row end use
        // the row's last block) and the result is masked, so all SL * J block
        // dot products sit in one basic block and their latencies overlap.
        float acc[SL];
#pragma unroll
        for (int sl = 0; sl < SL; ++sl) {
            const int srow = sl * RPL + rsub;
            acc[sl] = 0.f;
#pragma unroll
            for (int t = 0; t < J; ++t) {
                const int j = jl + LPR * t;
                const float d = block_dot<FMT>(stage, srow * row_bytes + BB * min(j, nb - 1), av[t]);
                acc[sl] += (j < nb) ? d : 0.f;
            }
            if ((GLU ? srow % HS : srow) >= rows) acc[sl] = 0.f;
        }
        // One butterfly reduction for all SL rows of the lane group; lane
        // jl then holds the sum of row sl = jl / (LPR / SL), stored by the
        // first lane of each run: one store instruction for the pass.
        const float sum = rows_sum<SL, LPR>(acc, jl);
        const int sl_mine = jl / (LPR / SL);
        const int srow_mine = sl_mine * RPL + rsub;
        if constexpr (GLU) {
            // Up row srow + HS is held D lanes up: by sl + SL/2 of the same
            // lane group (SL >= 2), or by lane group rsub + RPL/2 (SL == 1).
            constexpr int D = SL >= 2 ? LPR / 2 : kWave / 2;
            const float up = __shfl_down(sum, D, kWave);
            if (jl % (LPR / SL) == 0 && srow_mine < HS && srow_mine < rows)
                c[row0 + srow_mine] = silu(sum) * up;
        } else if constexpr (MODE == kModeTopk) {
            top.offer(resid, sum, static_cast<uint32_t>(row0 + srow_mine),
                      jl % (LPR / SL) == 0 && srow_mine < rows);
        } else {
            if (jl % (LPR / SL) == 0 && srow_mine < rows) {
                float *dst = c + row0 + srow_mine;
                *dst = resid ? *dst + sum : sum;
            }
        }
    }
    if constexpr (MODE == kModeTopk)
        top.store(reinterpret_cast<TopkCand *>(c) + static_cast<int64_t>(blockIdx.x) * resid, resid);
}

// K-split quantized GEMV for long rows (store mode, optional residual).
// Workgroup g (KW = ceil(nb / 64) waves) owns rows [g S, g S + S) and wave w
// the 64-block slice w of every row: lane l decodes block 64 w + l against
// a[32 (64 w + l) ..] held in 32 VGPRs, however long K is.  Each wave copies
// the S slices of its rows (S byte ranges of up to 64 blocks, each a whole
// number of 16-byte chunks because K % 256 == 0) into its own LDS region with
// coalesced 128-bit loads, decodes them, reduces its S row partials with one
// butterfly, and the KW wave partials are summed in wave order through LDS.
// One pass per workgroup: as for the f16 GEMV, fresh workgroups from the
// hardware dispatcher stream HBM better than persistent waves, and with `a`
// spread over the waves no wave re-reads a long activation vector per row.
template <int FMT, int S>
__global__ __launch_bounds__(kSplitMaxWaves * kWave) void gemv_q_ksplit(const float *__restrict__ a,
                                                                        const uint8_t *__restrict__ b,
                                                                        float *__restrict__ c, int64_t n,
                                                                        int64_t k, int resid) {
    extern __shared__ uint4 stage4[];
    constexpr int BB = QB<FMT>::kBytes;
    constexpr int SLICE = kWave * BB;       // bytes of a full 64-block slice of a row
    constexpr int SCH = SLICE / 16;         // its 16-byte chunks (136 for Q8_0, 72 for Q4_0)
    constexpr int LPS = (SCH + kWave - 1) / kWave;  // chunk loads per lane and row
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int kw = blockDim.x / kWave;
    const int nb = static_cast<int>(k >> 5);
    const int64_t row_bytes = static_cast<int64_t>(nb) * BB;
    const int nbw = min(kWave, nb - kWave * w);  // blocks in this wave's slice, a multiple of 8
    const int sch = nbw * BB / 16;               // chunks of the slice
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * S;
    const int rows = static_cast<int>(min<int64_t>(S, n - r0));

    uint4 v[S][LPS];
#pragma unroll
    for (int r = 0; r < S; ++r) {
        // Rows past the end are read clamped; their sums are never stored.
        const int64_t row = min<int64_t>(r0 + r, n - 1);
        const uint4 *src = reinterpret_cast<const uint4 *>(b + row * row_bytes + static_cast<int64_t>(w) * SLICE);
#pragma unroll
        for (int u = 0; u < LPS; ++u)
            if (u * kWave < sch) v[r][u] = load_nt16(src + min(u * kWave + lane, sch - 1));
    }
    const int j = kWave * w + lane;
    float av[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < nb) x = reinterpret_cast<const float4 *>(a + 32 * j)[i];
        av[4 * i + 0] = x.x;
        av[4 * i + 1] = x.y;
        av[4 * i + 2] = x.z;
        av[4 * i + 3] = x.w;
    }
    uint4 *stage = stage4 + w * S * SCH;  // this wave's region: S slices at a stride of SCH chunks
#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
        for (int u = 0; u < LPS; ++u)
            if (u * kWave < sch && u * kWave + lane < sch) stage[r * SCH + u * kWave + lane] = v[r][u];
    __syncthreads();
    const uint8_t *st = reinterpret_cast<const uint8_t *>(stage);
    const int pb = BB * min(lane, nbw - 1);  // lanes past the slice decode its last block, masked
    float acc[S];
#pragma unroll
    for (int r = 0; r < S; ++r) {
        acc[r] = block_dot<FMT>(st, r * SLICE + pb, av);
        if (lane >= nbw || r >= rows) acc[r] = 0.f;
    }
    // rows_sum leaves row r's partial in lanes r * (64 / S) ..; one lane per row keeps it.
    const float sum = rows_sum<S, kWave>(acc, lane);
    __shared__ float part[kSplitMaxWaves][S];
    if (lane % (kWave / S) == 0) part[w][lane / (kWave / S)] = sum;
    __syncthreads();
    if (w == 0 && lane < rows) {
        float t = part[0][lane];
        for (int q = 1; q < kw; ++q) t += part[q][lane];
        float *dst = c + r0 + lane;
        *dst = resid ? *dst + t : t;
    }
}

// ------------------------------------ Q8_0 and Q4_0 from row chunks ----
// Quantized GEMV that decodes every weight byte in the register it was loaded
// into: no LDS staging, one pass per workgroup (as the f16 K-split kernel).
// A block is B bytes (Q8_0: 34, Q4_0: 18) and each code byte carries W
// weights (1 or 2).  With K % 256 == 0 a row of nb blocks is C = B nb / 16
// whole 16-byte chunks.  A workgroup owns RB rows.  "Full" unit U (< C / 64)
// gives lane L chunk 64 U + L of every one of the RB rows (one activation
// window, RB rows); the last rem = C % 64 chunks of the RB rows form rem * RB
// (row, chunk) pairs.  With R2 = rem rounded up to a power of two, pair
// e = R2 r + co (remainder chunk co < rem of row r) sits on lane e % 64 of the
// "remainder" unit e / 64: a row's remainder chunks are consecutive lanes of
// one aligned group of R2 lanes (coalesced), summed by a butterfly inside the
// group.  Wave w takes full units w NF .. w NF + NF - 1 and remainder units
// w NR .. w NR + NR - 1.  A row's sum is its full-unit sum (the same lanes and
// the same waves for every row) plus its remainder sum, added once at the
// end, so equal rows give equal f32 results wherever they sit.
//
// Chunk c (bytes 16c .. 16c + 15 of a row) holds codes of at most two blocks
// (a block is longer than a chunk and at most one starts inside it): j0, the
// block in progress at byte 16c - 1, and j0 + 1 when that block's scale
// starts inside the chunk, at the even byte p = B (j0 + 1) - 16 c <= 14.
// Dwords 0 .. bd - 1 hold codes of j0 and dwords bd .. 3 codes of j0 + 1, with
// bd = (p + 2) / 4 (bd = 4 when no block starts in the chunk); the two scale
// bytes are paired with zero activations.  Code byte i takes the W
// activations from s0 + W i before the scale and s0 + W (i - 2) after it,
// s0 = 32 j0 + W (16 c - B j0 - 2).  The scale of j0 + 1 is read from the
// chunk itself; the scale of j0 lies in chunk c - 1 or c - 2 of the same row
// (dsrc lanes back), whose lane extracted it as its own start scale and hands
// it over with ds_bpermute; lanes whose source chunk is in another unit load
// those two bytes from memory instead (a buffer load that every other lane
// turns into an out-of-range no-op).
template <int FMT>
struct QC {
    static constexpr int kB = QB<FMT>::kBytes;
    static constexpr int kW = FMT == QFMT_Q8_0 ? 1 : 2;  // weights per code byte
    static constexpr int kX = 16 * kW;                   // activations per chunk
};
struct ChunkGeo {
    int p;     // byte of the block start in the chunk, or >= 16 when none
    int bd;    // dwords of block j0
    int s0;    // activation index of byte 0
    int j0;    // block in progress at the chunk start (-1 for chunk 0)
    int dsrc;  // chunk c - dsrc holds the scale of j0 (1 or 2)
};
template <int FMT>
__device__ __forceinline__ ChunkGeo chunk_geo(int c) {
    constexpr int B = QC<FMT>::kB, W = QC<FMT>::kW;
    ChunkGeo g;
    g.j0 = (16 * c + B - 1) / B - 1;
    g.p = B * (g.j0 + 1) - 16 * c;
    g.bd = g.p <= 14 ? (g.p + 2) >> 2 : 4;
    g.s0 = 32 * g.j0 + W * (16 * c - B * g.j0 - 2);
    g.dsrc = B * g.j0 >= 16 * (c - 1) ? 1 : 2;
    return g;
}

// Byte offsets (into a) of the activation groups of the chunk: group t covers
// code bytes 2t, 2t + 1 (2 W activations); the scale's group gets an
// out-of-range offset (the buffer load returns zeros), as do groups of units
// past the end.
template <int FMT>
__device__ __forceinline__ uint32_t act_group_offset(const ChunkGeo &g, int t, bool valid) {
    constexpr int W = QC<FMT>::kW;
    const int hp = g.p >> 1;  // the scale's group (>= 8: none)
    const int idx = g.s0 + 2 * W * t - (t > hp ? 2 * W : 0);
    return (valid && t != hp) ? static_cast<uint32_t>(idx) * 4u : 0x80000000u;
}

// The f16 bits at byte p (even, <= 14) of a 16-byte chunk: the dword pair
// holding it picked with a bit mask (v_bfi_b32; written as selects of the
// vector's fields, the compiler turned them into a dynamically indexed stack
// copy), then bytes p % 8 and p % 8 + 1 of the pair moved to the low half by
// one v_perm_b32 (selector 0x0c: a zero byte).  sel = half_selector(p).
__device__ __forceinline__ uint32_t half_selector(int p) {
    const uint32_t b = static_cast<uint32_t>(p) & 7u;
    return 0x0c0c0000u | ((b + 1u) << 8) | b;
}
__device__ __forceinline__ uint32_t chunk_half(const uint4 &v, int p, uint32_t sel) {
    const uint32_t m8 = 0u - ((static_cast<uint32_t>(p) >> 3) & 1u);
    const uint32_t lo = (v.z & m8) | (v.x & ~m8);
    const uint32_t hi = (v.w & m8) | (v.y & ~m8);
    return __builtin_amdgcn_perm(hi, lo, sel);
}

constexpr int kQcStream = 2;  // non-temporal buffer loads: every weight is read once

// One (weight row, chunk) against MR rows of activations: adds d_j0 * (codes
// of j0 . x_m) + d_j1 * (codes of j1 . x_m) to acc[m] for each m, the codes
// decoded once; h0, h1 hold the f16 bits of d_j0, d_j1 (low half), picked
// per dword and fed to the FMA as an f16 operand.  Q8_0: byte i of the chunk
// is one int8 code against x_m[i].  Q4_0: byte i holds codes for x_m[2i]
// (low nibble) and x_m[2i + 1] (high nibble); the high-nibble codes come out
// of q4_pair scaled by 16, and the caller has scaled the odd activations by
// the exact 1/16.  Each dword's products form one chain per row of A started
// from +0 (an FMA, so that f16 codes stay mixed-precision FMA operands).
template <int FMT, int MR>
__device__ __forceinline__ void chunk_dot(const uint4 &v, const float (&x)[MR][QC<FMT>::kX], uint32_t h0,
                                          uint32_t h1, int bd, float (&acc)[MR]) {
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    if constexpr (FMT == QFMT_Q8_0) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t q = wd[d];
            const float c0 = static_cast<float>(static_cast<int8_t>(q & 0xffu));
            const float c1 = static_cast<float>(static_cast<int8_t>((q >> 8) & 0xffu));
            const float c2 = static_cast<float>(static_cast<int8_t>((q >> 16) & 0xffu));
            const float c3 = static_cast<float>(static_cast<int8_t>(q >> 24));
            const uint32_t hs = d < bd ? h0 : h1;
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float t = c0 * x[m][4 * d + 0];
                t = fmaf(c1, x[m][4 * d + 1], t);
                t = fmaf(c2, x[m][4 * d + 2], t);
                t = fmaf(c3, x[m][4 * d + 3], t);
                acc[m] = fmaf(half_bits_to_float(hs), t, acc[m]);
            }
        }
    } else {
        // Codes of all four dwords first, then the dword chains advanced
        // together (dependent mixed-precision FMAs back to back stall).
        const Q4Consts kc = q4_consts();
        h2 pc[4][4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t q = wd[d], q8 = wd[d] >> 8;
            pc[d][0] = q4_pair<false>(q, kc);   // bytes 0, 2 low nibbles: x[8d], x[8d + 4]
            pc[d][1] = q4_pair<true>(q, kc);    // bytes 0, 2 high nibbles: x[8d + 1], x[8d + 5]
            pc[d][2] = q4_pair<false>(q8, kc);  // bytes 1, 3 low nibbles: x[8d + 2], x[8d + 6]
            pc[d][3] = q4_pair<true>(q8, kc);   // bytes 1, 3 high nibbles: x[8d + 3], x[8d + 7]
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float t[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) t[d] = fmaf(static_cast<float>(pc[d][0].x), x[m][8 * d], 0.f);
#pragma unroll
            for (int i = 1; i < 4; ++i)
#pragma unroll
                for (int d = 0; d < 4; ++d) t[d] = fmaf(static_cast<float>(pc[d][i].x), x[m][8 * d + i], t[d]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int d = 0; d < 4; ++d) t[d] = fmaf(static_cast<float>(pc[d][i].y), x[m][8 * d + 4 + i], t[d]);
#pragma unroll
            for (int d = 0; d < 4; ++d) acc[m] = fmaf(half_bits_to_float(d < bd ? h0 : h1), t[d], acc[m]);
        }
    }
}

// The activation window of a chunk in row row_off / (4 K) of A: 8 groups of
// 2 W floats (zeros at the scale's group, for units past the end and for rows
// past the end of A); Q4_0 odd (high-nibble)
// activations are scaled by 1/16 (a power of two: exact unless the product
// underflows f32's normal range, where it is rounded as a subnormal).
template <int FMT>
__device__ __forceinline__ void load_window(__amdgpu_buffer_rsrc_t ra, const ChunkGeo &g, bool ok,
                                            float (&x)[QC<FMT>::kX], uint32_t row_off) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        // The row offset goes into the range-checked (vector) offset, so a
        // row past the end of A reads zeros.
        const uint32_t o = act_group_offset<FMT>(g, t, ok);
        const int off = static_cast<int>(o == 0x80000000u ? o : o + row_off);
        if constexpr (FMT == QFMT_Q8_0) {
            const float2 f2 = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(ra, off, 0, 0));
            x[2 * t] = f2.x;
            x[2 * t + 1] = f2.y;
        } else {
            // Whole-vector cast: a bit cast of one ext-vector element reads
            // element 0 in this compiler.
            const float4 f4 = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0));
            x[4 * t] = f4.x;
            x[4 * t + 1] = f4.y;
            x[4 * t + 2] = f4.z;
            x[4 * t + 3] = f4.w;
        }
    }
}

constexpr int kQcMaxWaves = 4;

// v when keep, else +0 (through the bits, so that no branch is formed).
__device__ __forceinline__ float masked(float v, bool keep) {
    return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & (0u - static_cast<uint32_t>(keep)));
}

// MR rows of A (m_rows <= MR of them real, row-major [m_rows, K]; c is
// [m_rows, n]): every chunk is decoded once and applied to each row of A.
template <int FMT, int RB, int NF, int NR, int MODE = kModeStore, int MR = 1>
__global__ __launch_bounds__(kQcMaxWaves * kWave) void gemv_q_chunks(const float *__restrict__ a,
                                                                     const uint8_t *__restrict__ b,
                                                                     float *__restrict__ c, int64_t n, int64_t k,
                                                                     int resid, int m_rows) {
    static_assert(MODE != kModeArgmax || MR == 1, "the fused argmax is for one row of A");
    static_assert(RB * MR <= kWave, "one butterfly reduces every (row, row of A) sum");
    constexpr int NU = NF + NR;
    constexpr int B = QC<FMT>::kB, X = QC<FMT>::kX;
    constexpr uint32_t kOut = 0x80000000u;  // an out-of-range buffer offset: the load returns zeros
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    const int kw = blockDim.x / kWave;
    const int nb = static_cast<int>(k >> 5);
    const int C = (B * nb) >> 4;
    const int q = C >> 6, rem = C & 63;
    const int lr = rem > 0 ? 32 - __clz(rem - 1) : 0;  // R2 = 1 << lr
    const int P = rem > 0 ? RB << lr : 0;              // remainder pairs, padding included
    const uint32_t row_bytes = static_cast<uint32_t>(B) * static_cast<uint32_t>(nb);
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * RB;
    // The host checks n * row_bytes < 2^31 and 4 K MR < 2^31: every offset
    // below fits 31 bits and kOut (plus a row offset of A) is out of range of
    // both resources.  Rows of A past m_rows read as zeros.
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(b), 0, static_cast<int>(static_cast<uint32_t>(n) * row_bytes), 0x00020000);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(a), 0, static_cast<int>(4 * k * m_rows), 0x00020000);
    const uint32_t sbase = static_cast<uint32_t>(r0) * row_bytes;  // soffset of the workgroup's first row

    // Unit geometry.  Every load of a unit past the end (full units beyond
    // C / 64, remainder lanes beyond rem * RB) is out of range: its data,
    // scales and activations are zero, and bd = 0 makes both of its scales
    // the chunk's own (zero) one, so it adds exactly 0 with no branch.
    ChunkGeo geo[NU];
    uint32_t voff[NU];  // byte offset of the unit's chunk (remainder: from row r0)
    int co[NR > 0 ? NR : 1], rrow[NR > 0 ? NR : 1];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const int u = w * NF + f;
        const bool ok = u < q;
        geo[f] = chunk_geo<FMT>(ok ? 64 * u + lane : 0);
        if (!ok) geo[f].bd = 0;
        voff[f] = ok ? 16u * static_cast<uint32_t>(64 * u + lane) : kOut;
    }
#pragma unroll
    for (int g = 0; g < NR; ++g) {
        const int e = 64 * (w * NR + g) + lane;
        const bool ok = e < P && (e & ((1 << lr) - 1)) < rem;
        co[g] = ok ? e & ((1 << lr) - 1) : 0;
        rrow[g] = e < P ? e >> lr : 0;
        geo[NF + g] = chunk_geo<FMT>(64 * q + co[g]);
        if (!ok) geo[NF + g].bd = 0;
        const uint32_t roff = static_cast<uint32_t>(min<int64_t>(rrow[g], n - 1 - r0)) * row_bytes;
        voff[NF + g] = ok ? roff + 16u * static_cast<uint32_t>(64 * q + co[g]) : kOut;
    }

    // Loads in the order the decode consumes them: the activation windows
    // (Q4_0 scales half of them before any decode), the scale fallbacks, then
    // the weights.
    uint32_t rowoff[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) rowoff[r] = sbase + static_cast<uint32_t>(min<int64_t>(r, n - 1 - r0)) * row_bytes;
    float x[NU][MR][X];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int m = 0; m < MR; ++m)
            load_window<FMT>(ra, geo[u], voff[u] != kOut, x[u][m], static_cast<uint32_t>(4 * k * m));
    // Scales of j0 whose source chunk is in another unit: full units, lanes
    // 0 .. dsrc - 1; remainder units, the first dsrc chunks of each row's
    // remainder.  Every other lane's load is out of range.
    uint32_t fb[NF][RB], fr[NR > 0 ? NR : 1];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const bool need = geo[f].bd > 0 && lane < geo[f].dsrc;
        const uint32_t o = need ? static_cast<uint32_t>(B) * static_cast<uint32_t>(geo[f].j0) : kOut;
#pragma unroll
        for (int r = 0; r < RB; ++r)
            fb[f][r] = __builtin_amdgcn_raw_buffer_load_b16(rb, static_cast<int>(o), static_cast<int>(rowoff[r]), 0);
    }
#pragma unroll
    for (int g = 0; g < NR; ++g) {
        const ChunkGeo &ge = geo[NF + g];
        const bool need = ge.bd > 0 && co[g] < ge.dsrc;
        const uint32_t roff = static_cast<uint32_t>(min<int64_t>(rrow[g], n - 1 - r0)) * row_bytes;
        const uint32_t o = need ? roff + static_cast<uint32_t>(B) * static_cast<uint32_t>(ge.j0) : kOut;
        fr[g] = __builtin_amdgcn_raw_buffer_load_b16(rb, static_cast<int>(o), static_cast<int>(sbase), 0);
    }
    // Then the weight chunks, row by row (rows past n read the last row; never
    // stored), so that the decode of each row waits only for its own loads.
    uint4 wv[NF][RB];
    uint4 wr[NR > 0 ? NR : 1];
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rb, static_cast<int>(voff[f]),
                                                                 static_cast<int>(rowoff[r]), kQcStream);
            wv[f][r] = make_uint4(v.x, v.y, v.z, v.w);
        }
#pragma unroll
    for (int g = 0; g < NR; ++g) {
        const u32x4 v =
            __builtin_amdgcn_raw_buffer_load_b128(rb, static_cast<int>(voff[NF + g]), static_cast<int>(sbase), kQcStream);
        wr[g] = make_uint4(v.x, v.y, v.z, v.w);
    }
    // Every load above is issued before any decode (the scheduler otherwise
    // sinks some weight loads below the first unit's decode).
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FMT == QFMT_Q4_0) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int i = 1; i < X; i += 2) x[u][m][i] *= 0.0625f;
    }

    float acc[RB][MR];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[r][m] = 0.f;
    // Scale of j0: a lane with bd == 0 (no code of j0) reads its own start
    // scale through the permute (source = itself), fallback lanes their load.
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const ChunkGeo &g = geo[f];
        const int src = (g.bd == 0 ? lane : lane - g.dsrc) * 4;
        const bool fbl = g.bd > 0 && lane < g.dsrc;
        const uint32_t sel = half_selector(g.p);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const uint32_t own = chunk_half(wv[f][r], g.p, sel);
            const uint32_t got = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src, static_cast<int>(own)));
            const uint32_t b0 = fbl ? fb[f][r] : got;
            const uint32_t b1 = g.p <= 14 ? own : b0;
            chunk_dot<FMT, MR>(wv[f][r], x[f], b0, b1, g.bd, acc[r]);
        }
    }
    // Remainder sums: each row's group of R2 lanes reduced by a butterfly;
    // every lane files its value (unconditional stores: no branch), and row r
    // later reads the one of its group's first lane, pair R2 r.
    __shared__ float rpart[MR][kQcMaxWaves * (NR > 0 ? NR : 1) * kWave];
#pragma unroll
    for (int gi = 0; gi < NR; ++gi) {
        const ChunkGeo &g = geo[NF + gi];
        const uint32_t own = chunk_half(wr[gi], g.p, half_selector(g.p));
        const uint32_t got = static_cast<uint32_t>(
            __builtin_amdgcn_ds_bpermute((g.bd == 0 ? lane : lane - g.dsrc) * 4, static_cast<int>(own)));
        const uint32_t b0 = (g.bd > 0 && co[gi] < g.dsrc) ? fr[gi] : got;
        const uint32_t b1 = g.p <= 14 ? own : b0;
        float rsm[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) rsm[m] = 0.f;
        chunk_dot<FMT, MR>(wr[gi], x[NF + gi], b0, b1, g.bd, rsm);
        // The steps of group_sum<64>, the partner's value kept (bit mask) only
        // while the group is that large: no branch and no select for the
        // compiler to turn into one (a branch here splits the kernel, and the
        // compiler then waits on every load before decoding the full units).
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float rs = rsm[m];
            rs += masked(dpp_f32<0xb1>(rs), lr >= 1);
            rs += masked(dpp_f32<0x4e>(rs), lr >= 2);
            rs += masked(dpp_f32<0x141>(rs), lr >= 3);
            rs += masked(dpp_f32<0x140>(rs), lr >= 4);
            rs += masked(__shfl_xor(rs, 16, kWave), lr >= 5);
            rs += masked(__shfl_xor(rs, 32, kWave), lr >= 6);
            rpart[m][(w * NR + gi) * kWave + lane] = rs;
        }
    }
    // Full-unit sums: value j = r MR + m (weight row r, row m of A) of every
    // lane, reduced by one butterfly (lane j 64 / (RB MR) ends with sum j),
    // then the waves in order through LDS, then the remainder.
    constexpr int RM = RB * MR;
    float accf[RM];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) accf[r * MR + m] = acc[r][m];
    const float sum = rows_sum<RM, kWave>(accf, lane);
    __shared__ float part[kQcMaxWaves][RM];
    if (lane % (kWave / RM) == 0) part[w][lane / (kWave / RM)] = sum;
    __syncthreads();
    if constexpr (MODE == kModeArgmax) {
        // resid is the slot set: the workgroup's best row goes to one slot.
        if (w != 0) return;
        unsigned long long key = 0ull;
        if (lane < RB && r0 + lane < n) {
            float t = part[0][lane];
            for (int qq = 1; qq < kw; ++qq) t += part[qq][lane];
            if (rem > 0) t += rpart[0][lane << lr];
            key = argmax_key(t, static_cast<uint32_t>(r0 + lane));
        }
#pragma unroll
        for (int d = 1; d < RB; d *= 2) key = max(key, static_cast<unsigned long long>(__shfl_xor(key, d, kWave)));
        if (lane == 0 && key != 0ull) atomicMax(&g_argmax_slots[resid][blockIdx.x % kArgmaxSlots], key);
    } else if (w == 0 && lane < RM && r0 + lane / MR < n && lane % MR < m_rows) {
        const int r = lane / MR, m = lane % MR;
        float t = part[0][lane];
        for (int qq = 1; qq < kw; ++qq) t += part[qq][lane];
        if (rem > 0) t += rpart[m][r << lr];
        float *dst = c + static_cast<int64_t>(m) * n + r0 + r;
        *dst = resid ? *dst + t : t;
    }
}

// Any K % 32 == 0 and 2-byte aligned b: one wave per row, lanes stride over
// blocks, reading each block with 2-byte loads.
template <int FMT, bool TOPK>
__global__ __launch_bounds__(256) void gemv_q_any(const float *__restrict__ a, const uint8_t *__restrict__ b,
                                                  float *__restrict__ c, int64_t n, int64_t k, int resid) {
    constexpr int BB = QB<FMT>::kBytes;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) / kWave;
    const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) / kWave;
    const int64_t nb = k >> 5;
    WaveTopk top;
    if constexpr (TOPK) top.init();
    for (int64_t row = wave; row < n; row += nwaves) {
        const uint8_t *brow = b + row * nb * BB;
        float acc = 0.f;
        for (int64_t j = lane; j < nb; j += kWave) {
            const uint16_t *blk = reinterpret_cast<const uint16_t *>(brow + j * BB);
            const float *aj = a + 32 * j;
            float sumq = 0.f;
            if constexpr (FMT == QFMT_Q8_0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint32_t two = blk[1 + i];
                    sumq = fmaf(static_cast<float>(static_cast<int8_t>(two & 0xffu)), aj[2 * i], sumq);
                    sumq = fmaf(static_cast<float>(static_cast<int8_t>(two >> 8)), aj[2 * i + 1], sumq);
                }
            } else {
                // u16 i holds code bytes 2i (weights 4i, 4i+1) and 2i+1 (4i+2, 4i+3)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t two = blk[1 + i];
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        sumq = fmaf(static_cast<float>(static_cast<int>((two >> (4 * t)) & 0xfu) - 8), aj[4 * i + t],
                                    sumq);
                }
            }
            acc = fmaf(half_bits_to_float(blk[0]), sumq, acc);
        }
        acc = wave_sum(acc);
        if constexpr (TOPK)
            top.offer(resid, acc, static_cast<uint32_t>(row), lane == 0);
        else if (lane == 0)
            c[row] = resid ? c[row] + acc : acc;
    }
    if constexpr (TOPK) top.store(reinterpret_cast<TopkCand *>(c) + wave * resid, resid);
}

// ---------------------------------------------------------------- helpers --

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Number of workers for `items` work items when at most `cap` fit at once:
// the fewest that still finish in the same number of rounds, so that every
// worker gets the same count (within one).
inline int64_t balanced_workers(int64_t items, int64_t cap) {
    if (items <= cap) return items;
    const int64_t rounds = (items + cap - 1) / cap;
    return (items + rounds - 1) / rounds;
}

// SwiGLU as one GEMV over all 2n rows into scratch and one element-wise pass.
template <typename Gemv2n>
hipError_t glu_two_pass(float *c, int64_t n, hipStream_t s, Gemv2n &&gemv2n) {
    ScratchLease lease;
    void *scratch = nullptr;
    hipError_t e = lease.acquire(static_cast<size_t>(2 * n) * 4, s, &scratch);
    if (e != hipSuccess) return e;
    float *gu = static_cast<float *>(scratch);
    e = gemv2n(gu);
    if (e == hipSuccess) e = launch_reduce_splits(gu, c, 1, n, 2 * n, 1, kEpiGlu, s);
    const hipError_t er = lease.release();
    return e != hipSuccess ? e : er;
}

// Tuning hooks (unset or 0 = automatic): WQ_GEMV_SL forces the rows per lane
// group and pass of the staged quantized GEMV (1, 2 or 4), WQ_GEMV_SROWS the rows
// per workgroup of the K-split quantized GEMV (1, 2 or 4).
int env_int(const char *name) {
    const char *e = std::getenv(name);
    return e ? std::atoi(e) : 0;
}
int forced_sl() {
    static const int v = env_int("WQ_GEMV_SL");
    return v;
}
int forced_srows() {
    static const int v = env_int("WQ_GEMV_SROWS");
    return v;
}

// Launch helpers.  aux: the residual flag (kModeStore) or k (kModeTopk);
// *lists (kModeTopk): the number of per-wave lists the launch writes.

// K-split launch: T = 16-byte chunk slots per lane for the whole row
// (ceil(K / 512)); T2 of them per wave and KW = ceil(T / T2) waves; one
// workgroup per row block.
template <int T2, int RB, int MODE>
hipError_t run_f16_ksplit(const float *a, const uint16_t *b, float *c, int64_t n, int64_t k, hipStream_t s,
                          int resid) {
    constexpr int OC = MODE == kModeGlu ? RB / 2 : RB;
    const int64_t T = (k / 8 + kWave - 1) / kWave;
    const int kw = static_cast<int>((T + T2 - 1) / T2);
    const int64_t blocks = (n + OC - 1) / OC;
    if (kw < 1 || kw > kSplitMaxWaves || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (blocks == 0) return hipSuccess;
    const bool full = k == 512LL * T2 * kw;
    if (trace_enabled())
        fprintf(stderr, "[wqmm] gemv_f16_ksplit<T2=%d,RB=%d,full=%d,mode=%d> n=%lld k=%lld grid=%lld block=%d\n",
                T2, RB, full ? 1 : 0, MODE, (long long)n, (long long)k, (long long)blocks, kw * kWave);
    if (full)
        hipLaunchKernelGGL((gemv_f16_ksplit<T2, RB, true, MODE>), dim3(static_cast<unsigned>(blocks)),
                           dim3(kw * kWave), 0, s, a, b, c, n, k, resid);
    else
        hipLaunchKernelGGL((gemv_f16_ksplit<T2, RB, false, MODE>), dim3(static_cast<unsigned>(blocks)),
                           dim3(kw * kWave), 0, s, a, b, c, n, k, resid);
    return hipGetLastError();
}

// Shapes the K-split kernel takes: K % 8 == 0, 16-byte aligned a and b, and
// K <= 32768 (at most 16 waves of at most four chunk slots per lane).
inline bool f16_ksplit_ok(const float *a, const uint16_t *b, int64_t k) {
    const int64_t T = (k / 8 + kWave - 1) / kWave;
    return k % 8 == 0 && aligned16(a) && aligned16(b) && T >= 1 && T <= 4 * kSplitMaxWaves;
}

// Chunk slots per wave by K: one up to K = 8192, two up to 16384, four up to
// 32768.  Requires f16_ksplit_ok.
template <int MODE>
hipError_t f16_ksplit(const float *a, const uint16_t *b, float *c, int64_t n, int64_t k, hipStream_t s,
                      int resid) {
    const int64_t T = (k / 8 + kWave - 1) / kWave;
    if (T <= kSplitMaxWaves) return run_f16_ksplit<1, 4, MODE>(a, b, c, n, k, s, resid);
    if (T <= 2 * kSplitMaxWaves) return run_f16_ksplit<2, 4, MODE>(a, b, c, n, k, s, resid);
    return run_f16_ksplit<4, 4, MODE>(a, b, c, n, k, s, resid);
}

template <int FMT, int J, int LPR, int SL, int MODE = kModeStore>
hipError_t run_q_staged_sl(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, hipStream_t s,
                           int cus, int aux, int64_t *lists = nullptr) {
    constexpr int S = SL * (kWave / LPR);
    constexpr int HS = MODE == kModeGlu ? S / 2 : S;
    const int row_bytes = static_cast<int>((k >> 5) * QB<FMT>::kBytes);
    const int64_t passes = (n + HS - 1) / HS;
    // 12 single-wave workgroups per CU: measured best on MI355X (N = 151936).
    const int64_t blocks = balanced_workers(passes, static_cast<int64_t>(cus) * 12);
    const size_t lds = (static_cast<size_t>(S) * row_bytes + 1023) / 1024 * 1024;  // whole 1 KiB writes
    if (lists) *lists = blocks;
    if (trace_enabled())
        fprintf(stderr,
                "[wqmm] gemv_q_staged<fmt=%d,J=%d,LPR=%d,SL=%d,mode=%d> n=%lld k=%lld S=%d grid=%lld block=64 "
                "lds=%zu\n",
                FMT, J, LPR, SL, MODE, (long long)n, (long long)k, S, (long long)blocks, lds);
    hipLaunchKernelGGL((gemv_q_staged<FMT, J, LPR, SL, MODE>), dim3(blocks), dim3(64), lds, s, a, b, c, n, k,
                       passes, aux);
    return hipGetLastError();
}

// Rows per pass: as many as fit the stage (S * row_bytes <= kStage), but few
// enough that a small matrix still gives every CU about four waves (a wave
// decodes its rows after its loads land); SL is a power of two.
template <int FMT, int J, int LPR, int MODE = kModeStore>
hipError_t run_q_staged(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, hipStream_t s,
                        int cus, int aux, int64_t *lists = nullptr) {
    constexpr int RPL = kWave / LPR;
    const int row_bytes = static_cast<int>((k >> 5) * QB<FMT>::kBytes);
    const int64_t s_fit = QB<FMT>::kStage / row_bytes;
    const int64_t s_fill = std::max<int64_t>(1, n / (4LL * cus));
    // At most 4 rows per lane group and pass: with 12 waves per CU that was
    // measured faster than 8 or 16 rows for both formats at K = 2048.
    int64_t sl_max = std::max<int64_t>(1, std::min<int64_t>(4, std::min(s_fit, s_fill) / RPL));
    // Rows of 128 or more blocks (K >= 4096) with whole rows per lane group: one
    // row per pass, so a wave walks several passes with the next one in flight
    // (measured on MI355X at 11008 x 4096: Q8_0 16.4 -> 14.1 us, Q4_0 14.1 ->
    // 12.9 us; four rows per pass need 17 KiB of LDS per wave, so only 9 waves
    // fit on a CU and the 2752 passes take two rounds).
    if (MODE == kModeStore && LPR == kWave && k >= 4096) sl_max = 1;
    if (forced_sl() > 0) sl_max = forced_sl();
    if constexpr (J <= 2)
        if (sl_max >= 4 && 4 * RPL <= s_fit)
            return run_q_staged_sl<FMT, J, LPR, 4, MODE>(a, b, c, n, k, s, cus, aux, lists);
    if constexpr (J <= 4)
        if (sl_max >= 2 && 2 * RPL <= s_fit)
            return run_q_staged_sl<FMT, J, LPR, 2, MODE>(a, b, c, n, k, s, cus, aux, lists);
    return run_q_staged_sl<FMT, J, LPR, 1, MODE>(a, b, c, n, k, s, cus, aux, lists);
}

// The fused SwiGLU variant (n outputs, 2n rows): as run_q_staged over the 2n
// rows, but a pass needs at least two rows (one gate, one up), so with 64
// lanes per row SL >= 2.  Returns false (nothing launched) when no variant
// fits the stage.
template <int FMT, int J, int LPR>
bool run_q_staged_glu(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, hipStream_t s, int cus,
                      hipError_t *e) {
    constexpr int RPL = kWave / LPR;
    const int row_bytes = static_cast<int>((k >> 5) * QB<FMT>::kBytes);
    const int64_t s_fit = QB<FMT>::kStage / row_bytes;
    const int64_t s_fill = std::max<int64_t>(1, 2 * n / (4LL * cus));
    const int64_t sl_max = std::max<int64_t>(1, std::min<int64_t>(4, std::min(s_fit, s_fill) / RPL));
    if constexpr (J <= 2)
        if (sl_max >= 4 && 4 * RPL <= s_fit) {
            *e = run_q_staged_sl<FMT, J, LPR, 4, kModeGlu>(a, b, c, n, k, s, cus, 0);
            return true;
        }
    if constexpr (J <= 4)
        if ((sl_max >= 2 || RPL == 1) && 2 * RPL <= s_fit) {
            *e = run_q_staged_sl<FMT, J, LPR, 2, kModeGlu>(a, b, c, n, k, s, cus, 0);
            return true;
        }
    if constexpr (RPL >= 2) {
        *e = run_q_staged_sl<FMT, J, LPR, 1, kModeGlu>(a, b, c, n, k, s, cus, 0);
        return true;
    }
    return false;
}

// Upper bound of the per-wave lists any top-k GEMV launch writes: f16 and the
// plain kernels use at most 16 waves per CU (plus a partial workgroup), the
// staged kernel 12.
int64_t max_topk_lists(int cus) { return static_cast<int64_t>(cus) * 16 + 4; }

// Staged kernel when K % 256 == 0, a and b are 16-byte aligned and a row fits
// the stage with at most 8 blocks per lane; otherwise the plain kernel.
// MODE kModeStore (aux = residual flag) or kModeTopk (aux = k).
// The K-split kernel: 4 rows per workgroup while the workgroup's stage fits
// 64 KiB, else 2 or 1.  Measured on MI355X (Q8_0 and Q4_0, N = 1024 .. 8192,
// K = 4352 .. 11008): 4 rows beat 1 and 2 at every N (the activation slice a
// wave loads is amortised over more rows) and 8 (more staging registers).
template <int FMT>
hipError_t run_q_ksplit(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, hipStream_t s,
                        int resid) {
    const int kw = static_cast<int>((k / 32 + 63) / 64);
    const size_t slice = static_cast<size_t>(kWave) * QB<FMT>::kBytes;
    int srows = 4;
    while (srows > 1 && static_cast<size_t>(kw) * srows * slice > 65536) srows /= 2;
    if (forced_srows() > 0) srows = forced_srows();
    const int64_t blocks = (n + srows - 1) / srows;
    const size_t lds = static_cast<size_t>(kw) * srows * slice;
    if (trace_enabled())
        fprintf(stderr, "[wqmm] gemv_q_ksplit<fmt=%d,S=%d> n=%lld k=%lld grid=%lld block=%d lds=%zu\n", FMT, srows,
                (long long)n, (long long)k, (long long)blocks, kw * kWave, lds);
    const dim3 grid(static_cast<unsigned>(blocks)), block(kw * kWave);
    switch (srows) {
        case 4: hipLaunchKernelGGL((gemv_q_ksplit<FMT, 4>), grid, block, lds, s, a, b, c, n, k, resid); break;
        case 2: hipLaunchKernelGGL((gemv_q_ksplit<FMT, 2>), grid, block, lds, s, a, b, c, n, k, resid); break;
        default: hipLaunchKernelGGL((gemv_q_ksplit<FMT, 1>), grid, block, lds, s, a, b, c, n, k, resid); break;
    }
    return hipGetLastError();
}

// Plan of the register-chunk GEMV: RB rows per workgroup, NF full and NR
// remainder units per wave, KW <= 4 waves.  A forced plan that needs more
// waves falls back to the other kernels.
struct QcPlan {
    int rb, nf, nr, kw;
};
template <int FMT>
bool qc_fit(int64_t k, int rb, int nf, int nr, QcPlan *pl) {
    const int64_t nb = k / 32, C = QC<FMT>::kB * nb / 16, q = C / 64, rem = C % 64;
    int64_t r2 = rem > 0 ? 1 : 0;  // rem rounded up to a power of two
    while (r2 < rem) r2 *= 2;
    const int64_t P = r2 * rb;
    const int64_t kw = std::max<int64_t>(std::max<int64_t>((q + nf - 1) / nf, (P + 64 * nr - 1) / (64 * nr)), 1);
    if (kw > kQcMaxWaves) return false;
    *pl = QcPlan{rb, nf, nr, static_cast<int>(kw)};
    return true;
}
// Forced plan (wq_set_gemv_plan, both formats): rb * 256 + nf * 16 + nr,
// 0 = automatic, -1 = the kernel switched off.
std::atomic<int> g_qc_override{0};
bool qc_enabled() { return g_qc_override.load(std::memory_order_relaxed) >= 0; }
template <int FMT>
bool qc_plan(const float *a, const uint8_t *b, int64_t n, int64_t k, QcPlan *pl) {
    const int64_t nb = k / 32;
    if (nb % 8 != 0 || nb == 0 || !aligned16(a) || !aligned16(b) || n < 1) return false;
    if (n * QC<FMT>::kB * nb >= (int64_t(1) << 31) || 4 * k >= (int64_t(1) << 31)) return false;
    if (const int f = g_qc_override.load(std::memory_order_relaxed); f > 0)
        return qc_fit<FMT>(k, f >> 8, (f >> 4) & 15, f & 15, pl);
    // Measured on MI355X (M = 1, every plan against the staged / K-split
    // kernels, same box, us):
    //   Q8_0 151936x2048 (16,1,1) 54.3, staged 57.5; 11008x4096 (16,1,1) 12.6,
    //   (8,1,1) 13.2, K-split 14.1; 4096x11008 (4,3,1) 14.9, K-split 19.5;
    //   4096x4096 (8,1,1) 7.1, (4,2,1) 7.4; 2048x6144 (4,2,1) 6.3, K-split 7.3;
    //   6144x2048 and 2048x2048 staged 6.1 and 4.3, no plan faster.
    //   Q4_0 11008x4096 (8,1,1) 9.8, staged 13.1; 4096x11008 (4,3,1) 11.2,
    //   K-split 15.2; 4096x4096 (4,1,1) 5.9, staged 8.3; 2048x6144 (4,1,1) 5.5,
    //   K-split 6.2; rows of 64 blocks (K = 2048, the LM head 40.9 against
    //   41.3) keep the staged kernel.
    if constexpr (FMT == QFMT_Q8_0) {
        if (nb < 128) return n >= 65536 && qc_fit<FMT>(k, 16, 1, 1, pl);
        if (n >= 8192 && qc_fit<FMT>(k, 16, 1, 1, pl)) return true;
        if (n >= 4096 && qc_fit<FMT>(k, 8, 1, 1, pl)) return true;
        return qc_fit<FMT>(k, 4, 2, 1, pl) || qc_fit<FMT>(k, 4, 3, 1, pl);
    } else {
        if (nb < 128) return false;
        if (n >= 8192 && qc_fit<FMT>(k, 8, 1, 1, pl)) return true;
        return qc_fit<FMT>(k, 4, 1, 1, pl) || qc_fit<FMT>(k, 4, 3, 1, pl);
    }
}

template <int FMT, int RB, int NF, int NR, int MODE = kModeStore, int MR = 1>
hipError_t run_qc(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, hipStream_t s, int resid,
                  int kw, int m_rows = 1) {
    const int64_t blocks = (n + RB - 1) / RB;
    if (trace_enabled())
        fprintf(stderr,
                "[wqmm] gemv_q_chunks<fmt=%d,RB=%d,NF=%d,NR=%d,mode=%d,MR=%d> m=%d n=%lld k=%lld grid=%lld "
                "block=%d\n",
                FMT, RB, NF, NR, MODE, MR, m_rows, (long long)n, (long long)k, (long long)blocks, kw * kWave);
    hipLaunchKernelGGL((gemv_q_chunks<FMT, RB, NF, NR, MODE, MR>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kw * kWave), 0, s, a, b, c, n, k, resid, m_rows);
    return hipGetLastError();
}

// Returns false (nothing launched) when no instantiated plan fits.  MODE
// kModeStore (aux: residual flag) or kModeArgmax (aux: the slot set).
template <int FMT, int MODE = kModeStore>
bool launch_qc(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, hipStream_t s, int aux,
               hipError_t *e) {
    QcPlan pl;
    if (!qc_plan<FMT>(a, b, n, k, &pl)) return false;
    if (pl.rb == 8 && pl.nf == 2 && pl.nr == 1) *e = run_qc<FMT, 8, 2, 1, MODE>(a, b, c, n, k, s, aux, pl.kw);
    else if (pl.rb == 4 && pl.nf == 2 && pl.nr == 1) *e = run_qc<FMT, 4, 2, 1, MODE>(a, b, c, n, k, s, aux, pl.kw);
    else if (pl.rb == 4 && pl.nf == 3 && pl.nr == 1) *e = run_qc<FMT, 4, 3, 1, MODE>(a, b, c, n, k, s, aux, pl.kw);
    else if (pl.rb == 4 && pl.nf == 1 && pl.nr == 1) *e = run_qc<FMT, 4, 1, 1, MODE>(a, b, c, n, k, s, aux, pl.kw);
    else if (pl.rb == 8 && pl.nf == 1 && pl.nr == 1) *e = run_qc<FMT, 8, 1, 1, MODE>(a, b, c, n, k, s, aux, pl.kw);
    else if (pl.rb == 16 && pl.nf == 1 && pl.nr == 1) *e = run_qc<FMT, 16, 1, 1, MODE>(a, b, c, n, k, s, aux, pl.kw);
    else if (pl.rb == 2 && pl.nf == 2 && pl.nr == 1) *e = run_qc<FMT, 2, 2, 1, MODE>(a, b, c, n, k, s, aux, pl.kw);
    else return false;
    return true;
}

// Several rows of A (2 <= m <= MR) through one register-chunk launch.  The
// activation windows take NU * MR * (16 or 32) VGPRs, so fewer plans are
// compiled: MR = 2 Q8_0 (16,1,1) (8,1,1) (4,2,1) (4,3,1), Q4_0 (8,1,1) (4,1,1)
// (4,2,1); MR = 4 (Q8_0 only) (8,1,1) (4,1,1).
template <int FMT, int MR>
bool qc_compiled_rows(int rb, int nf, int nr) {
    if (nr != 1) return false;
    if constexpr (MR == 2 && FMT == QFMT_Q8_0)
        return (rb == 16 && nf == 1) || (rb == 8 && nf == 1) || (rb == 4 && nf == 2) || (rb == 4 && nf == 3);
    else if constexpr (MR == 2)
        return (rb == 8 && nf == 1) || (rb == 4 && nf == 1) || (rb == 4 && nf == 2);
    else if constexpr (MR == 4 && FMT == QFMT_Q8_0)
        return (rb == 8 && nf == 1) || (rb == 4 && nf == 1);
    return false;
}
template <int FMT, int MR>
bool qc_plan_rows(const float *a, const uint8_t *b, int64_t n, int64_t k, QcPlan *pl) {
    const int64_t nb = k / 32;
    if (nb % 8 != 0 || nb == 0 || !aligned16(a) || !aligned16(b) || n < 1) return false;
    if (n * QC<FMT>::kB * nb >= (int64_t(1) << 31) || 4 * k * MR >= (int64_t(1) << 31)) return false;
    if (const int f = g_qc_override.load(std::memory_order_relaxed); f > 0) {
        const int rb = f >> 8, nf = (f >> 4) & 15, nr = f & 15;
        return qc_compiled_rows<FMT, MR>(rb, nf, nr) && qc_fit<FMT>(k, rb, nf, nr, pl);
    }
    if constexpr (MR == 2 && FMT == QFMT_Q8_0) {
        if (n >= 8192 && qc_fit<FMT>(k, 16, 1, 1, pl)) return true;
        if (n >= 4096 && qc_fit<FMT>(k, 8, 1, 1, pl)) return true;
        return qc_fit<FMT>(k, 4, 2, 1, pl) || qc_fit<FMT>(k, 4, 3, 1, pl);
    } else if constexpr (MR == 2) {
        if (n >= 8192 && qc_fit<FMT>(k, 8, 1, 1, pl)) return true;
        return qc_fit<FMT>(k, 4, 1, 1, pl) || qc_fit<FMT>(k, 4, 2, 1, pl);
    } else if constexpr (MR == 4 && FMT == QFMT_Q8_0) {
        return qc_fit<FMT>(k, 8, 1, 1, pl) || qc_fit<FMT>(k, 4, 1, 1, pl);
    }
    return false;
}
template <int FMT, int MR>
bool launch_qc_rows(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k, hipStream_t s,
                    int resid, hipError_t *e) {
    QcPlan pl;
    if (!qc_plan_rows<FMT, MR>(a, b, n, k, &pl)) return false;
    const int mr = static_cast<int>(m);
    if constexpr (MR == 2 && FMT == QFMT_Q8_0) {
        if (pl.rb == 16 && pl.nf == 1) *e = run_qc<FMT, 16, 1, 1, kModeStore, 2>(a, b, c, n, k, s, resid, pl.kw, mr);
        else if (pl.rb == 8 && pl.nf == 1) *e = run_qc<FMT, 8, 1, 1, kModeStore, 2>(a, b, c, n, k, s, resid, pl.kw, mr);
        else if (pl.rb == 4 && pl.nf == 2) *e = run_qc<FMT, 4, 2, 1, kModeStore, 2>(a, b, c, n, k, s, resid, pl.kw, mr);
        else if (pl.rb == 4 && pl.nf == 3) *e = run_qc<FMT, 4, 3, 1, kModeStore, 2>(a, b, c, n, k, s, resid, pl.kw, mr);
        else return false;
    } else if constexpr (MR == 2) {
        if (pl.rb == 8 && pl.nf == 1) *e = run_qc<FMT, 8, 1, 1, kModeStore, 2>(a, b, c, n, k, s, resid, pl.kw, mr);
        else if (pl.rb == 4 && pl.nf == 1) *e = run_qc<FMT, 4, 1, 1, kModeStore, 2>(a, b, c, n, k, s, resid, pl.kw, mr);
        else if (pl.rb == 4 && pl.nf == 2) *e = run_qc<FMT, 4, 2, 1, kModeStore, 2>(a, b, c, n, k, s, resid, pl.kw, mr);
        else return false;
    } else if constexpr (MR == 4 && FMT == QFMT_Q8_0) {
        if (pl.rb == 8 && pl.nf == 1) *e = run_qc<FMT, 8, 1, 1, kModeStore, 4>(a, b, c, n, k, s, resid, pl.kw, mr);
        else if (pl.rb == 4 && pl.nf == 1) *e = run_qc<FMT, 4, 1, 1, kModeStore, 4>(a, b, c, n, k, s, resid, pl.kw, mr);
        else return false;
    } else {
        return false;
    }
    return true;
}

template <int FMT, int MODE>
hipError_t gemv_q_rows(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, hipStream_t s, int cus,
                       int aux, int64_t *lists) {
    const int64_t nb = k / 32;
    const int64_t row_bytes = nb * QB<FMT>::kBytes;
    if constexpr (MODE == kModeStore) {
        hipError_t e = hipSuccess;
        if (qc_enabled() && launch_qc<FMT>(a, b, c, n, k, s, aux, &e)) return e;
    }
    // Long rows (more than 128 blocks, up to 16 waves of 64): K split over the waves of a workgroup.
    if (MODE == kModeStore && nb % 8 == 0 && nb > 128 && nb <= 64 * kSplitMaxWaves && aligned16(a) && aligned16(b))
        return run_q_ksplit<FMT>(a, b, c, n, k, s, aux);
    if (nb % 8 == 0 && aligned16(a) && aligned16(b) && row_bytes <= QB<FMT>::kStage && nb <= 512) {
        if (nb >= 64) {
            switch ((nb + 63) / 64) {
                case 1: return run_q_staged<FMT, 1, 64, MODE>(a, b, c, n, k, s, cus, aux, lists);
                case 2: return run_q_staged<FMT, 2, 64, MODE>(a, b, c, n, k, s, cus, aux, lists);
                case 3: return run_q_staged<FMT, 3, 64, MODE>(a, b, c, n, k, s, cus, aux, lists);
                case 4: return run_q_staged<FMT, 4, 64, MODE>(a, b, c, n, k, s, cus, aux, lists);
                case 5: return run_q_staged<FMT, 5, 64, MODE>(a, b, c, n, k, s, cus, aux, lists);
                case 6: return run_q_staged<FMT, 6, 64, MODE>(a, b, c, n, k, s, cus, aux, lists);
                case 7: return run_q_staged<FMT, 7, 64, MODE>(a, b, c, n, k, s, cus, aux, lists);
                default: return run_q_staged<FMT, 8, 64, MODE>(a, b, c, n, k, s, cus, aux, lists);
            }
        } else if (nb >= 32) {
            if (nb == 32) return run_q_staged<FMT, 1, 32, MODE>(a, b, c, n, k, s, cus, aux, lists);
            return run_q_staged<FMT, 2, 32, MODE>(a, b, c, n, k, s, cus, aux, lists);
        } else {
            if (nb <= 16) return run_q_staged<FMT, 1, 16, MODE>(a, b, c, n, k, s, cus, aux, lists);
            return run_q_staged<FMT, 2, 16, MODE>(a, b, c, n, k, s, cus, aux, lists);
        }
    }
    const int64_t waves = balanced_workers(n, static_cast<int64_t>(cus) * 16);
    const int64_t blocks = (waves + 3) / 4;
    if (lists) *lists = blocks * 4;
    if (trace_enabled())
        fprintf(stderr, "[wqmm] gemv_q_any<fmt=%d,topk=%d> n=%lld k=%lld grid=%lld block=256\n", FMT,
                MODE == kModeTopk, (long long)n, (long long)k, (long long)blocks);
    hipLaunchKernelGGL((gemv_q_any<FMT, MODE == kModeTopk>), dim3(blocks), dim3(256), 0, s, a, b, c, n, k, aux);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_gemv_q(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, hipStream_t s,
                         int epi) {
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    const int64_t nb = k / 32;
    const int64_t row_bytes = nb * QB<FMT>::kBytes;
    const bool staged = nb % 8 == 0 && aligned16(a) && aligned16(b) && row_bytes <= QB<FMT>::kStage && nb <= 512;
    if (epi == kEpiGlu) {
        if (staged) {
            bool done = false;
            if (nb >= 64) {
                switch ((nb + 63) / 64) {
                    case 1: done = run_q_staged_glu<FMT, 1, 64>(a, b, c, n, k, s, di.cus, &e); break;
                    case 2: done = run_q_staged_glu<FMT, 2, 64>(a, b, c, n, k, s, di.cus, &e); break;
                    case 3: done = run_q_staged_glu<FMT, 3, 64>(a, b, c, n, k, s, di.cus, &e); break;
                    case 4: done = run_q_staged_glu<FMT, 4, 64>(a, b, c, n, k, s, di.cus, &e); break;
                    default: break;
                }
            } else if (nb >= 32) {
                done = nb == 32 ? run_q_staged_glu<FMT, 1, 32>(a, b, c, n, k, s, di.cus, &e)
                                : run_q_staged_glu<FMT, 2, 32>(a, b, c, n, k, s, di.cus, &e);
            } else {
                done = nb <= 16 ? run_q_staged_glu<FMT, 1, 16>(a, b, c, n, k, s, di.cus, &e)
                                : run_q_staged_glu<FMT, 2, 16>(a, b, c, n, k, s, di.cus, &e);
            }
            if (done) return e;
        }
        return glu_two_pass(c, n, s, [&](float *gu) { return launch_gemv_q<FMT>(a, b, gu, 2 * n, k, s, kEpiNone); });
    }
    return gemv_q_rows<FMT, kModeStore>(a, b, c, n, k, s, di.cus, epi == kEpiResidual, nullptr);
}

// f16 rows of any K and alignment (shapes the K-split kernel does not take):
// one wave per row.  MODE kModeStore or kModeTopk.
template <int MODE>
hipError_t gemv_f16_rows(const float *a, const uint16_t *b, float *c, int64_t n, int64_t k, hipStream_t s,
                         int cus, int aux, int64_t *lists) {
    const int64_t waves = balanced_workers(n, static_cast<int64_t>(cus) * 16);
    const int64_t blocks = (waves + 3) / 4;
    if (lists) *lists = blocks * 4;
    if (trace_enabled())
        fprintf(stderr, "[wqmm] gemv_f16_any<topk=%d> n=%lld k=%lld grid=%lld block=256\n", MODE == kModeTopk,
                (long long)n, (long long)k, (long long)blocks);
    hipLaunchKernelGGL((gemv_f16_any<MODE == kModeTopk>), dim3(blocks), dim3(256), 0, s, a, b, c, n, k, aux);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_f16(const float *a, const uint16_t *b, float *c, int64_t n, int64_t k,
                           hipStream_t s, int epi) {
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    if (epi == kEpiGlu) {
        if (f16_ksplit_ok(a, b, k)) return f16_ksplit<kModeGlu>(a, b, c, n, k, s, 0);
        return glu_two_pass(c, n, s, [&](float *gu) { return launch_gemv_f16(a, b, gu, 2 * n, k, s, kEpiNone); });
    }
    if (f16_ksplit_ok(a, b, k)) return f16_ksplit<kModeStore>(a, b, c, n, k, s, epi == kEpiResidual);
    return gemv_f16_rows<kModeStore>(a, b, c, n, k, s, di.cus, epi == kEpiResidual, nullptr);
}

bool set_gemv_plan_override(int rb, int nf, int nr) {
    if (rb == 0 && nf == 0 && nr == 0) {
        g_qc_override.store(0, std::memory_order_relaxed);
        return true;
    }
    if (rb == -1 && nf == 0 && nr == 0) {
        g_qc_override.store(-1, std::memory_order_relaxed);
        return true;
    }
    static const int kPlans[][3] = {{8, 2, 1}, {4, 2, 1}, {4, 3, 1}, {4, 1, 1}, {8, 1, 1}, {16, 1, 1}, {2, 2, 1}};
    for (const auto &pl : kPlans)
        if (pl[0] == rb && pl[1] == nf && pl[2] == nr) {
            g_qc_override.store(rb * 256 + nf * 16 + nr, std::memory_order_relaxed);
            return true;
        }
    return false;
}

hipError_t launch_gemv_q8_0(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k,
                            hipStream_t s, int epi) {
    return launch_gemv_q<QFMT_Q8_0>(a, b, c, n, k, s, epi);
}

hipError_t launch_gemv_q4_0(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k,
                            hipStream_t s, int epi) {
    return launch_gemv_q<QFMT_Q4_0>(a, b, c, n, k, s, epi);
}

bool launch_gemv_q_rows(const float *a, const uint8_t *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                        hipStream_t s, int epi, hipError_t *e) {
    if ((epi != kEpiNone && epi != kEpiResidual) || !qc_enabled() || m < 2 || m > 4) return false;
    const int resid = epi == kEpiResidual;
    if (fmt == QFMT_Q8_0)
        return m <= 2 ? launch_qc_rows<QFMT_Q8_0, 2>(a, b, c, m, n, k, s, resid, e)
                      : launch_qc_rows<QFMT_Q8_0, 4>(a, b, c, m, n, k, s, resid, e);
    if (fmt == QFMT_Q4_0 && m == 2) return launch_qc_rows<QFMT_Q4_0, 2>(a, b, c, m, n, k, s, resid, e);
    return false;
}

// Two rows of A cost the windows 32 registers per unit.  With at most three
// units per wave the kernel beats the weight stream on MI355X (Q8_0, two rows:
// 2048 x 2048 5.3 against 6.1 us, 6144 x 2048 7.4 against 8.3, 2048 x 6144 7.8
// against 9.2, 11008 x 4096 14.8 against 16.2); with four it does not (4096 x
// 11008, plan (4, 3, 1): 20.0 against 15.8 us), nor do Q4_0 or three and four
// rows (Q8_0 4 x 11008 x 4096: 24.6 against 18.0 us).
bool gemv_q_rows_auto(const float *a, const uint8_t *b, int fmt, int64_t m, int64_t n, int64_t k, int epi) {
    if (fmt != QFMT_Q8_0 || m != 2 || (epi != kEpiNone && epi != kEpiResidual) || !qc_enabled()) return false;
    QcPlan pl;
    return qc_plan_rows<QFMT_Q8_0, 2>(a, b, n, k, &pl) && pl.nf + pl.nr <= 3;
}

// Routes of an LM-head top-k call.  The logits route runs the fastest store
// GEMV into scratch and merges the logits 64 at a time: f16 rows the K-split
// kernel takes, and quantized rows of whole 256-column groups for k > 1 (the
// register-chunk / staged store kernels beat the per-wave lists once k is
// large: measured at N = 151936, k = 50, Q8_0 71.3 against 73.7 us, Q4_0 56.6
// against 59.3 us).  Top-1 of f16 (K-split) and Q8_0 / Q4_0 (register-chunk)
// rows takes the argmax fused into the GEMV.  Everything else keeps per-wave
// top-k lists inside the GEMV and merges them.
static bool lm_head_f16_logits_route(const float *a, const void *b, int fmt, int64_t n, int64_t k) {
    return fmt != QFMT_Q8_0 && fmt != QFMT_Q4_0 && n > 0 && f16_ksplit_ok(a, static_cast<const uint16_t *>(b), k);
}
static bool lm_head_q_logits_route(const float *a, const void *b, int fmt, int64_t n, int64_t k, int topk) {
    return (fmt == QFMT_Q8_0 || fmt == QFMT_Q4_0) && topk > 1 && n > 0 && (k / 32) % 8 == 0 && aligned16(a) &&
           aligned16(b);
}
static bool lm_head_logits_route(const float *a, const void *b, int fmt, int64_t n, int64_t k, int topk) {
    return lm_head_f16_logits_route(a, b, fmt, n, k) || lm_head_q_logits_route(a, b, fmt, n, k, topk);
}
static bool lm_head_q_argmax_route(const float *a, const void *b, int fmt, int64_t n, int64_t k, int topk) {
    QcPlan pl;
    const uint8_t *b8 = static_cast<const uint8_t *>(b);
    if (topk != 1 || n < 1 || !qc_enabled()) return false;
    if (fmt == QFMT_Q8_0) return qc_plan<QFMT_Q8_0>(a, b8, n, k, &pl);
    return fmt == QFMT_Q4_0 && qc_plan<QFMT_Q4_0>(a, b8, n, k, &pl);
}

size_t lm_head_topk_scratch_bytes(const float *a, const void *b, int fmt, int64_t n, int64_t k, int topk, int cus) {
    const size_t part = static_cast<size_t>(kTopkGroups) * topk * sizeof(TopkCand);
    if (lm_head_logits_route(a, b, fmt, n, k, topk)) return static_cast<size_t>((n * 4 + 255) / 256 * 256) + part;
    return static_cast<size_t>(max_topk_lists(cus)) * topk * sizeof(TopkCand) + part;
}

hipError_t launch_lm_head_topk(const float *a, const void *b, int fmt, int64_t n, int64_t k, int topk,
                               float *vals, uint32_t *ids, hipStream_t s, void *workspace, size_t workspace_bytes) {
    if (topk < 1 || topk > kTopkMax) return hipErrorInvalidValue;
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    const size_t need = lm_head_topk_scratch_bytes(a, b, fmt, n, k, topk, di.cus);
    ScratchLease lease;
    void *scratch = workspace;
    if (scratch) {
        if (workspace_bytes < need) return hipErrorInvalidValue;
    } else {
        e = lease.acquire(need, s, &scratch);
        if (e != hipSuccess) return e;
    }
    const uint16_t *b16 = static_cast<const uint16_t *>(b);
    const uint8_t *b8 = static_cast<const uint8_t *>(b);
    // Fused argmax: slot set of this stream, or the allocation-free entry point's own.
    const int set = workspace ? kStreamSlots : lease.slot();
    bool argmax_done = false;
    if (topk == 1 && set >= 0 && lm_head_f16_logits_route(a, b, fmt, n, k)) {
        e = f16_ksplit<kModeArgmax>(a, b16, nullptr, n, k, s, set);
        argmax_done = true;
    } else if (set >= 0 && lm_head_q_argmax_route(a, b, fmt, n, k, topk)) {
        argmax_done = fmt == QFMT_Q8_0 ? launch_qc<QFMT_Q8_0, kModeArgmax>(a, b8, nullptr, n, k, s, set, &e)
                                       : launch_qc<QFMT_Q4_0, kModeArgmax>(a, b8, nullptr, n, k, s, set, &e);
    }
    if (argmax_done) {
        if (e == hipSuccess) {
            if (trace_enabled()) fprintf(stderr, "[wqmm] argmax_finish set=%d\n", set);
            hipLaunchKernelGGL(argmax_finish, dim3(1), dim3(1024), 0, s, set, vals, ids);
            e = hipGetLastError();
        }
    } else if (lm_head_logits_route(a, b, fmt, n, k, topk)) {
        // The logits go to scratch (608 KB at N = 151936) and the merge reads
        // them 64 at a time.  A per-workgroup top-k list inside the f16 K-split
        // kernel would need a loop over row blocks, which costs more than the
        // logits round trip.
        const int64_t lbytes = (n * 4 + 255) / 256 * 256;
        float *logits = static_cast<float *>(scratch);
        TopkCand *partial = reinterpret_cast<TopkCand *>(static_cast<char *>(scratch) + lbytes);
        if (fmt == QFMT_Q8_0)
            e = gemv_q_rows<QFMT_Q8_0, kModeStore>(a, b8, logits, n, k, s, di.cus, 0, nullptr);
        else if (fmt == QFMT_Q4_0)
            e = gemv_q_rows<QFMT_Q4_0, kModeStore>(a, b8, logits, n, k, s, di.cus, 0, nullptr);
        else
            e = f16_ksplit<kModeStore>(a, b16, logits, n, k, s, 0);
        if (e == hipSuccess) e = launch_topk_merge(nullptr, 0, logits, n, topk, partial, vals, ids, s);
    } else {
        const int64_t cap = max_topk_lists(di.cus);
        TopkCand *cand = static_cast<TopkCand *>(scratch);
        TopkCand *partial = cand + cap * topk;
        float *out = reinterpret_cast<float *>(cand);
        // Every top-k launch below writes at most `cap` lists: balanced_workers never
        // exceeds its cap (16 waves per CU, rounded up to whole workgroups of 4, or
        // 12 single-wave workgroups per CU for the staged kernel).  Every list the
        // merge reads is written first by the same call, so the buffer needs no
        // clearing.  n == 0: no GEMV, and the merge of zero lists writes sentinels.
        int64_t lists = 0;
        if (n == 0)
            e = hipSuccess;
        else if (fmt == QFMT_Q8_0)
            e = gemv_q_rows<QFMT_Q8_0, kModeTopk>(a, b8, out, n, k, s, di.cus, topk, &lists);
        else if (fmt == QFMT_Q4_0)
            e = gemv_q_rows<QFMT_Q4_0, kModeTopk>(a, b8, out, n, k, s, di.cus, topk, &lists);
        else
            e = gemv_f16_rows<kModeTopk>(a, b16, out, n, k, s, di.cus, topk, &lists);
        if (e == hipSuccess) e = launch_topk_merge(cand, lists, nullptr, 0, topk, partial, vals, ids, s);
    }
    const hipError_t er = lease.release();
    return e != hipSuccess ? e : er;
}

}  // namespace wq
