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

// Workgroups are dealt round-robin to the 8 XCDs of the chip (workgroup b runs
// on XCD b % 8).  Tile id for workgroup `bid` of `tiles`, such that XCD x
// receives a contiguous range of tile ids (neighbouring tiles share operand
// rows and so hit the same L2).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int bid, int tiles) {
    const int q = tiles / kXcds, r = tiles % kXcds;
    const int x = bid % kXcds, local = bid / kXcds;
    return x < r ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Cross-row exchange of a pair of values on gfx950 (v_permlane16_swap_b32 /
// v_permlane32_swap_b32, one VALU instruction): with H = 16, the odd 16-lane
// rows of a trade places with the even rows of b; with H = 32, the upper 32
// lanes of a with the lower 32 lanes of b.  Afterwards, in every lane,
// x = a and y = b of the lower (bit H clear) side of a lane pair, or of the
// upper side, so x + y is a_l + a_partner(l) in lanes with bit H clear and
// b_partner(l) + b_l in the others: one step of a butterfly over lane xor H
// for two values at once, with no select and no LDS permute.
struct SwapPair {
    float x, y;
};
template <int H>
__device__ __forceinline__ SwapPair lane_swap(float a, float b) {
    static_assert(H == 16 || H == 32, "swap distance");
    const unsigned ua = __builtin_bit_cast(unsigned, a), ub = __builtin_bit_cast(unsigned, b);
    unsigned r0, r1;
    if constexpr (H == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
        r0 = r[0], r1 = r[1];  // elements copied to scalars before any bit cast
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(ua, ub, false, false);
        r0 = r[0], r1 = r[1];
    }
    return SwapPair{__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1)};
}

// Sum over aligned groups of G lanes (G a power of two up to 64); every lane
// of a group receives the group's sum.  Within a 16-lane DPP row:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror;
// across rows: lane xor 16 and 32 (a value swapped with itself).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group size");
    if constexpr (G >= 2) v += dpp_f32<0xb1>(v);
    if constexpr (G >= 4) v += dpp_f32<0x4e>(v);
    if constexpr (G >= 8) v += dpp_f32<0x141>(v);
    if constexpr (G >= 16) v += dpp_f32<0x140>(v);
    if constexpr (G >= 32) {
        const SwapPair p = lane_swap<16>(v, v);
        v = p.x + p.y;
    }
    if constexpr (G >= 64) {
        const SwapPair p = lane_swap<32>(v, v);
        v = p.x + p.y;
    }
    return v;
}

// Maximum over aligned groups of G lanes, every lane of a group receiving it
// (the same lane pairings as group_sum).
template <int G>
__device__ __forceinline__ float group_max(float v) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "group size");
    if constexpr (G >= 2) v = fmaxf(v, dpp_f32<0xb1>(v));
    if constexpr (G >= 4) v = fmaxf(v, dpp_f32<0x4e>(v));
    if constexpr (G >= 8) v = fmaxf(v, dpp_f32<0x141>(v));
    if constexpr (G >= 16) v = fmaxf(v, dpp_f32<0x140>(v));
    if constexpr (G >= 32) {
        const SwapPair p = lane_swap<16>(v, v);
        v = fmaxf(p.x, p.y);
    }
    if constexpr (G >= 64) {
        const SwapPair p = lane_swap<32>(v, v);
        v = fmaxf(p.x, p.y);
    }
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
        float w[N / 2];
        if constexpr (H == 32 || H == 16) {
            // Lanes with bit H clear keep rows 0 .. N/2 - 1, the others the rest.
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                const SwapPair p = lane_swap<H>(v[i], v[N / 2 + i]);
                w[i] = p.x + p.y;
            }
        } else {
            const bool hi = (g & H) != 0;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                const float send = hi ? v[i] : v[N / 2 + i];
                const float keep = hi ? v[N / 2 + i] : v[i];
                w[i] = keep + bit_partner<H>(send);
            }
        }
        return rows_sum<N / 2, H>(w, g);
    }
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// A block starts at an even LDS byte offset pb (rows are whole 16-byte chunks
// and blocks are 34 or 18 bytes long), so it lies in the dword-aligned window
// starting at pb & ~3.  The window is read with aligned 32-bit LDS loads
// (ds_read2_b32), which measured faster on MI355X than 16-byte reads at
// 2-byte aligned addresses; for a block at pb = 2 (mod 4) everything sits two
// bytes higher, and one v_perm_b32 per code dword, with a per-lane selector,
// realigns it.  Returns the scale bits and fills codes[0..NW).
template <int NW>
__device__ __forceinline__ uint32_t block_window(const uint8_t *stage, int pb, uint32_t (&codes)[NW]) {
    const uint32_t *w32 = reinterpret_cast<const uint32_t *>(stage + (pb & ~3));
    uint32_t w[NW + 1];
#pragma unroll
    for (int i = 0; i <= NW; ++i) w[i] = w32[i];
    const bool hi = (pb & 2) != 0;
    // v_perm_b32(x, y, sel): byte b of the result is byte sel.b of the pair
    // (y = bytes 0-3, x = bytes 4-7).  Codes start at window byte 2 (hi: 4).
    const uint32_t sel = hi ? 0x07060504u : 0x05040302u;
#pragma unroll
    for (int i = 0; i < NW; ++i) codes[i] = __builtin_amdgcn_perm(w[i + 1], w[i], sel);
    return hi ? w[0] >> 16 : w[0] & 0xffffu;
}

// SiLU as on the pages' silu_mul kernel: x / (1 + e^-x), in f32.
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// ----------------------------------------------------------------- top-k --
// A (logit, token id) candidate.  Ranking (the pages' TopKCandidate rule): a
// higher value first, equal values by the lower id; NaN values are never
// taken, and empty slots hold the sentinel (-inf, kTopkNoId).
struct TopkCand {
    float v;
    uint32_t id;
};
constexpr int kTopkMax = 64;  // one list entry per lane of a wave
constexpr uint32_t kTopkNoId = 0xffffffffu;

// Branch-free (bitwise) so that it compiles to compares and mask logic.
__device__ __forceinline__ bool cand_better(float av, uint32_t aid, float bv, uint32_t bid) {
    return (av > bv) | ((av == bv) & (aid < bid));
}

// A wave's running top-k list (k <= 64), sorted across lanes: lane r holds
// rank r (lanes >= k hold scratch).  kv / kid: the entry of rank k - 1, the
// bar a new candidate must beat (wave-uniform).
// Value of lane (lane ^ D) for D = 1, 2, 4, 8 (DPP within a row of 16:
// quad permutes and the row / half-row mirrors, xor 15 and xor 7), 16
// (ds_swizzle bit mode within 32 lanes) and 32 (ds_bpermute).
template <int D>
__device__ __forceinline__ int xor_lane(int x) {
    if constexpr (D == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
    if constexpr (D == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
    if constexpr (D == 4)  // row_half_mirror (xor 7), then quad_perm [3,2,1,0] (xor 3)
        return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, false), 0x1B, 0xf, 0xf, false);
    if constexpr (D == 8)  // row_mirror (xor 15), then row_half_mirror (xor 7)
        return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x140, 0xf, 0xf, false), 0x141, 0xf, 0xf, false);
    if constexpr (D == 16) return __builtin_amdgcn_ds_swizzle(x, 0x401f);  // and 0x1f, xor 0x10
    if constexpr (D == 32)
        return __builtin_amdgcn_ds_bpermute(((static_cast<int>(threadIdx.x) & (kWave - 1)) ^ 32) * 4, x);
    return x;
}

struct WaveTopk {
    float v, kv;
    uint32_t id, kid;

    // Compare-exchange with lane ^ D: the lower lane of the pair keeps the
    // better entry when `desc`, the worse otherwise.
    template <int D>
    __device__ __forceinline__ void bitonic_step(int lane, bool desc) {
        const float pv = __builtin_bit_cast(float, xor_lane<D>(__builtin_bit_cast(int, v)));
        const uint32_t pid = static_cast<uint32_t>(xor_lane<D>(static_cast<int>(id)));
        const bool lower = (lane & D) == 0;
        const bool keep_better = lower == desc;
        const bool partner_better = cand_better(pv, pid, v, id);
        const bool take = keep_better == partner_better;
        v = take ? pv : v;
        id = take ? pid : id;
    }

    // One block-size stage of the bitonic sort (blocks of S lanes sorted
    // best first when lane & S == 0, worst first otherwise; S == 64: best first).
    template <int S>
    __device__ __forceinline__ void sort_block(int lane) {
        const bool desc = S == kWave || (lane & S) == 0;
        if constexpr (S >= 64) bitonic_step<32>(lane, desc);
        if constexpr (S >= 32) bitonic_step<16>(lane, desc);
        if constexpr (S >= 16) bitonic_step<8>(lane, desc);
        if constexpr (S >= 8) bitonic_step<4>(lane, desc);
        if constexpr (S >= 4) bitonic_step<2>(lane, desc);
        bitonic_step<1>(lane, desc);
    }

    __device__ __forceinline__ void init() {
        v = kv = -__builtin_huge_valf();
        id = kid = kTopkNoId;
    }

    // Every lane may offer one candidate (pv, pid) (valid, not NaN).  Offers
    // that beat the bar are inserted one at a time, lowest lane first: the
    // insert position is the number of entries that rank before the
    // candidate (a prefix of the lanes), and the entries from there on move
    // up one lane (DPP wave_shr:1, a gfx9 whole-wave shift).  The loop runs
    // once per accepted candidate and is wave-uniform; every cross-lane step
    // is a readlane, a ballot or a DPP move, no LDS permute.
    __device__ __forceinline__ void offer(int k, float pv, uint32_t pid, bool valid) {
        const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
        valid = valid && !__builtin_isnan(pv);
        uint64_t m = __builtin_amdgcn_ballot_w64(valid & cand_better(pv, pid, kv, kid));
        while (m) {
            const int j = static_cast<int>(__builtin_ctzll(m));
            const float cv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), j));
            const uint32_t cid = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(pid), j));
            const int pos =
                static_cast<int>(__builtin_popcountll(__builtin_amdgcn_ballot_w64((lane < k) & cand_better(v, id, cv, cid))));
            const int uv = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x138, 0xf, 0xf, false);
            const int uid = __builtin_amdgcn_update_dpp(0, static_cast<int>(id), 0x138, 0xf, 0xf, false);
            v = lane == pos ? cv : lane > pos ? __builtin_bit_cast(float, uv) : v;
            id = lane == pos ? cid : lane > pos ? static_cast<uint32_t>(uid) : id;
            kv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), k - 1));
            kid = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(id), k - 1));
            valid &= lane != j;
            m = __builtin_amdgcn_ballot_w64(valid & cand_better(pv, pid, kv, kid));
        }
    }

    // Merge of a list (bv, bid) sorted across the 64 lanes (best first,
    // sentinels last) into this one: the top 64 of the union are
    // better(mine[i], theirs[63 - i]) lane by lane, a bitonic sequence, which
    // a 6-step bitonic merge sorts.  Entries of rank >= k are dropped first.
    __device__ __forceinline__ void merge_sorted(int k, float bv, uint32_t bid) {
        const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
        // Both branches produce values and the four fields are assigned once
        // afterwards: assigning them inside the branches let the compiler merge
        // the stores through a selected pointer and keep the list in scratch.
        float nv, nkv;
        uint32_t nid, nkid;
        if (k == 1) {  // the better of the two first entries
            const float fv = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, bv)));
            const uint32_t fid = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bid)));
            const bool take = cand_better(fv, fid, kv, kid);
            nkv = take ? fv : kv;
            nkid = take ? fid : kid;
            nv = nkv;
            nid = nkid;
        } else {
            WaveTopk m;
            m.v = lane >= k ? -__builtin_huge_valf() : v;
            m.id = lane >= k ? kTopkNoId : id;
            const int rev = (kWave - 1 - lane) * 4;
            const float rv = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(rev, __builtin_bit_cast(int, bv)));
            const uint32_t rid = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(rev, static_cast<int>(bid)));
            const bool take = cand_better(rv, rid, m.v, m.id);
            m.v = take ? rv : m.v;
            m.id = take ? rid : m.id;
            m.bitonic_step<32>(lane, true);
            m.bitonic_step<16>(lane, true);
            m.bitonic_step<8>(lane, true);
            m.bitonic_step<4>(lane, true);
            m.bitonic_step<2>(lane, true);
            m.bitonic_step<1>(lane, true);
            nv = m.v;
            nid = m.id;
            nkv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m.v), k - 1));
            nkid = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(m.id), k - 1));
        }
        v = nv;
        id = nid;
        kv = nkv;
        kid = nkid;
    }

    // The best of the 64 lanes' (v, id) in every lane (xor butterfly).
    __device__ __forceinline__ void best_all() {
        best_step<32>();
        best_step<16>();
        best_step<8>();
        best_step<4>();
        best_step<2>();
        best_step<1>();
    }
    template <int D>
    __device__ __forceinline__ void best_step() {
        const float pv = __builtin_bit_cast(float, xor_lane<D>(__builtin_bit_cast(int, v)));
        const uint32_t pid = static_cast<uint32_t>(xor_lane<D>(static_cast<int>(id)));
        const bool take = cand_better(pv, pid, v, id);
        v = take ? pv : v;
        id = take ? pid : id;
    }

    // Sorts the 64 lanes' (v, id) best first (a full bitonic sort).
    __device__ __forceinline__ void sort64() {
        const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
        sort_block<2>(lane);
        sort_block<4>(lane);
        sort_block<8>(lane);
        sort_block<16>(lane);
        sort_block<32>(lane);
        sort_block<64>(lane);
    }

    // Entries of rank < k as they stand (lane r writes rank r).
    __device__ __forceinline__ void store(TopkCand *out, int k) const {
        const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
        if (lane < k) out[lane] = TopkCand{v, id};
    }
};

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
// m (2 .. 4) rows of A [m, k] against Q8_0 (fmt 1) or Q4_0 (fmt 2) weights in
// one register-chunk GEMV launch, c [m, n], epilogue kEpiNone or kEpiResidual.
// Returns false (nothing launched) when no compiled plan takes the call
// (Q4_0 beyond 2 rows, K % 256 != 0, misaligned operands, ...); *e gets the
// launch status otherwise.
bool launch_gemv_q_rows(const float *a, const uint8_t *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                        hipStream_t s, int epi, hipError_t *e);
// Whether the automatic route gives the call to launch_gemv_q_rows rather than
// the weight stream: two Q8_0 rows of A under a plan of at most three units
// per wave (the case measured faster).
bool gemv_q_rows_auto(const float *a, const uint8_t *b, int fmt, int64_t m, int64_t n, int64_t k, int epi);
// Top-k of the LM-head logits w . a (w [n, k] in format fmt, one token):
// the GEMV keeps a top-k list per wave, then launch_topk_merge reduces the
// lists.  vals / ids: topk entries in rank order (1 <= topk <= kTopkMax).
// workspace: nullptr (scratch from the per-stream cache) or a device buffer of
// at least lm_head_topk_scratch_bytes(...) bytes that the call uses instead.
hipError_t launch_lm_head_topk(const float *a, const void *b, int fmt, int64_t n, int64_t k, int topk,
                               float *vals, uint32_t *ids, hipStream_t s, void *workspace = nullptr,
                               size_t workspace_bytes = 0);
// The fixed workspace of the allocation-free entry point (wqmm_api.hip): its
// size, and its device address on the current device.
constexpr size_t kNoAllocBytes = size_t(4) << 20;
hipError_t noalloc_workspace(void **ptr);
// Scratch bytes launch_lm_head_topk needs for these arguments on `cus` CUs.
size_t lm_head_topk_scratch_bytes(const float *a, const void *b, int fmt, int64_t n, int64_t k, int topk, int cus);
// Merge of candidate lists into the final top-k.  Lists are either `lists`
// arrays of topk TopkCand (cand) or, with cand == nullptr, a logits vector
// of n values cut into lists of 64 consecutive ids.  Two kernels: up to
// kTopkGroups workgroups each reduce a share of the lists into `partial`
// (kTopkGroups * topk entries), then one workgroup reduces those.
constexpr int kTopkGroups = 256;
hipError_t launch_topk_merge(const TopkCand *cand, int64_t lists, const float *logits, int64_t n, int topk,
                             TopkCand *partial, float *vals, uint32_t *ids, hipStream_t s);

// Decode attention for one query token (q [hq, d], K/V caches [len, hkv * d]
// in f32 (kvf 0) or f16 (kvf 1), out [hq, d]); d in {64, 128, 256}, hq / hkv
// in 1..8.  Split over the cache in partitions, then a merge pass.
hipError_t launch_decode_attention(const float *q, const void *k, const void *v, int kvf, float *out, int64_t len,
                                   int d, int hq, int hkv, float scale, hipStream_t s);
// Partition size (tokens) every later attention call uses; 0 = automatic.
void set_attn_partition_override(int64_t tokens);

// n = output columns; with kEpiGlu the weights have 2n rows.
hipError_t launch_gemm(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n,
                       int64_t k, hipStream_t s, int epi = kEpiNone);
// Product through the f16 matrix cores with A split into hi / lo f16 halves
// (hgemm_ok: K % 32 == 0, 16-byte aligned a and b, quantized weights under
// 2 GiB); n = output columns (2n
// weight rows with kEpiGlu).  Uses the stream's scratch for the split A.
// nw: weight rows (2n with kEpiGlu).
bool hgemm_ok(const float *a, const void *b, int fmt, int64_t m, int64_t nw, int64_t k);
hipError_t launch_hgemm(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                        hipStream_t s, int epi = kEpiNone);
// Tile shape and K splits of that product; test hook forcing them ((0, 0, 0)
// clears; false for a tile that is not compiled in).
void hgemm_plan(int64_t m, int64_t n, int64_t k, int fmt, int cus, int *bm, int *bn, int *splits);
bool set_hgemm_plan_override(int bm, int bn, int splits);
// Small-M product for Q8_0 / Q4_0 weights with K % 256 == 0 and 16-byte
// aligned a and b (smallm_ok), 1 <= M <= 16; n = output columns (2n weight
// rows with kEpiGlu).
bool smallm_ok(const float *a, const void *b, int fmt, int64_t m, int64_t k);
hipError_t launch_smallm(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                         hipStream_t s, int epi = kEpiNone);
// Weight stream through the f16 matrix cores for Q8_0 / Q4_0 weights,
// 1 <= M <= 16, K % 256 == 0, 16-byte aligned a and b (wstream_ok); epi
// kEpiNone or kEpiResidual.
bool wstream_ok(const float *a, const void *b, int fmt, int64_t m, int64_t n, int64_t k);
hipError_t launch_wstream(const float *a, const void *b, int fmt, float *c, int64_t m, int64_t n, int64_t k,
                          hipStream_t s, int epi = kEpiNone);
// Test hook: workgroup shape 1..7 and K splits; 0 = automatic.
bool set_wstream_plan_override(int shape, int splits);
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
// Forces the register-chunk Q8_0 GEMV plan (rb, nf, nr); (0, 0, 0) automatic,
// (-1, 0, 0) off.  False for a plan that is not instantiated.
bool set_gemv_plan_override(int rb, int nf, int nr);
hipError_t launch_fill_zero(float *c, int64_t count, hipStream_t s);
// Read-bandwidth probe (variant v: 2^v 16-byte chunks per lane); out gets one
// dword per wave.
hipError_t launch_read_probe(const void *p, int64_t bytes, uint32_t *out, int variant, hipStream_t s);
hipError_t launch_pack_f16(const float *w, uint16_t *out, int64_t count, hipStream_t s);
hipError_t launch_quantize_q8_0(const float *w, uint8_t *out, int64_t count, hipStream_t s);

// Scratch for split-K partial sums and the like.  One buffer per (device,
// stream), grown on demand from the device's default memory pool
// (stream-ordered) and kept for reuse: uses on one stream are ordered by the
// stream, uses on different streams never share a buffer.  A lease holds the
// device's lock from acquire() until the kernels that use the buffer are
// enqueued.  Requests above kScratchCacheBytes, and streams beyond the first
// eight seen on a device, take a private stream-ordered allocation.
constexpr size_t kScratchCacheBytes = size_t(256) << 20;
constexpr int kStreamSlots = 8;  // streams per device with a cached scratch buffer
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
    // Index (0 .. kStreamSlots - 1) of the per-stream cache slot the lease
    // holds, the same for every lease on this stream; -1 for a private
    // allocation (a stream beyond the cached ones, or a large request).
    int slot() const { return slot_; }

  private:
    int slot_ = -1;
    int dev_ = -1;
    hipStream_t s_ = nullptr;
    void *priv_ = nullptr;  // private allocation (large requests)
    bool held_ = false;     // device lock held
};

// Set by WQ_TRACE=1: one line per launch on stderr.
bool trace_enabled();

}  // namespace wq
