// Top-k merge: candidate lists (or a logits vector) -> the final top-k.
//
// The selection is the one of the pages' lm_head two-stage block top-k
// (dispatch_lm_head_block_stage1_enc / dispatch_block_topk_merge_enc,
// lattice-inference 0.9.0 dispatch.rs) and of the k = 1 argmax and k = 50
// tournament kernels (logits_argmax_first / _merge, logits_topk_select50_first
// / _merge, lattice-inference 0.1.2 metal_qwen35.rs): exact top-k under the
// TopKCandidate ranking.  Those use 32-lane SIMD-group argmax rounds repeated
// k times and fan-in-16 merge passes; here a 64-lane wave keeps a sorted list
// with one entry per lane (WaveTopk).  A batch of 64 candidates that cannot
// beat the list's k-th entry costs one compare (a whole sorted list is judged
// by its first entry); otherwise it is merged with one 64-lane bitonic merge
// (DPP and swizzle compare-exchanges), after a bitonic sort if it came
// unsorted (raw logits).  Each wave keeps kBatch list loads in flight.
//
// One or two launches, no atomics: a workgroup (16 waves, then a pairwise LDS
// merge tree of their 16 lists) folds a share of the batches into one list.
// Up to 128 batches take one workgroup that writes the result; more take up
// to kTopkGroups workgroups writing partial lists and one more over those.
#include "wq_internal.h"

#include <algorithm>

namespace wq {
namespace {

constexpr int kMergeWaves = 16;  // waves per merge workgroup
constexpr int kBatch = 8;        // lists a wave loads before it merges them

// Where a batch of 64 candidates comes from.
enum { kSrcSorted = 0, kSrcFlat = 1, kSrcLogits = 2 };

// Batch l as 64 lanes.  kSrcSorted: candidate list l, sorted, topk entries
// (lanes >= topk get the sentinel); kSrcFlat: candidates 64 l .. 64 l + 63 of
// an array of n single entries (lists of one); kSrcLogits: ids 64 l ..
// 64 l + 63 of a logits vector, NaN as the sentinel.  Ids past n: sentinel.
// Every lane loads from an in-bounds index (clamped) and the sentinel is
// selected by value afterwards: selecting between a load and a local sentinel
// object made the compiler keep the sentinel on the stack and issue generic
// (flat) loads through a selected pointer.
template <int SRC>
__device__ __forceinline__ TopkCand load_batch(const TopkCand *cand, const float *logits, int64_t n, int topk,
                                               int64_t l) {
    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    const float ninf = -__builtin_huge_valf();
    if constexpr (SRC == kSrcSorted) {
        const bool in = lane < topk;
        const TopkCand x = cand[l * topk + (in ? lane : 0)];
        return TopkCand{in ? x.v : ninf, in ? x.id : kTopkNoId};
    }
    const int64_t i = l * kWave + lane;
    const bool in = i < n;
    const int64_t j = in ? i : n - 1;  // n >= 1 whenever a batch exists
    if constexpr (SRC == kSrcFlat) {
        const TopkCand x = cand[j];
        return TopkCand{in ? x.v : ninf, in ? x.id : kTopkNoId};
    }
    const float x = logits[j];
    const bool ok = in && !__builtin_isnan(x);
    return TopkCand{ok ? x : ninf, ok ? static_cast<uint32_t>(i) : kTopkNoId};
}

// Folds one batch into the wave's list.  A sorted list whose best entry does
// not beat the bar is skipped whole; an unsorted batch is skipped when no lane
// beats it, else sorted first (for k = 1 only its best is found).  Then one
// bitonic merge (for k = 1, one compare).
__device__ __forceinline__ void fold_batch(WaveTopk &t, int topk, TopkCand c, bool sorted) {
    if (sorted) {
        const float bv = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, c.v)));
        const uint32_t bid = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(c.id)));
        if (!cand_better(bv, bid, t.kv, t.kid)) return;
    } else {
        if (__builtin_amdgcn_ballot_w64(cand_better(c.v, c.id, t.kv, t.kid)) == 0) return;
        WaveTopk b;
        b.v = c.v;
        b.id = c.id;
        if (topk == 1)
            b.best_all();
        else
            b.sort64();
        c.v = b.v;
        c.id = b.id;
    }
    t.merge_sorted(topk, c.v, c.id);
}

// Batches first, first + step, ... below end, kBatch loads in flight at a time.
template <int SRC>
__device__ __forceinline__ void fold_batches(WaveTopk &t, int topk, const TopkCand *cand, const float *logits,
                                             int64_t n, int64_t first, int64_t end, int64_t step) {
    for (int64_t l = first; l < end; l += kBatch * step) {
        TopkCand c[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int64_t lq = l + q * step;
            c[q] = lq < end ? load_batch<SRC>(cand, logits, n, topk, lq)
                            : TopkCand{-__builtin_huge_valf(), kTopkNoId};
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
            if (l + q * step < end) fold_batch(t, topk, c[q], SRC == kSrcSorted);
    }
}

// The workgroup's wave lists folded into wave 0's list by a pairwise tree
// through LDS: at level h, wave w (w % 2h == 0) merges the list of wave w + h.
__device__ __forceinline__ void fold_waves(WaveTopk &t, int topk, TopkCand (*lds)[kWave]) {
    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1), w = static_cast<int>(threadIdx.x) / kWave;
#pragma unroll
    for (int h = 1; h < kMergeWaves; h *= 2) {
        if (w % (2 * h) == h) {
            const bool in = lane < topk;
            lds[w][lane] = TopkCand{in ? t.v : -__builtin_huge_valf(), in ? t.id : kTopkNoId};
        }
        __syncthreads();
        if (w % (2 * h) == 0) fold_batch(t, topk, lds[w + h][lane], true);
    }
}

// Workgroup g folds batches [g * per, min(batches, (g + 1) * per)) into one
// list: written to partial[g] (topk entries), or, when vals is given (a grid
// of one workgroup), to vals / ids as the result.
template <int SRC>
__global__ __launch_bounds__(kMergeWaves * kWave) void topk_reduce(const TopkCand *__restrict__ cand,
                                                                   const float *__restrict__ logits, int64_t n,
                                                                   int64_t batches, int64_t per, int topk,
                                                                   TopkCand *__restrict__ partial,
                                                                   float *__restrict__ vals,
                                                                   uint32_t *__restrict__ ids) {
    __shared__ TopkCand lds[kMergeWaves][kWave];
    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1), w = static_cast<int>(threadIdx.x) / kWave;
    WaveTopk t;
    t.init();
    const int64_t l0 = static_cast<int64_t>(blockIdx.x) * per, l1 = std::min<int64_t>(batches, l0 + per);
    fold_batches<SRC>(t, topk, cand, logits, n, l0 + w, l1, kMergeWaves);
    fold_waves(t, topk, lds);
    if (w != 0) return;
    if (vals) {
        if (lane < topk) vals[lane] = t.v, ids[lane] = t.id;
    } else {
        t.store(partial + static_cast<int64_t>(blockIdx.x) * topk, topk);
    }
}

template <int SRC>
hipError_t launch_reduce(const TopkCand *cand, const float *logits, int64_t n, int64_t batches, int64_t per,
                         int64_t grid, int topk, TopkCand *partial, float *vals, uint32_t *ids, hipStream_t s) {
    hipLaunchKernelGGL((topk_reduce<SRC>), dim3(static_cast<unsigned>(grid)), dim3(kMergeWaves * kWave), 0, s, cand,
                       logits, n, batches, per, topk, partial, vals, ids);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_topk_merge(const TopkCand *cand, int64_t lists, const float *logits, int64_t n, int topk,
                             TopkCand *partial, float *vals, uint32_t *ids, hipStream_t s) {
    if (topk < 1 || topk > kTopkMax) return hipErrorInvalidValue;
    // Sources: sorted lists; for k = 1 the lists are single entries, read flat
    // 64 at a time; or a logits vector, 64 ids at a time.
    const int src = !cand ? kSrcLogits : topk == 1 ? kSrcFlat : kSrcSorted;
    const int64_t count = src == kSrcSorted ? lists : src == kSrcFlat ? lists : n;  // entries of the flat sources
    const int64_t batches = src == kSrcSorted ? lists : (count + kWave - 1) / kWave;
    auto first = [&](int64_t per, int64_t grid, float *v, uint32_t *i) {
        if (src == kSrcSorted) return launch_reduce<kSrcSorted>(cand, logits, count, batches, per, grid, topk, partial, v, i, s);
        if (src == kSrcFlat) return launch_reduce<kSrcFlat>(cand, logits, count, batches, per, grid, topk, partial, v, i, s);
        return launch_reduce<kSrcLogits>(cand, logits, count, batches, per, grid, topk, partial, v, i, s);
    };
    // Few batches: one workgroup writes the result directly.
    if (batches <= static_cast<int64_t>(kMergeWaves) * kBatch) {
        if (trace_enabled())
            fprintf(stderr, "[wqmm] topk_reduce<src=%d> batches=%lld topk=%d grid=1 (final)\n", src,
                    (long long)batches, topk);
        return first(std::max<int64_t>(batches, 1), 1, vals, ids);
    }
    // About one batch per wave, at most kTopkGroups partial lists, then one
    // workgroup over those (flat for k = 1: single entries).  The first pass
    // is bound by the instruction rate of the CUs it occupies (a batch that
    // beats a wave's bar costs a 64-lane sort and merge), so it spreads the
    // batches over as many CUs as there are groups of 16: measured at
    // n = 151936, k = 50, 4 batches per wave on 38 CUs took 12.5 us.
    const int64_t want = (batches + kMergeWaves - 1) / kMergeWaves;
    const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(kTopkGroups, want));
    const int64_t per = (batches + groups - 1) / groups;
    const int64_t used = (batches + per - 1) / per;  // no empty workgroup
    if (trace_enabled())
        fprintf(stderr, "[wqmm] topk_reduce<src=%d> batches=%lld topk=%d grid=%lld per=%lld; then final\n", src,
                (long long)batches, topk, (long long)used, (long long)per);
    hipError_t e = first(per, used, nullptr, nullptr);
    if (e != hipSuccess) return e;
    if (topk == 1)
        return launch_reduce<kSrcFlat>(partial, nullptr, used, (used + kWave - 1) / kWave,
                                       std::max<int64_t>((used + kWave - 1) / kWave, 1), 1, topk, nullptr, vals, ids, s);
    return launch_reduce<kSrcSorted>(partial, nullptr, used, used, used, 1, topk, nullptr, vals, ids, s);
}

}  // namespace wq
