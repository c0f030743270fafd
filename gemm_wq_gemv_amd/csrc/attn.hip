// Decode attention for one query token with a split KV cache (grouped-query).
//
// The operation is that of the pages' decode_attention and of its partitioned
// form decode_attention_flash_partial + decode_attention_flash_reduce
// (lattice-inference 0.1.2 metal_qwen35.rs), dispatched by
// dispatch_decode_attention (lattice-inference 0.9.0 dispatch.rs): query head
// h reads KV head h / G, scores s_t = scale * q . k_t over the cache, an
// online softmax, out = sum_t softmax(s)_t v_t.  Caches are token-major
// [len, hkv * d], f32 or f16 (the pages' f16-KV variant).
//
// The pages run one 256-thread threadgroup per KV head (or per KV head and
// 1024-token partition) with one thread per output dimension for P.V and one
// thread per token for Q.K (each thread walking a whole K row).  On CDNA4 the
// work is a stream of K and V rows, so both products keep the rows coalesced:
//  * a lane owns E = d / 64 consecutive dimensions; one K (or V) row of a
//    head is one 64-lane load of 4E (f32) or 2E (f16) bytes per lane;
//  * Q.K for a tile of TT tokens and the GP (padded) query heads of the group
//    leaves TT * GP <= 64 partial dots per lane, reduced across the wave by
//    one butterfly (rows_sum): afterwards each (head, token) score sits in its
//    own lane(s), the TT tokens of a head in one aligned lane group;
//  * the online-softmax update (tile max, rescale, exponentials, tile sum)
//    runs inside that lane group with DPP reductions, on scores kept in log2
//    units (scale * log2(e) folded into the query), so that each weight is
//    one v_exp_f32;
//  * P.V broadcasts each weight with a readlane and accumulates
//    acc[g][e] += p[g][t] * v_t[e] per lane;
//  * a wave's K and V rows for a tile load together, into one of two
//    register buffers, while the previous tile is computed;
//  * the workgroup's 4 waves take the partition's tiles round-robin and merge
//    their (m, l, acc) states through LDS at the end; with more than one
//    partition the states go to scratch and attn_reduce merges them (16 waves
//    per workgroup, 16 partitions loaded at a time per wave).
// Partitions are sized so that about one workgroup per CU exists (>= 32
// tokens each); one partition writes the output directly.
#include "wq_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>

namespace wq {
namespace {

constexpr int kAttnWaves = 4;
std::atomic<int64_t> g_attn_ptok{0};  // forced partition size in tokens; 0 = automatic

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D, int GP, int KVF>
struct AttnShape {
    static constexpr int E = D / kWave;                          // dimensions per lane
    static constexpr int TT = (KVF == 1 && GP <= 4) ? 16 : 8;    // tokens per tile
    static constexpr int N = TT * GP;                            // partial dots per lane per tile (<= 64)
    static constexpr int R = kWave / N;                          // lanes holding each reduced score
    static constexpr int HL = kWave / GP;                        // lanes of one head's scores
    static constexpr int WR = KVF == 0 ? E : (E >= 2 ? E / 2 : 1);  // dwords per lane and row
    static_assert(E >= 1 && N <= kWave, "shape");
};

// This lane's slice of one cache row (E elements at element offset `off`) as
// raw dwords: f32 bits, or f16 pairs (one half, zero-extended, when E == 1).
template <int KVF, int E, int WR>
__device__ __forceinline__ void load_raw(const void *c, int64_t off, uint32_t (&x)[WR]) {
    if constexpr (KVF == 0) {
        const float *p = static_cast<const float *>(c) + off;
        if constexpr (E == 4) {
            const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
            x[0] = t.x, x[1] = t.y, x[2] = t.z, x[3] = t.w;
        } else if constexpr (E == 2) {
            const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
            x[0] = t.x, x[1] = t.y;
        } else {
            x[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
        }
    } else {
        const uint16_t *p = static_cast<const uint16_t *>(c) + off;
        if constexpr (E == 4) {
            const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
            x[0] = t.x, x[1] = t.y;
        } else if constexpr (E == 2) {
            x[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
        } else {
            x[0] = __builtin_nontemporal_load(p);
        }
    }
}

// Element e of a raw row slice as f32 (exact for f16).
template <int KVF>
__device__ __forceinline__ float elem(const uint32_t *x, int e) {
    if constexpr (KVF == 0) return __builtin_bit_cast(float, x[e]);
    return half_bits_to_float((e & 1) ? x[e >> 1] >> 16 : x[e >> 1] & 0xffffu);
}

// 2^x (v_exp_f32).  Scores are kept in log2 units (scaled by scale * log2 e
// once, in the query), so every softmax weight is one exponential.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float lane_value(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// K and V rows of one tile for this lane.  Tokens past the partition end
// re-read its last token (in bounds); their scores are masked.
template <int D, int GP, int KVF>
struct TileBuf {
    using S = AttnShape<D, GP, KVF>;
    uint32_t k[S::TT][S::WR], v[S::TT][S::WR];

    __device__ __forceinline__ void load(const void *kc, const void *vc, int64_t t0, int64_t t_last, int64_t kv_dim,
                                         int64_t col) {
#pragma unroll
        for (int t = 0; t < S::TT; ++t) {
            const int64_t off = std::min<int64_t>(t0 + t, t_last) * kv_dim + col;
            load_raw<KVF, S::E, S::WR>(kc, off, k[t]);
        }
#pragma unroll
        for (int t = 0; t < S::TT; ++t) {
            const int64_t off = std::min<int64_t>(t0 + t, t_last) * kv_dim + col;
            load_raw<KVF, S::E, S::WR>(vc, off, v[t]);
        }
    }
};

// Workgroup (kvh, part) = (blockIdx.x % hkv, blockIdx.x / hkv) covers cache
// tokens [part * ptok, min(len, (part + 1) * ptok)) for the G query heads of
// KV head kvh.  parts == 1: out gets the result; else partials gets
// (m, l, acc[D]) per query head at ((part * hq + h) * (D + 2)), m in log2
// units (the running maximum of scale * log2(e) * q . k).
template <int D, int GP, int KVF>
__global__ __launch_bounds__(kAttnWaves * kWave) void attn_partial(const float *__restrict__ q,
                                                                   const void *__restrict__ kc,
                                                                   const void *__restrict__ vc,
                                                                   float *__restrict__ out,
                                                                   float *__restrict__ partials, int64_t len,
                                                                   int hq, int hkv, int g_real, float scale2,
                                                                   int64_t ptok, int parts) {
    using S = AttnShape<D, GP, KVF>;
    using B = TileBuf<D, GP, KVF>;
    constexpr int E = S::E, TT = S::TT, N = S::N, R = S::R, HL = S::HL;
    __shared__ float sm[kAttnWaves][GP], sl[kAttnWaves][GP];
    __shared__ float sacc[kAttnWaves][GP][D];

    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int kvh = static_cast<int>(blockIdx.x) % hkv, part = static_cast<int>(blockIdx.x) / hkv;
    const int64_t t_begin = static_cast<int64_t>(part) * ptok;
    const int64_t t_end = std::min<int64_t>(len, t_begin + ptok);
    const int64_t kv_dim = static_cast<int64_t>(hkv) * D;
    const int64_t col = static_cast<int64_t>(kvh) * D + lane * E;  // this lane's first element in a row
    const int h0 = kvh * g_real;                                    // first query head of the group

    float qv[GP][E];
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e)
            qv[g][e] = g < g_real ? q[static_cast<int64_t>(h0 + g) * D + lane * E + e] * scale2 : 0.f;

    // Running state (log2 units): m_run / l_run of this lane's head (lane / HL), the same
    // in every lane of that head's group; acc[g][e] for every head.
    float m_run = -__builtin_huge_valf(), l_run = 0.f;
    float acc[GP][E];
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = 0.f;

    const int rt = (lane / R) % TT;  // token (within the tile) of the score this lane holds
    const bool leader = lane % R == 0;
    const int ntiles = static_cast<int>((t_end - t_begin + TT - 1) / TT);

    auto compute = [&](const B &b, int tile) {
        const int64_t t0 = t_begin + static_cast<int64_t>(tile) * TT;
        const int cnt = static_cast<int>(std::min<int64_t>(TT, t_end - t0));
        float pd[N];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float kf[E];
#pragma unroll
            for (int e = 0; e < E; ++e) kf[e] = elem<KVF>(b.k[t], e);
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                float x = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) x = fmaf(qv[g][e], kf[e], x);
                pd[g * TT + t] = x;
            }
        }
        // Cross-lane steps run in every lane; only then are invalid tokens masked.
        const float dot = rows_sum<N, kWave>(pd, lane);
        const bool valid = rt < cnt;
        const float s = valid ? dot : -__builtin_huge_valf();
        const float m_new = fmaxf(m_run, group_max<HL>(s));
        const float alpha = m_run == -__builtin_huge_valf() ? 0.f : ex2(m_run - m_new);
        const float p = valid ? ex2(s - m_new) : 0.f;
        l_run = alpha * l_run + group_sum<HL>(leader ? p : 0.f);
        m_run = m_new;
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            const float a = lane_value(alpha, g * HL);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[g][e] *= a;
        }
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            float vf[E];
#pragma unroll
            for (int e = 0; e < E; ++e) vf[e] = elem<KVF>(b.v[t], e);
            // The token's weights for every head first: a readlane result used
            // by the next instruction costs a wait state.
            float pg[GP];
#pragma unroll
            for (int g = 0; g < GP; ++g) pg[g] = lane_value(p, (g * TT + t) * R);
#pragma unroll
            for (int g = 0; g < GP; ++g)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[g][e] = fmaf(pg[g], vf[e], acc[g][e]);
        }
    };

    // Two register buffers: the next tile's K and V rows load while the
    // current tile is computed.
    B b0, b1;
    const int64_t t_last = t_end - 1;
    auto load = [&](B &b, int tile) {
        b.load(kc, vc, t_begin + static_cast<int64_t>(tile) * TT, t_last, kv_dim, col);
    };
    int tile = w;
    if (tile < ntiles) load(b0, tile);
    for (; tile < ntiles; tile += 2 * kAttnWaves) {
        if (tile + kAttnWaves < ntiles) load(b1, tile + kAttnWaves);
        compute(b0, tile);
        if (tile + kAttnWaves >= ntiles) break;
        if (tile + 2 * kAttnWaves < ntiles) load(b0, tile + 2 * kAttnWaves);
        compute(b1, tile + kAttnWaves);
    }

    // Merge the 4 waves' states.
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        if (lane == g * HL) sm[w][g] = m_run, sl[w][g] = l_run;
#pragma unroll
        for (int e = 0; e < E; ++e) sacc[w][g][lane * E + e] = acc[g][e];
    }
    __syncthreads();
    for (int idx = static_cast<int>(threadIdx.x); idx < g_real * D; idx += kAttnWaves * kWave) {
        const int g = idx / D, d = idx % D;
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int o = 0; o < kAttnWaves; ++o) mx = fmaxf(mx, sm[o][g]);
        float l = 0.f, a = 0.f;
#pragma unroll
        for (int o = 0; o < kAttnWaves; ++o) {
            const float c = sm[o][g] == -__builtin_huge_valf() ? 0.f : ex2(sm[o][g] - mx);
            l = fmaf(c, sl[o][g], l);
            a = fmaf(c, sacc[o][g][d], a);
        }
        const int64_t h = h0 + g;
        if (parts == 1) {
            out[h * D + d] = l > 0.f ? a / l : 0.f;
        } else {
            float *base = partials + (static_cast<int64_t>(part) * hq + h) * (D + 2);
            if (d == 0) base[0] = mx, base[1] = l;
            base[2 + d] = a;
        }
    }
}

constexpr int kReduceWaves = 16;
constexpr int kReduceLoads = 16;  // partitions a wave loads before it merges them

// Workgroup (h, chunk) = (blockIdx.x / (D / 64), blockIdx.x % (D / 64)):
// lane = dimension chunk * 64 + lane of query head h; wave w merges
// partitions w, w + 16, ... with kReduceLoads of them loaded at a time, then
// wave 0 merges the 16 wave states from LDS.  Empty partitions (m = -inf)
// weigh nothing.
template <int D>
__global__ __launch_bounds__(kReduceWaves * kWave) void attn_reduce(const float *__restrict__ partials,
                                                                    float *__restrict__ out, int hq, int parts) {
    constexpr int C = D / kWave;
    __shared__ float sm[kReduceWaves], sl[kReduceWaves], sa[kReduceWaves][kWave];
    const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int h = static_cast<int>(blockIdx.x) / C, d = (static_cast<int>(blockIdx.x) % C) * kWave + lane;
    float m = -__builtin_huge_valf(), l = 0.f, a = 0.f;
    constexpr int U = kReduceLoads;
    for (int p0 = w; p0 < parts; p0 += U * kReduceWaves) {
        float mp[U], lp[U], ap[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int p = p0 + u * kReduceWaves;
            mp[u] = -__builtin_huge_valf(), lp[u] = 0.f, ap[u] = 0.f;
            if (p < parts) {
                const float *base = partials + (static_cast<int64_t>(p) * hq + h) * (D + 2);
                mp[u] = base[0], lp[u] = base[1], ap[u] = base[2 + d];
            }
        }
        // New maximum first, then independent weights (no serial exp chain).
        float mn = m;
#pragma unroll
        for (int u = 0; u < U; ++u) mn = fmaxf(mn, mp[u]);
        if (mn == -__builtin_huge_valf()) continue;  // nothing but empty partitions so far
        const float ca = m == -__builtin_huge_valf() ? 0.f : ex2(m - mn);
        l *= ca;
        a *= ca;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float cp = mp[u] == -__builtin_huge_valf() ? 0.f : ex2(mp[u] - mn);
            l = fmaf(cp, lp[u], l);
            a = fmaf(cp, ap[u], a);
        }
        m = mn;
    }
    if (lane == 0) sm[w] = m, sl[w] = l;
    sa[w][lane] = a;
    __syncthreads();
    if (w != 0) return;
    float mx = -__builtin_huge_valf();
#pragma unroll
    for (int o = 0; o < kReduceWaves; ++o) mx = fmaxf(mx, sm[o]);
    float lt = 0.f, at = 0.f;
#pragma unroll
    for (int o = 0; o < kReduceWaves; ++o) {
        const float c = sm[o] == -__builtin_huge_valf() ? 0.f : ex2(sm[o] - mx);
        lt = fmaf(c, sl[o], lt);
        at = fmaf(c, sa[o][lane], at);
    }
    out[static_cast<int64_t>(h) * D + d] = lt > 0.f ? at / lt : 0.f;
}

template <int D, int GP, int KVF>
hipError_t run_attn(const float *q, const void *k, const void *v, float *out, int64_t len, int hq, int hkv,
                    float scale, hipStream_t s, int cus) {
    // About one workgroup per CU, at least 32 tokens per partition (or the
    // size set through set_attn_partition_override).  Measured on MI355X
    // (head_dim 256, 8 query heads over 2 KV heads, forced sizes 32 .. 1024
    // against the earlier two workgroups per CU and 64 tokens at least): f32
    // caches 14 % faster at 1K tokens, 4-7 % at 4K .. 128K; f16 caches 2-4 %
    // faster at 1K .. 32K, 2-4 % slower at 4K and 128K.
    const int64_t want = std::max<int64_t>(1, (static_cast<int64_t>(cus) + hkv - 1) / hkv);
    int64_t ptok = (len + want - 1) / want;
    ptok = std::max<int64_t>(32, (ptok + 31) / 32 * 32);
    const int64_t forced = g_attn_ptok.load(std::memory_order_relaxed);
    if (forced > 0) ptok = forced;
    const int64_t parts = (len + ptok - 1) / ptok;
    if (parts * hkv > 0x7fffffffLL || parts > 0x7fffffffLL) return hipErrorInvalidValue;
    const int g_real = hq / hkv;
    // Scores in log2 units: scale * log2(e) folded into the query.
    const float scale2 = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
    ScratchLease lease;
    float *partials = nullptr;
    if (parts > 1) {
        void *p = nullptr;
        hipError_t e = lease.acquire(static_cast<size_t>(parts) * hq * (D + 2) * sizeof(float), s, &p);
        if (e != hipSuccess) return e;
        partials = static_cast<float *>(p);
    }
    if (trace_enabled())
        fprintf(stderr, "[wqmm] attn_partial<D=%d,GP=%d,kvf=%d> len=%lld hq=%d hkv=%d ptok=%lld parts=%lld grid=%lld\n",
                D, GP, KVF, (long long)len, hq, hkv, (long long)ptok, (long long)parts, (long long)(parts * hkv));
    hipLaunchKernelGGL((attn_partial<D, GP, KVF>), dim3(static_cast<unsigned>(parts * hkv)),
                       dim3(kAttnWaves * kWave), 0, s, q, k, v, out, partials, len, hq, hkv, g_real, scale2, ptok,
                       static_cast<int>(parts));
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && parts > 1) {
        hipLaunchKernelGGL((attn_reduce<D>), dim3(static_cast<unsigned>(hq * (D / kWave))),
                           dim3(kReduceWaves * kWave), 0, s, partials, out, hq, static_cast<int>(parts));
        e = hipGetLastError();
    }
    const hipError_t er = lease.release();
    return e != hipSuccess ? e : er;
}

template <int D, int KVF>
hipError_t run_group(const float *q, const void *k, const void *v, float *out, int64_t len, int hq, int hkv,
                     float scale, hipStream_t s, int cus) {
    const int g = hq / hkv;
    if (g <= 1) return run_attn<D, 1, KVF>(q, k, v, out, len, hq, hkv, scale, s, cus);
    if (g <= 2) return run_attn<D, 2, KVF>(q, k, v, out, len, hq, hkv, scale, s, cus);
    if (g <= 4) return run_attn<D, 4, KVF>(q, k, v, out, len, hq, hkv, scale, s, cus);
    return run_attn<D, 8, KVF>(q, k, v, out, len, hq, hkv, scale, s, cus);
}

}  // namespace

void set_attn_partition_override(int64_t tokens) { g_attn_ptok.store(tokens, std::memory_order_relaxed); }

hipError_t launch_decode_attention(const float *q, const void *k, const void *v, int kvf, float *out, int64_t len,
                                   int d, int hq, int hkv, float scale, hipStream_t s) {
    if (hkv < 1 || hq < hkv || hq % hkv != 0 || hq / hkv > 8) return hipErrorInvalidValue;
    if (len == 0) return launch_fill_zero(out, static_cast<int64_t>(hq) * d, s);
    DeviceInfo di;
    hipError_t e = device_info(&di);
    if (e != hipSuccess) return e;
    if (d == 64)
        return kvf ? run_group<64, 1>(q, k, v, out, len, hq, hkv, scale, s, di.cus)
                   : run_group<64, 0>(q, k, v, out, len, hq, hkv, scale, s, di.cus);
    if (d == 128)
        return kvf ? run_group<128, 1>(q, k, v, out, len, hq, hkv, scale, s, di.cus)
                   : run_group<128, 0>(q, k, v, out, len, hq, hkv, scale, s, di.cus);
    if (d == 256)
        return kvf ? run_group<256, 1>(q, k, v, out, len, hq, hkv, scale, s, di.cus)
                   : run_group<256, 0>(q, k, v, out, len, hq, hkv, scale, s, di.cus);
    return hipErrorInvalidValue;
}

}  // namespace wq
