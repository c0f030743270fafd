/*
 * wqmm.h -- C ABI of libwqmm, the mixed-precision weight matmul for AMD
 * Instinct MI355X (gfx950):
 *
 *     C[M,N] = A[M,K] . B[N,K]^T          (C is overwritten, beta = 0)
 *
 * Source of the operation: lattice-inference 0.9.0,
 * forward/metal_qwen35/inner/dispatch.rs -- dispatch_matmul_half (doc
 * comment: C[M,N] = A[M,K] @ B_half[N,K]^T, A f32 activations, B f16 weights
 * widened to f32 before accumulation, C f32), dispatch_matmul_q8 (Q8_0
 * weights [N, K/32 * 34]) and dispatch_gemm_q8 (M == 1 takes the decode
 * GEMV, M > 1 the tiled GEMM; m == 0 or n == 0 is a no-op; K must be a
 * non-zero multiple of 32).  Formats: lattice-inference 0.1.2,
 * forward/metal_qwen35.rs -- kernel gemv_q8_decode (block = f16 scale, then
 * 32 int8), quantize_row_q8_0, f32_to_f16; kernels gemv_q4_decode, gemm_q4
 * and gemm_q4_tiled (Q4_0 block = f16 scale, then 16 bytes of 4-bit codes;
 * dispatch_gemm_q4 on the 0.9.0 page routes M as for Q8_0).  The same product as
 * sgemm(RowMajor, NoTrans, Trans, alpha = 1, beta = 0): ferrum-kernels
 * 0.7.7, attention/metal/pipelines.rs, MetalPipelines::gemm.
 *
 * Layouts (all row-major, tightly packed, no stride arguments):
 *   a  f32 [M, K]                         lda = K
 *   b  f16 bit patterns [N, K]            2*N*K bytes
 *      or Q8_0 bytes [N, K/32 * 34]       row n starts at byte n*(K/32)*34;
 *         block j of the row at +34*j: bytes 0..1 a little-endian f16 scale d,
 *         bytes 2..33 int8 codes q; weight (n, 32*j + i) = d * q[i]
 *      or Q4_0 bytes [N, K/32 * 18]       row n starts at byte n*(K/32)*18;
 *         block j at +18*j: bytes 0..1 the little-endian f16 scale d, byte
 *         2 + i holds code u of weight 2i (low nibble) and of weight 2i + 1
 *         (high nibble); weight = (u - 8) * d
 *   c  f32 [M, N]                         ldc = N
 * Accumulation is in f32; the summation order is unspecified, so results may
 * differ from a serial f32 sum by rounding only.  The weight decode itself is
 * exact (f16 -> f32 widening; d * q and (u - 8) * d are exact in f32).
 *
 * Pointers: a, b, c (and w, out of the packing calls) are DEVICE pointers on
 * the current HIP device.  The caller owns all memory; the library never
 * allocates, frees or keeps caller buffers.  Buffers must stay alive until the
 * enqueued work has run.  A GEMM that splits K takes a scratch buffer of
 * splits*M*N*4 bytes (the other users of scratch say so below) from the
 * device's default memory pool, stream-ordered on the call's stream
 * (hipMallocAsync / hipFreeAsync); wq_gemm_plan tells when.  The library keeps
 * one such buffer per stream it has seen (up to 256 MiB each, for the first
 * eight streams of a device) and reuses it on that stream without further
 * synchronisation; a stream must therefore have finished its libwqmm work
 * before it is destroyed.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  Every call only enqueues work and returns without synchronising;
 * c is written when the stream runs.  Calls are reentrant and thread-safe.
 *
 * Errors: every call validates all arguments before it enqueues anything.
 * On any error nothing is launched and c is not touched.  Alignment: a and c
 * must be 4-byte aligned, b 2-byte aligned.  c must not overlap a or b.
 * m == 0 or n == 0 returns WQ_OK without touching any pointer.  For f16,
 * K == 0 is allowed and writes zeros to c (the empty sum); a and b may then be
 * NULL.  Q8_0 and Q4_0 need K > 0 and K % 32 == 0.
 */
#ifndef WQMM_H
#define WQMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight storage formats (the pages' QuantFormat plus their f16 weights). */
typedef enum wq_format {
    WQ_FMT_F16 = 0,  /* IEEE-754 binary16 bit patterns */
    WQ_FMT_Q8_0 = 1, /* 34-byte Q8_0 blocks of 32 weights */
    WQ_FMT_Q4_0 = 2  /* 18-byte Q4_0 blocks of 32 weights */
} wq_format;

/* Status codes returned by every entry point. */
typedef enum wq_status {
    WQ_OK = 0,
    WQ_ERR_NULL = 1,    /* a required pointer is NULL */
    WQ_ERR_SHAPE = 2,   /* negative dimension, or a byte count overflows int64 */
    WQ_ERR_K = 3,       /* Q8_0 / Q4_0 with K == 0 or K % 32 != 0 */
    WQ_ERR_FORMAT = 4,  /* fmt is not a wq_format */
    WQ_ERR_ALIGN = 5,   /* a or c not 4-byte aligned, or b not 2-byte aligned */
    WQ_ERR_LAUNCH = 6,  /* the HIP runtime failed to enqueue a kernel or scratch */
    WQ_ERR_ALIAS = 7,   /* c overlaps a or b */
    WQ_ERR_ROUTE = 8,   /* not a wq_route value */
    WQ_ERR_EPILOGUE = 9, /* not a wq_epilogue value */
    WQ_ERR_TOPK = 10,    /* top-k count outside 1 .. WQ_TOPK_MAX */
    WQ_ERR_WORKSPACE = 11 /* needs more scratch than the fixed no-allocation workspace */
} wq_status;

/* Kernel families wq_matmul can route to. */
typedef enum wq_route {
    WQ_ROUTE_AUTO = 0,  /* choose by M (wq_route_for) */
    WQ_ROUTE_GEMV = 1,  /* decode GEMV: one launch per row of A, except 2 to 4
                           Q8_0 rows (2 Q4_0 rows) with K % 256 == 0 and
                           16-byte aligned a and b, which the register-chunk
                           kernel takes in one launch (each weight chunk read
                           once and applied to every row) */
    WQ_ROUTE_GEMM = 2,  /* LDS-tiled fp32-MFMA GEMM */
    WQ_ROUTE_SKINNY = 3, /* small-M weight-streaming fp32-MFMA product: one
                            launch per block of up to 16 rows of A */
    WQ_ROUTE_STREAM = 4, /* small-M weight stream through the f16 matrix cores
                            with f32 results (Q8_0 / Q4_0, K % 256 == 0,
                            M * K <= 196608 per block of rows, 16-byte aligned
                            a and b, no SwiGLU; other calls on this route take
                            WQ_ROUTE_SKINNY): one launch per block of up to 16
                            rows of A */
    WQ_ROUTE_GEMM_HL = 5 /* LDS-tiled GEMM on the f16 matrix cores with f32
                            results: each row of A is scaled by a power of two
                            and split into hi + lo f16 halves (22 significant
                            bits), weights are exact in f16, products exact in
                            f32 and summed in f32 (K % 32 == 0, 16-byte aligned
                            a and b; other calls on this route take
                            WQ_ROUTE_GEMM).  Scratch: M * K * 4 bytes for the
                            split A, plus the split-K partial sums */
} wq_route;

/* ---------------------------------------------------------------------- */
/* Decode GEMV, M = 1: c[n] = sum_k a[k] * w[n, k].  a is f32 [K], c f32 [N].
 * The weights stream from HBM once; a is held on chip.  Passage: kernel
 * gemv_decode_m1 (f16), gemv_q8_decode (Q8_0) and gemv_q4_decode (Q4_0),
 * lattice-inference 0.1.2 metal_qwen35.rs; dispatch_matmul_half /
 * dispatch_matmul_q8 / dispatch_matmul_q4, lattice-inference 0.9.0
 * dispatch.rs.  There is no m argument: a GEMV computes one row. */
int wq_gemv_f16(const float *a, const uint16_t *b, float *c, int64_t n, int64_t k, void *stream);
int wq_gemv_q8_0(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, void *stream);
int wq_gemv_q4_0(const float *a, const uint8_t *b, float *c, int64_t n, int64_t k, void *stream);

/* Prefill GEMM, any M >= 1: C = A . B^T through LDS tiles of A and of the
 * dequantised B, with fp32 matrix-core (MFMA) accumulation.  Passage: kernels
 * matmul_bt, gemm_q8 and gemm_q4_tiled (tiling prior art), lattice-inference
 * 0.1.2 metal_qwen35.rs; dispatch_gemm_q8, lattice-inference 0.9.0 dispatch.rs. */
int wq_gemm_f16(const float *a, const uint16_t *b, float *c, int64_t m, int64_t n, int64_t k,
                void *stream);
int wq_gemm_q8_0(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k,
                 void *stream);
int wq_gemm_q4_0(const float *a, const uint8_t *b, float *c, int64_t m, int64_t n, int64_t k,
                 void *stream);

/* M-routed product for either format (fmt is a wq_format).  M == 1 takes the
 * GEMV.  Q8_0 / Q4_0 with K % 256 == 0 take, for 2 <= M <= 16, the f16
 * matrix-core weight stream (activations carried as two f16 parts, hi + lo,
 * after a power-of-two scaling per row and K range, so the product keeps f32
 * accuracy; f32 accumulation); other quantized shapes the fp32 small-M kernel
 * up to M == 4, f16 weights up to M == 8; larger M the tiled GEMM on the f16
 * matrix cores (WQ_ROUTE_GEMM_HL, A split the same way per row), unless a
 * route is forced (wq_set_forced_route).  The small-M kernels read every weight
 * once per 16 rows of A; when they split K (and for the SwiGLU epilogue on the
 * fp32 small-M kernel) they use the same scratch as the GEMM (splits*M*N*4
 * bytes, 2n columns for SwiGLU).  Passage: dispatch_gemm_q8 and dispatch_gemm,
 * lattice-inference 0.9.0 dispatch.rs (M == 1 decode, M > 1 batched
 * product). */
int wq_matmul(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt,
              void *stream);

/* Epilogues fused into the product (wq_matmul_ex). */
typedef enum wq_epilogue {
    WQ_EPI_NONE = 0,     /* c = a . b^T, as wq_matmul */
    WQ_EPI_RESIDUAL = 1, /* c += a . b^T: c holds the residual stream on entry */
    WQ_EPI_SWIGLU = 2    /* b has 2n rows, gate rows 0..n-1 then up rows n..2n-1;
                            c = silu(a . gate^T) * (a . up^T), silu(x) = x / (1 + e^-x) */
} wq_epilogue;

/* wq_matmul with an epilogue applied to each output before it is stored, so
 * that the extra pass over C (or over a [M, 2n] gate||up buffer) that the
 * pages spend on a separate element-wise kernel is not needed.
 *
 * WQ_EPI_RESIDUAL -- c[i,j] = c[i,j] + sum_k a[i,k] w[j,k].  Passage:
 *   encode_layer_prefill on the oxibonsai-kernels 0.1.4 page,
 *   gpu_backend/metal_prefill/functions.rs, which adds the attention output
 *   and down projections into the hidden state inside the GEMM
 *   (gemm_q1_v7_residual), and whose ternary twin spells the same step as a
 *   GEMM plus residual_add; add_buf on the lattice-inference 0.1.2 page.
 *   The residual is read from c itself (in place, as those calls do).
 * WQ_EPI_SWIGLU -- b is the fused gate||up weight, [2n, K] in the format's
 *   layout (gate rows first, then up rows; the up half starts at row n, byte
 *   n * row_bytes), and c is [m, n]:
 *   c[i,j] = silu(g) * u, g = sum_k a[i,k] gate[j,k], u = sum_k a[i,k] up[j,k].
 *   Passage: same page, fused_gate_up_swiglu_gemm, and the ternary twin's
 *   GEMM over n_rows = 2 * inter followed by batched_swiglu;
 *   dispatch_silu_mul_fused on the lattice-inference 0.9.0 page (first half
 *   of a gate||up buffer = silu(first half) * second half) and kernel
 *   silu_mul on the 0.1.2 page (silu(g) = g / (1 + exp(-g)), times up).
 *   Tiled-GEMM and small-M routes apply the epilogue in the kernel when K is
 *   not split, else in the pass that sums the splits; the M == 1 route runs
 *   the GEMV over all 2n rows into scratch (2*M*n*4 bytes, stream-ordered as
 *   for split-K) and then one element-wise pass.
 * Sub-matrices of fused weight buffers (gate or up alone, q||k||v) need no
 * offset argument: pass b advanced by whole rows (row r starts at byte
 * r * row_bytes, always 2-byte aligned).
 * Routing and K rules are those of wq_matmul.  K == 0 (f16): NONE writes
 * zeros, RESIDUAL leaves c as it is, SWIGLU writes silu(0) * 0 = 0.
 * Returns WQ_ERR_EPILOGUE for an unknown epi (before any other check);
 * otherwise as wq_matmul, with the weight bounds (overlap, size) taken over
 * the 2n rows for SWIGLU. */
int wq_matmul_ex(const float *a, const void *b, float *c, int64_t m, int64_t n, int64_t k, int fmt,
                 int epi, void *stream);

/* ---------------------------------------------------------------------- */
/* LM-head top-k (greedy and top-k sampling front end).
 *
 * Candidates are (logit, token id) pairs ranked as the pages' TopKCandidate
 * (topk_better, lattice-inference 0.1.2 metal_qwen35.rs): a higher logit
 * first, equal logits by the lower id; a NaN logit is never selected.  The
 * result is the exact top-k under that ranking of the f32 logits the kernels
 * compute, written in rank order to vals[0..topk-1] (f32) and ids[0..topk-1]
 * (u32); when fewer than topk candidates exist the rest is (-inf,
 * WQ_TOPK_NO_ID), the pages' sentinel (-INFINITY, UINT_MAX).  1 <= topk <=
 * WQ_TOPK_MAX (the pages' block-local k values go up to 64) else
 * WQ_ERR_TOPK; n < WQ_TOPK_NO_ID.  vals and ids are device pointers
 * (4-byte aligned, not overlapping each other or the inputs).  Scratch:
 * about (16 * CUs + 260) * topk * 8 bytes per call, stream-ordered as above. */
#define WQ_TOPK_MAX 64
#define WQ_TOPK_NO_ID 0xffffffffu

/* Fused LM-head GEMV + top-k for one token: logits[j] = sum_k a[k] w[j, k]
 * for the [n, K] weights b in format fmt (layouts as for the GEMV), and their
 * top-k.  Routes:
 *  - topk == 1, f16 rows on the K-split GEMV (K % 8 == 0, K <= 32768, 16-byte
 *    aligned a and b) or Q8_0 rows on the register-chunk GEMV (the shapes
 *    wq_set_gemv_plan describes): every workgroup folds its best (logit, id)
 *    into one of 4096 device slots with a 64-bit atomic max of an
 *    order-keeping key, and a one-workgroup pass takes the best slot and
 *    clears the slots for the next call (one slot set per cached stream, one
 *    for the allocation-free entry point);
 *  - topk > 1 on those f16 rows, and on Q8_0 / Q4_0 rows with K % 256 == 0 and
 *    16-byte aligned a and b: the GEMV writes the logits to scratch and the
 *    merge reads them 64 at a time;
 *  - everything else (Q4_0 top-1 among them): every wave of the GEMV keeps a
 *    sorted top-k list of the rows it computed, without writing the n logits,
 *    and two small passes merge the lists.
 * The logits are the ones wq_matmul computes for the same arguments, so the
 * result equals wq_matmul followed by wq_topk.
 * Passage: dispatch_lm_head_block_stage1_enc (fused LM-head GEMV with a
 * block-local exact top-k writing compact (logit, token_id) candidates) and
 * dispatch_block_topk_merge_enc (merge of those candidates), lattice-inference
 * 0.9.0 dispatch.rs; k == 1 is the argmax of logits_argmax_first / _merge.
 * n == 0 gives sentinels only; K == 0 (f16) makes every logit 0. */
int wq_lm_head_topk(const float *a, const void *b, int64_t n, int64_t k, int fmt, int topk, float *vals,
                    uint32_t *ids, void *stream);

/* wq_lm_head_topk for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and the same result, bit for bit, but the scratch lives in a fixed
 * array of wq_noalloc_workspace_bytes() (4 MiB) that the library's code object
 * holds in every GPU's memory from load until the process ends; the call itself
 * allocates and frees nothing.  It returns WQ_ERR_WORKSPACE (before anything is
 * enqueued) when the call needs more than that: (n * 4 rounded up to 256) +
 * 256 * topk * 8 bytes on the logits route, else (16 * CUs + 260) * topk * 8
 * bytes -- at most 2.3 MB on MI355X, and 0.7 MB for an LM head at vocab
 * 151936 on the logits route.  Every list or logit the merge reads is written
 * earlier in the same call, so the array needs no clearing (the top-1 slots
 * are a separate fixed array, cleared by the call that fills them).
 * All calls on one GPU share its array and slots:
 * calls that may overlap in time on one GPU (different streams, or several host
 * threads without ordering) race; calls on one stream are ordered and safe. */
int wq_lm_head_topk_noalloc(const float *a, const void *b, int64_t n, int64_t k, int fmt, int topk, float *vals,
                            uint32_t *ids, void *stream);
/* Size of the fixed workspace of the allocation-free entry point (bytes). */
size_t wq_noalloc_workspace_bytes(void);

/* Top-k of an existing f32 logits vector [n] (device): the same selection
 * over logits a caller already has.  Passage: dispatch_topk_enc,
 * lattice-inference 0.9.0 dispatch.rs (argmax for k == 1, tournament merge
 * passes for k > 1). */
int wq_topk(const float *logits, int64_t n, int topk, float *vals, uint32_t *ids, void *stream);

/* ---------------------------------------------------------------------- */
/* Decode attention for one query token over a KV cache (grouped-query,
 * split over the cache).
 *
 * out[h, d] = sum_t p_t v[t, kvh * head_dim + d] with p = softmax over
 * t < cache_len of s_t = scale * sum_d q[h, d] k[t, kvh * head_dim + d] and
 * kvh = h / (num_q_heads / num_kv_heads).  Passage: kernels decode_attention,
 * decode_attention_flash_partial and decode_attention_flash_reduce (online
 * softmax over the cache, per-partition (m, l, acc) partials merged by the
 * same recurrence), lattice-inference 0.1.2 metal_qwen35.rs;
 * dispatch_decode_attention (direct or partitioned, f32 or f16 cache) and
 * validate_flash_decode_shape (GQA group 1..8, q_dim = num_q_heads *
 * head_dim, kv_dim = num_kv_heads * head_dim), lattice-inference 0.9.0
 * dispatch.rs.
 *
 * Layouts (device pointers, row-major): q f32 [num_q_heads, head_dim]; k_cache
 * and v_cache [cache_len, num_kv_heads * head_dim], f32 (kv_fmt WQ_KV_F32) or
 * binary16 bit patterns (WQ_KV_F16), token-major as the pages' flat
 * [max_cache_len * kv_dim] caches, 16-byte aligned; out f32 [num_q_heads,
 * head_dim], 4-byte aligned, not overlapping the inputs.  head_dim is 64, 128
 * or 256 (the pages support 256), num_q_heads a multiple of num_kv_heads with
 * a group of at most WQ_ATTN_MAX_GROUP, else WQ_ERR_SHAPE; an unknown kv_fmt
 * is WQ_ERR_FORMAT.  cache_len == 0 writes zeros (the reduce pass's empty
 * result).  Accumulation in f32; scratch for the partitions' partial states
 * ((num_q_heads * (head_dim + 2) * 4 bytes per partition) as above. */
#define WQ_ATTN_MAX_GROUP 8
enum { WQ_KV_F32 = 0, WQ_KV_F16 = 1 };
int wq_decode_attention(const float *q, const void *k_cache, const void *v_cache, float *out, int64_t cache_len,
                        int head_dim, int num_q_heads, int num_kv_heads, int kv_fmt, float scale, void *stream);

/* Test/tuning hook (host only): every later wq_decode_attention call in the
 * process splits the cache into partitions of `tokens` tokens (0 restores
 * the automatic size, about one workgroup per compute unit and at least 32
 * tokens).  Returns WQ_ERR_SHAPE for tokens < 0.  Not thread-safe with
 * respect to concurrent attention calls that expect the automatic size. */
int wq_set_attn_partition(int64_t tokens);

/* ---------------------------------------------------------------------- */
/* Weight preparation (done once, at load time).
 * wq_pack_f16: out[i] = binary16 bits of w[i], round to nearest even, with
 *   subnormals; overflow gives infinity.  Passage: f32_to_f16 and
 *   make_buffer_f16, lattice-inference 0.1.2 metal_qwen35.rs.
 * wq_quantize_q8_0: count f32 values (count % 32 == 0, else WQ_ERR_K) into
 *   count/32 Q8_0 blocks written to out (count/32*34 bytes).  Per block:
 *   amax = max|v|, d = amax/127, id = 1/d (0 if d == 0), scale bytes =
 *   f16(d) little-endian, q = clamp(round_half_away(v*id), -127, 127), all in
 *   f32.  A row-major [N, K] matrix with K % 32 == 0 gives the [N, K/32*34]
 *   layout above.  Passage: quantize_row_q8_0 and make_buffer_q8_0,
 *   lattice-inference 0.1.2 metal_qwen35.rs.
 * w and out are device pointers (w 4-byte aligned, out 2-byte aligned for
 * f16); count == 0 is a no-op; out must not overlap w. */
int wq_pack_f16(const float *w, uint16_t *out, int64_t count, void *stream);
int wq_quantize_q8_0(const float *w, uint8_t *out, int64_t count, void *stream);

/* ---------------------------------------------------------------------- */
/* Measurement hook: the achievable-read ceiling.  Reads `bytes` bytes at p
 * (device, 16-byte aligned, bytes % 16 == 0, else WQ_ERR_ALIGN / WQ_ERR_SHAPE)
 * once with 128-bit non-temporal loads -- the loads the GEMVs stream weights
 * with -- in workgroups of 256 lanes that each read 1, 2, 4 or 8 slabs of
 * 4 KiB (variant 0..3).  out (device, 4-byte aligned, room for
 * ceil(bytes / 1024) uint32) only receives a value when a workgroup's XOR
 * checksum hits a fixed pattern, so the loads are kept.  It computes nothing of the
 * product; the benchmark times it to report each bandwidth-bound kernel against
 * a plain read of the same bytes as well as against the HBM peak. */
int wq_read_probe(const void *p, int64_t bytes, uint32_t *out, int variant, void *stream);

/* ---------------------------------------------------------------------- */
/* Routing and introspection (host only; these never touch the GPU). */

/* The route wq_matmul takes for these arguments when nothing is forced
 * (WQ_ROUTE_GEMV, WQ_ROUTE_STREAM, WQ_ROUTE_SKINNY or WQ_ROUTE_GEMM_HL) with
 * 16-byte aligned operands and no epilogue, or a negative wq_status on bad
 * arguments.  M == 1 takes the GEMV; quantized M <= 16 with K % 256 == 0 the
 * weight stream, except M == 2 Q8_0 rows whose register-chunk plan keeps at
 * most three units per wave (K % 256 == 0 and K <= 8448), which take the GEMV
 * route. */
int wq_route_for(int64_t m, int64_t n, int64_t k, int fmt);

/* The tiling the GEMM uses for (m, n, k, fmt) on a device with `cus` compute
 * units (256 on MI355X): tile rows *bm, tile columns *bn and the number of K
 * splits *splits (1 = no split; otherwise partial tiles are summed by a
 * second, deterministic pass).  Returns a wq_status; all dimensions must be
 * positive. */
int wq_gemm_plan(int64_t m, int64_t n, int64_t k, int fmt, int cus, int *bm, int *bn, int *splits);

/* Test and tuning hook: force every later GEMM onto tile (bm, bn) with
 * `splits` K splits (capped at the number of 32-wide k-steps); (0, 0, 0)
 * restores the cost model.  Tiles: 128x128, 128x96, 128x64, 64x128, 64x64,
 * 32x128, 16x128, 16x64.  Returns WQ_ERR_SHAPE for anything else.  Results
 * do not depend on the tiling beyond f32 rounding. */
int wq_set_gemm_plan(int bm, int bn, int splits);

/* The tiling of the f16 matrix-core GEMM (WQ_ROUTE_GEMM_HL) for (m, n, k,
 * fmt) on `cus` compute units, as wq_gemm_plan; k % 32 == 0. */
int wq_hgemm_plan(int64_t m, int64_t n, int64_t k, int fmt, int cus, int *bm, int *bn, int *splits);

/* Test and tuning hook: force every later WQ_ROUTE_GEMM_HL product onto tile
 * (bm, bn) (128x128, 128x64, 64x128 or 64x64) with `splits` K splits (capped
 * at K / 32); (0, 0, 0) restores the cost model.  WQ_ERR_SHAPE otherwise. */
int wq_set_hgemm_plan(int bm, int bn, int splits);

/* Test and tuning hook for the Q8_0 and Q4_0 decode GEMV (M == 1,
 * K % 256 == 0, 16-byte aligned operands, N * row bytes < 2^31): force every
 * later call of either format whose shape fits onto the register-chunk kernel
 * with rb rows per workgroup and nf full / nr remainder 64-chunk units per wave
 * (the kernel takes at most 4 waves; shapes that would need more keep the
 * other kernels); (0, 0, 0) restores the measured rule, (-1, 0, 0) switches
 * the kernel off.  Plans: (8,2,1) (4,2,1) (4,3,1) (4,1,1) (8,1,1) (16,1,1)
 * (2,2,1); anything else returns WQ_ERR_SHAPE.  Results do not depend on the
 * plan beyond f32 rounding. */
int wq_set_gemv_plan(int rb, int nf, int nr);

/* Test and tuning hook for the f16 matrix-core weight stream
 * (WQ_ROUTE_STREAM): workgroup shape 1..14 (index into the compiled set of
 * (tiles of 16 weight rows per wave, K sub-ranges per workgroup, tile groups
 * per workgroup, weights staged through LDS): (1,4,1,0) (1,8,1,0) (2,4,1,0)
 * (1,2,2,0) (2,1,4,0) (1,1,4,0) (2,8,1,0) (1,4,1,1) (1,1,4,1) (2,1,4,1)
 * (1,8,1,1) (1,2,2,1) (1,1,8,1) (2,1,8,1)) and the number of K splits across
 * workgroups (at most min(K / 256, 16); raised where one split's activations
 * would not fit the kernel's staging); 0 = automatic for either.  Returns
 * WQ_ERR_SHAPE for a shape outside 0..14 or negative splits.  Results do not depend on the plan beyond
 * f32 rounding. */
int wq_set_stream_plan(int shape, int splits);

/* Force every later wq_matmul call in the process onto one route
 * (WQ_ROUTE_AUTO restores the M rule).  Returns the previous setting, or
 * -WQ_ERR_ROUTE for an unknown value.  Meant for tests that check that all
 * routes agree (the pages' test hook forcing the fallback GEMM). */
int wq_set_forced_route(int route);

/* Kernel launches made so far per route (GEMV, GEMM, SKINNY, STREAM or GEMM_HL) by
 * any entry point, and a reset.  The pages keep such "path proof" counters. */
uint64_t wq_route_count(int route);
void wq_reset_route_counts(void);

/* Static text for a status code ("unknown status" for others). */
const char *wq_status_str(int status);

/* ABI version: 100 * major + minor. */
int wq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WQMM_H */
