/*
 * headq.h — C ABI of libheadq, the HeadQ key-side KV-cache hot path for AMD Instinct MI355X
 * (gfx950, CDNA4).
 *
 * HeadQ ("HeadQ: Model-Visible Distortion and Score-Space Correction for KV-Cache
 * Quantization"; Dutch technical summary "Technische Samenvatting", §3 "Algorithmisch
 * Overzicht") keeps each cached key as a low-bit base code plus a low-rank side code of its
 * residual in a query basis U_h, and adds the side code back as a logit correction at decode:
 *
 *   calibrate  U_h = top-r principal directions of post-RoPE calibration queries   (§3 step 1)
 *   write      k_base = B_b(k);  e = k - k_base;  z = Q_q(U_h^T e)                  (§3 step 2)
 *   read       s_j = q.k_base_j / sqrt(d) + (U_h^T q).z_hat_j / sqrt(d), softmax, sum_j p_j v_j
 *                                                                                   (§3 step 3)
 *
 * One call per phase: headq_calibrate (host), headq_cache_append (GPU), headq_decode_attn (GPU);
 * around them headq_prefill_attn (chunked-prefill attention, GPU), headq_score_diagnostics
 * (score-space diagnostics, GPU) and headq_calibrate_mean (the direction of the optional A^2 value
 * policy, host).
 *
 * Conventions
 *   Ownership  The caller owns every buffer. The library never allocates, frees or keeps device
 *              memory and holds no mutable global state; calls are re-entrant.
 *   Streams    GPU calls enqueue work on `stream` (a hipStream_t; NULL = the null stream) and
 *              return without synchronizing. Set HEADQ_SYNC_DEBUG=1 in the environment to make
 *              each GPU call synchronize and report asynchronous errors.
 *   Graphs     A GPU call is kernel launches on `stream` only (no allocation, copy, memset or
 *              synchronization outside debug mode), so callers may capture it in a HIP graph;
 *              the decode workspace's counters return to zero within every call, so a captured
 *              decode replays with the same workspace.
 *   Errors     Every argument is checked on the host before any HIP call, so a rejected call
 *              enqueues nothing. HEADQ_ERR_HIP reports a launch (or, in debug mode, execution)
 *              error from the HIP runtime.
 *   Numbers    fp16 = IEEE binary16 bits (uint16_t); bf16 = bfloat16 bits (uint16_t); both
 *              rounded to nearest even wherever the library produces them.
 *   Preconditions not checked on the device: keys, values and queries are finite and below
 *              65504 in magnitude (binary16 metadata must not overflow).
 *
 * Cache format (per layer). Every buffer is indexed [b][h] first (batch, KV head), then by
 * token; `cap` = capacity in tokens (a multiple of 32); G = 32 tokens per group; d = head_dim;
 * r = rank. All buffers must be 16-byte aligned.
 *   kcode  u8   [B][Hkv][cap][d/4]       2-bit base codes, d/16 little-endian 32-bit words per
 *                                        token: channel 16m + j (j = 8q + 2b + e) at bit
 *                                        8b + 4e + 2q of word m (one mask or one shift leaves
 *                                        one code per nibble, in channel order).
 *                                        base_bits 3 or 4: [B][Hkv][cap][d/2], one code per
 *                                        nibble, d/8 words per token, channel 8m + j at bit
 *                                        4*(j/2) + 16*(j%2) of word m
 *   kmeta  fp16 [B][Hkv][cap/G][2][d]    per (group, channel): row 0 = step s, row 1 = zero z
 *   scode  u8   [B][Hkv][cap][r/2]       4-bit side codes u = zc + 8; component 2i in the low
 *                                        nibble of byte i, component 2i+1 in the high nibble
 *   ssc    fp16 [B][Hkv][cap]            per-token side step sigma (z_hat = sigma * zc)
 *   v      (dense values) f32 or bf16 [B][Hkv][cap/G][d][G]: within a 32-token group the values
 *                                        are stored channel-major (token index fastest)
 *   vcode  u8   [B][Hkv][cap/G][d*8]     (2-bit values) per group, in matrix-operand order: lane
 *                                        l = 16*(t/8) + c%16 owns bytes [l*d/8, (l+1)*d/8), two
 *                                        per 16-channel tile c/16; token item i = t%8 = 4q+2b+e
 *                                        sits in byte b of that pair at bit 4e + 2q
 *   vmeta  fp16 [B][Hkv][cap/G][2][d/32][G]  (2-bit values) per (token, 32-channel group):
 *                                        row 0 = step, row 1 = zero, token index fastest
 *   ktail  key_dtype   [B][Hkv][G][d]    tokens of the unfinished last group (row t % 32), exact
 *   vtail  value_dtype [B][Hkv][G][d]    their values, exact (also in 2-bit mode)
 *   vpidx  u32  [B][Hkv][cap/G]          (value_protect = P > 0) byte i < P: the index in its group
 *                                        of the token in correction slot i (ascending); others 0
 *   vprot  bf16 [B][Hkv][cap/G][P][d]    (value_protect > 0) slot i: v - v_hat of that token, so
 *                                        that the token's value reads v_hat + correction
 * Paged caches (block_table != NULL): every array above except U and the tails is instead a pool
 * of n_pages pages, the [B][Hkv][cap/G] group index replaced by [n_pages][Hkv]: the group g of
 * batch row b lives in page block_table[b * max_pages + g] (one page = one 32-token group of all
 * KV heads; e.g. kcode [n_pages][Hkv][G][d/4], v [n_pages][Hkv][d][G], vpidx [n_pages][Hkv]);
 * `capacity` is then the
 * per-row logical capacity, at most 32 * max_pages. Pages are assigned by the caller; entries
 * outside [0, n_pages) are clamped by the kernels (to stay inside the pools).
 *   U      f32  [Hkv][d][r]              the side basis (device copy of headq_calibrate's output)
 */
#ifndef HEADQ_H
#define HEADQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum headq_status {
  HEADQ_OK = 0,
  HEADQ_ERR_NULL = 1,        /* a required pointer is NULL */
  HEADQ_ERR_SHAPE = 2,       /* inconsistent or out-of-range dimensions */
  HEADQ_ERR_ALIGN = 3,       /* a token count/offset is not a multiple of 32, or a buffer or
                                stride breaks the 16-byte alignment rule */
  HEADQ_ERR_CAPACITY = 4,    /* start + n_new > capacity, or n_ctx > capacity */
  HEADQ_ERR_WORKSPACE = 5,   /* *ws_bytes smaller than the size this call needs */
  HEADQ_ERR_NUMERIC = 6,     /* non-finite calibration input */
  HEADQ_ERR_UNSUPPORTED = 7, /* a well-formed setting libheadq does not implement */
  HEADQ_ERR_HIP = 8          /* the HIP runtime reported an error */
} headq_status;

/* element types */
enum { HEADQ_F32 = 0, HEADQ_BF16 = 1 };
/* value storage */
enum { HEADQ_V_DENSE = 0, HEADQ_V_Q2 = 1 };

typedef struct headq_config {
  int32_t head_dim;    /* d: 64 or 128 */
  int32_t n_q_heads;   /* Hq */
  int32_t n_kv_heads;  /* Hkv; g = Hq / Hkv query heads share one KV head (1 <= g <= 16);
                          query head hq reads KV head hq / g */
  int32_t batch;       /* B >= 1 */
  int64_t capacity;    /* tokens per (b, h) stream, a positive multiple of 32 */
  int32_t base_bits;   /* bits of the base key code: 2 (four codes per byte), or 3 / 4 (one code per
                          nibble, 7 / 15 levels; values stay 2-bit) */
  int32_t group;       /* tokens per base-quantizer group: 32 */
  int32_t rank;        /* r: 0, 4, 8, 16 or 32 (0 = base quantizer only) */
  int32_t side_bits;   /* bits per side-code component: 4 */
  int32_t key_dtype;   /* HEADQ_F32 or HEADQ_BF16: dtype of the keys given to append */
  int32_t value_dtype; /* HEADQ_F32 or HEADQ_BF16: dtype of the values given to append, and of
                          the dense value store */
  int32_t value_mode;  /* HEADQ_V_DENSE or HEADQ_V_Q2 (2-bit values, d = 128 or 64) */
  int32_t query_dtype; /* HEADQ_F32 or HEADQ_BF16: dtype of decode queries */
  int32_t value_protect; /* A^2 value policy: P tokens of every 32-token group that keep a bfloat16
                            correction on top of their 2-bit value codes; 0 (off), 1 or 2; P > 0
                            needs HEADQ_V_Q2 and base_bits 2 (see headq_calibrate_mean) */
} headq_config;

typedef struct headq_cache { /* device pointers, layouts in the header comment above */
  uint8_t* kcode;
  uint16_t* kmeta;
  uint8_t* scode;  /* may be NULL when rank == 0 */
  uint16_t* ssc;   /* may be NULL when rank == 0 */
  void* v;         /* dense values (value_mode == HEADQ_V_DENSE) */
  uint8_t* vcode;  /* 2-bit values (value_mode == HEADQ_V_Q2) */
  uint16_t* vmeta; /* 2-bit values (value_mode == HEADQ_V_Q2) */
  const float* U;  /* [Hkv][d][r]; may be NULL when rank == 0 */
  void* ktail;     /* dense tail keys; may be NULL if every append and n_ctx is group-aligned */
  void* vtail;     /* dense tail values; may be NULL likewise */
  const int32_t* block_table; /* device int32 [B][max_pages]: paged cache, or NULL (contiguous) */
  int64_t max_pages;          /* pages per batch row in block_table */
  int64_t n_pages;            /* pages in each pool */
  const float* vdir;          /* value_protect > 0: [Hkv][d], the policy's direction a_h
                                 (device copy of headq_calibrate_mean's output) */
  uint32_t* vpidx;            /* value_protect > 0: the policy's token indices per group */
  uint16_t* vprot;            /* value_protect > 0: the policy's bfloat16 corrections */
} headq_cache;

/*
 * headq_calibrate — learn the side basis U_h from calibration queries (host only, synchronous).
 * Summary §3 step 1: a rank-r basis per layer and head from PCA of post-RoPE calibration
 * queries. This library's reading: one basis per KV head, pooling the g query heads that read
 * it; the uncentered second moment (1/n) sum q q^T (the score error is q.e with the raw query);
 * columns are the eigenvectors of the r largest eigenvalues in decreasing order, each signed so
 * that its largest-magnitude entry (lowest index on ties) is positive. Computed in fp64
 * (Householder tridiagonalization + implicit symmetric QR with Wilkinson shifts).
 *   q_cal  host f32 [Hq][n_cal][d], post-RoPE calibration queries (read only)
 *   U      host f32 [Hkv][d][r] (written)
 *   eig    host f64 [Hkv][r] eigenvalues (written; may be NULL)
 * Errors: NULL, SHAPE (n_cal < 1, r > d), UNSUPPORTED (d, r), NUMERIC (non-finite input).
 */
headq_status headq_calibrate(const headq_config* cfg, const float* q_cal, int64_t n_cal, float* U,
                             double* eig);

/*
 * headq_calibrate_mean — the direction of the A^2 value policy (host only, synchronous).
 * Summary §2.2 measures value error by the A^2 surrogate sum_j p_j^2 |v_hat_j - v_j|^2 and §5
 * pairs HeadQ keys with an A^2-weighted value policy; the pages do not define the policy. This
 * library's reading (value_protect = P > 0, applied by headq_cache_append): per 32-token group the
 * P tokens of largest w_j * e_j keep a bfloat16 correction v_j - v_hat_j, where
 *   e_j = sum_c (v_jc - fma(code, s, z))^2, one f32 fma chain over c = 0..d-1 from +0,
 *   w_j = 2^n_j, n_j = clamp(rint(c2 * (a_h . k_j)), -64, 64), a_h . k_j one f32 fma chain over
 *         c = 0..d-1 from +0, c2 = f32(2 log2(e) / sqrt(d)): a power-of-two estimate of
 *         exp(2 a_h.k_j / sqrt(d)), to which E[p_j^2] is proportional within a group at first order,
 *   w_j * e_j compared exactly, ties to the lower token index, slots in ascending token order.
 * a_h is the mean post-RoPE calibration query of KV head h, pooling its g query heads: f64 sums
 * in head order, then query order, divided by g * n_cal, rounded to f32.
 *   q_cal  host f32 [Hq][n_cal][d] (read only)
 *   a      host f32 [Hkv][d] (written)
 * Errors: NULL, SHAPE (n_cal < 1), UNSUPPORTED (d), NUMERIC (non-finite input).
 */
headq_status headq_calibrate_mean(const headq_config* cfg, const float* q_cal, int64_t n_cal, float* a);

/*
 * headq_cache_append — quantize and store tokens [start, start + n_new) of every (b, h) stream.
 * Summary §3 step 2: base-quantize each key with B_b, take the residual e = k - k_base,
 * project it on U_h and side-quantize the projection with Q_q; the cache keeps the base key and
 * the side code. This library's numerics (the integer results are bit-exact with a plain CPU
 * evaluation of the same formulas):
 *   per (32-token group, channel): s = fp16((max - min) / 3), z = fp16(min)
 *   code = clamp(rint((k - z) * (1/s)), 0, 3)   (1/s = 0 when s == 0; ties to even)
 *   e = k - fma(code, s, z)                      (f32)
 *   y_i = sum_c U[c][i] e_c as one f32 fma chain over c = 0..d-1 starting from +0
 *   sigma = fp16(max_i |y_i| / 7), zc_i = clamp(rint(y_i * (1/sigma)), -7, 7) (all 0 if sigma == 0)
 * Dense values are copied into the cache layout; 2-bit values get the per-token quantizer over
 * 32-channel groups with the same numerics, and with value_protect > 0 every encoded group gets
 * the A^2 value policy's corrections (headq_calibrate_mean; its direction from cache->vdir).
 * Appends may be token-granular: every 32-token group that is whole once tokens
 * [start, start + n_new) are in is encoded (its tokens before `start` are taken from the tails), and the tokens of an unfinished last group are copied exactly into
 * ktail / vtail (rows t % 32). Appends to a stream must be sequential: the tails hold tokens
 * [32 * floor(start / 32), start) from earlier calls.
 *   k        device keys, key_dtype, element (b, h, t, c) at k[b*ks[0] + h*ks[1] + t*ks[2] + c]
 *   k_strides element strides {batch, kv head, token}; channel stride is 1
 *   v        device values (value_dtype; f32 or bf16 also in 2-bit mode), or NULL to leave the
 *            value store untouched; v_strides as for keys (ignored when v is NULL)
 *   start, n_new  token range of every stream, start + n_new <= capacity
 *   row_start  device int32 [B] or NULL: batch row b appends its n_new tokens at row_start[b]
 *            instead of `start` (rows at different lengths; `start` is then ignored). Requires
 *            both tails. Precondition row_start[b] + n_new <= capacity (a row that would pass the
 *            capacity is left untouched).
 * Errors: NULL (also: a range that is not group-aligned without ktail, or without vtail when v is
 * given), SHAPE, ALIGN (k, v and stride*element_size not multiples of 16 bytes), CAPACITY,
 * UNSUPPORTED, HIP. n_new == 0 is a no-op.
 */
headq_status headq_cache_append(const headq_config* cfg, const headq_cache* cache, const void* k,
                                const int64_t k_strides[3], const void* v, const int64_t v_strides[3],
                                int64_t start, int64_t n_new, const int32_t* row_start, void* stream);

/*
 * headq_decode_attn — one decode step of attention for every (b, query head) over the first
 * n_ctx cached tokens. Summary §3 step 3: the runtime query decodes the side code through
 * U_h^T q and the corrected logit q.k_base/sqrt(d) + (U_h^T q).z_hat/sqrt(d) is taken directly,
 * without rebuilding a full key; then softmax and the value readout sum_j p_j v_j (§1, §2.2).
 * Computed in f32 with exact softmax over the n_ctx tokens, split over token ranges that are
 * merged by log-sum-exp.
 *   q           device [B][Hq][d] in query_dtype (contiguous)
 *   n_ctx       tokens attended, 1 <= n_ctx <= capacity; the n_ctx % 32 tokens past the last
 *               whole group are read from ktail / vtail with exact keys and values (no side code)
 *   row_len     device int32 [B] or NULL: batch row b attends its first row_len[b] tokens
 *               (precondition 1 <= row_len[b] <= n_ctx; n_ctx then only bounds the rows, sizes
 *               the splits and is the row stride of logits_dbg). Requires both tails.
 *   out         device [B][Hq][d] in out_dtype (HEADQ_F32 or HEADQ_BF16), contiguous
 *   corr_scale  multiplies the correction: 1 = HeadQ, 0 = base code only, -1 = wrong sign
 *   logits_dbg  device f32 [B][Hq][n_ctx] corrected logits in natural-log units, or NULL
 *   n_splits    token splits per (b, h); 0 = automatic, else 1..max(1, n_ctx/32) (at most 128
 *               with dense bf16 or 2-bit values, the matrix-core path)
 *   ws, ws_bytes  device workspace. With ws == NULL the call only stores the bytes it needs in
 *               *ws_bytes and returns HEADQ_OK (nothing is launched). Otherwise *ws_bytes is
 *               the size of ws. The workspace must be zero-filled before its first use; every
 *               call leaves its leading counter region zero again, so one zeroed workspace
 *               serves any number of calls. Calls that share a workspace must not overlap.
 * With value_protect > 0 the readout adds p_t * correction_t for every token t the cache holds
 * a correction for (the matrix-core kernel; HEADQ_DECODE_KERNEL=valu then returns UNSUPPORTED).
 * Errors: NULL (also: n_ctx % 32 != 0 without both tails), SHAPE, ALIGN, CAPACITY, WORKSPACE,
 * UNSUPPORTED, HIP.
 */
headq_status headq_decode_attn(const headq_config* cfg, const headq_cache* cache, const void* q,
                               int64_t n_ctx, const int32_t* row_len, void* out, int32_t out_dtype, float corr_scale,
                               float* logits_dbg,
                               int32_t n_splits, void* ws, size_t* ws_bytes, void* stream);

/*
 * headq_prefill_attn — chunked-prefill attention over the cache: query token t of every batch row
 * sits at position start + t and attends the cached tokens 0 .. start + t (causal), with the
 * decode's corrected logit and readout (Summary §3 step 3, read once per query token; §1, §2.2).
 * The chunk's own keys and values must be in the cache already (headq_cache_append of tokens
 * [start, start + n_q) first), so the cache holds tokens [0, start + n_q); those past the last
 * whole group come from ktail / vtail, exactly. Runs on the matrix cores: dense bf16 or 2-bit
 * values (dense f32 values: UNSUPPORTED). Numerics as headq_decode_attn.
 *   q           device [B][n_q][Hq][d] in query_dtype (contiguous)
 *   start, n_q  first position and number of query tokens, start + n_q <= capacity
 *   out         device [B][n_q][Hq][d] in out_dtype (HEADQ_F32 or HEADQ_BF16), contiguous
 *   corr_scale  multiplies the correction (1 = HeadQ, 0 = base only, -1 = wrong sign)
 *   logits_dbg  device f32 [B][n_q][Hq][start + n_q]: logits of the attended tokens (natural-log
 *               units; entries past a token's causal limit are left untouched), or NULL
 * Errors: NULL (also: start + n_q not a multiple of 32 without both tails), SHAPE, ALIGN,
 * CAPACITY, UNSUPPORTED, HIP. With value_protect > 0 the readout adds the A^2 value policy's
 * corrections as the decode does.
 */
headq_status headq_prefill_attn(const headq_config* cfg, const headq_cache* cache, const void* q, int64_t start,
                                int64_t n_q, void* out, int32_t out_dtype, float corr_scale, float* logits_dbg,
                                void* stream);

/* Statistics of headq_score_diagnostics, per (batch row, query head). */
enum {
  HEADQ_DIAG_FISHER_VAR = 0, /* Var_p(ds): Fisher-weighted variance of the score error */
  HEADQ_DIAG_KL = 1,         /* KL(p || p_hat) of the exact against the cache's attention */
  HEADQ_DIAG_MEAN_DS = 2,    /* E_p[ds]: the softmax-null part of the score error */
  HEADQ_DIAG_MAX_ABS_DS = 3, /* max_j |ds_j| */
  HEADQ_DIAG_A2 = 4,         /* sum_j p_j^2 |v_hat_j - v_j|^2 (NaN without reference values) */
  HEADQ_DIAG_ENTROPY = 5,    /* -sum_j p_j log p_j of the exact attention */
  HEADQ_DIAG_NSTAT = 6
};

/*
 * headq_score_diagnostics — score-space diagnostics of the cache against the keys (and values)
 * it was written from, for calibration sweeps and the method's controls (wrong sign through
 * corr_scale = -1, random or other bases through U, rank 0). Summary §2.1: a key error reaches
 * the model only through the score error ds_j = s_hat_j - s_j, and the local KL between exact and
 * perturbed attention is its Fisher-weighted variance; §2.2: the A^2 surrogate weighs each
 * token's value distortion by p_j^2. Here s_j = q.k_j/sqrt(d) from the reference keys,
 * p = softmax(s), s_hat_j the cache's corrected logit of §3 step 3 (base key plus corr_scale
 * times the side correction; tokens in the tails are exact), v_hat_j the cache's value (with the
 * A^2 value policy's correction where the cache holds one). All arithmetic is f64; KL is
 * evaluated as log E_p[exp(ds)] - E_p[ds].
 *   q        device [B][Hq][d] in query_dtype (contiguous)
 *   k_ref    device reference keys in key_dtype, element (b, h, t, c) at
 *            k_ref[b*ks[0] + h*ks[1] + t*ks[2] + c] (as for headq_cache_append)
 *   v_ref    device reference values in value_dtype, or NULL (HEADQ_DIAG_A2 is then NaN)
 *   n_ctx    tokens, 1 <= n_ctx <= capacity (n_ctx % 32 != 0 needs both tails)
 *   stats    device f64 [B][Hq][HEADQ_DIAG_NSTAT] (written)
 *   n_splits workgroups per (b, h); 0 = automatic, else 1..ceil(n_ctx / 64)
 *   ws, ws_bytes  device workspace, 16-byte aligned; with ws == NULL only *ws_bytes is set
 *            (nothing launched). No zero-fill needed. Calls sharing ws must not overlap.
 * Errors: NULL, SHAPE, ALIGN, CAPACITY, WORKSPACE, UNSUPPORTED, HIP.
 */
headq_status headq_score_diagnostics(const headq_config* cfg, const headq_cache* cache, const void* q,
                                     const void* k_ref, const int64_t k_strides[3], const void* v_ref,
                                     const int64_t v_strides[3], int64_t n_ctx, float corr_scale, double* stats,
                                     int32_t n_splits, void* ws, size_t* ws_bytes, void* stream);

/* Human-readable name of a status code (static storage). */
const char* headq_status_string(headq_status s);

/* ---- layout sizes in bytes (inline helpers, not exported) ---- */
static inline size_t headq_kcode_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * c->capacity * (c->base_bits == 2 ? c->head_dim / 4 : c->head_dim / 2);
}
static inline size_t headq_kmeta_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * (c->capacity / 32) * 2 * c->head_dim * 2;
}
static inline size_t headq_scode_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * c->capacity * (c->rank / 2);
}
static inline size_t headq_ssc_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * c->capacity * 2;
}
static inline size_t headq_v_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * c->capacity * c->head_dim * (c->value_dtype == HEADQ_F32 ? 4 : 2);
}
static inline size_t headq_vcode_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * c->capacity * (c->head_dim / 4);
}
static inline size_t headq_vmeta_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * c->capacity * (c->head_dim / 32) * 2 * 2;
}
/* Paged pools: bytes of one page (one 32-token group of every KV head) of each array. */
static inline size_t headq_page_kcode_bytes(const headq_config* c) {
  return (size_t)c->n_kv_heads * 32 * (c->base_bits == 2 ? c->head_dim / 4 : c->head_dim / 2);
}
static inline size_t headq_page_kmeta_bytes(const headq_config* c) { return (size_t)c->n_kv_heads * 2 * c->head_dim * 2; }
static inline size_t headq_page_scode_bytes(const headq_config* c) { return (size_t)c->n_kv_heads * 32 * (c->rank / 2); }
static inline size_t headq_page_ssc_bytes(const headq_config* c) { return (size_t)c->n_kv_heads * 32 * 2; }
static inline size_t headq_page_v_bytes(const headq_config* c) {
  return (size_t)c->n_kv_heads * 32 * c->head_dim * (c->value_dtype == HEADQ_F32 ? 4 : 2);
}
static inline size_t headq_page_vcode_bytes(const headq_config* c) { return (size_t)c->n_kv_heads * c->head_dim * 8; }
static inline size_t headq_page_vmeta_bytes(const headq_config* c) { return (size_t)c->n_kv_heads * 2 * c->head_dim * 2; }
static inline size_t headq_vpidx_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * (c->capacity / 32) * 4;
}
static inline size_t headq_vprot_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * (c->capacity / 32) * c->value_protect * c->head_dim * 2;
}
static inline size_t headq_page_vpidx_bytes(const headq_config* c) { return (size_t)c->n_kv_heads * 4; }
static inline size_t headq_page_vprot_bytes(const headq_config* c) {
  return (size_t)c->n_kv_heads * c->value_protect * c->head_dim * 2;
}
static inline size_t headq_ktail_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * 32 * c->head_dim * (c->key_dtype == HEADQ_F32 ? 4 : 2);
}
static inline size_t headq_vtail_bytes(const headq_config* c) {
  return (size_t)c->batch * c->n_kv_heads * 32 * c->head_dim * (c->value_dtype == HEADQ_F32 ? 4 : 2);
}

#ifdef __cplusplus
}
#endif
#endif /* HEADQ_H */
