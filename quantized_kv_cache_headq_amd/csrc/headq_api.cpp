// headq_api.cpp — the C ABI of libheadq: argument checks, split choice, kernel dispatch.
//
// Every check runs on the host before the first HIP call, so a rejected call enqueues nothing.
// The library allocates no device memory: the caller passes the cache and the workspace.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "headq_internal.h"

namespace {

bool sync_debug() {
  static const bool on = [] {
    const char* s = std::getenv("HEADQ_SYNC_DEBUG");
    return s && s[0] && std::strcmp(s, "0") != 0;
  }();
  return on;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

headq_status finish(hipError_t launched, hipStream_t stream) {
  if (launched != hipSuccess) return HEADQ_ERR_HIP;
  if (hipGetLastError() != hipSuccess) return HEADQ_ERR_HIP;
  if (sync_debug()) {
    if (hipStreamSynchronize(stream) != hipSuccess) return HEADQ_ERR_HIP;
    if (hipGetLastError() != hipSuccess) return HEADQ_ERR_HIP;
  }
  return HEADQ_OK;
}

// Shape checks common to append and decode.
headq_status check_config(const headq_config* c) {
  if (!c) return HEADQ_ERR_NULL;
  if (c->head_dim != 64 && c->head_dim != 128) return HEADQ_ERR_UNSUPPORTED;
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->batch < 1 || c->capacity < 1) return HEADQ_ERR_SHAPE;
  if (c->n_q_heads % c->n_kv_heads) return HEADQ_ERR_SHAPE;
  if (c->n_q_heads / c->n_kv_heads > headq::kMaxGqa) return HEADQ_ERR_UNSUPPORTED;
  if (c->capacity % headq::kGroup) return HEADQ_ERR_ALIGN;
  if (c->base_bits < 2 || c->base_bits > 4 || c->group != headq::kGroup || c->side_bits != 4)
    return HEADQ_ERR_UNSUPPORTED;
  if (c->rank != 0 && c->rank != 4 && c->rank != 8 && c->rank != 16 && c->rank != 32) return HEADQ_ERR_UNSUPPORTED;
  if ((c->key_dtype != HEADQ_F32 && c->key_dtype != HEADQ_BF16) ||
      (c->value_dtype != HEADQ_F32 && c->value_dtype != HEADQ_BF16) ||
      (c->query_dtype != HEADQ_F32 && c->query_dtype != HEADQ_BF16))
    return HEADQ_ERR_UNSUPPORTED;
  if (c->value_mode != HEADQ_V_DENSE && c->value_mode != HEADQ_V_Q2) return HEADQ_ERR_UNSUPPORTED;
  if (c->value_protect < 0 || c->value_protect > 2) return HEADQ_ERR_UNSUPPORTED;
  if (c->value_protect && (c->value_mode != HEADQ_V_Q2 || c->base_bits != 2)) return HEADQ_ERR_UNSUPPORTED;
  return HEADQ_OK;
}

headq_status check_cache(const headq_config* c, const headq_cache* k) {
  if (!k || !k->kcode || !k->kmeta) return HEADQ_ERR_NULL;
  if (k->block_table && (k->max_pages < 1 || k->n_pages < 1 || c->capacity > 32 * k->max_pages))
    return HEADQ_ERR_SHAPE;
  if (c->rank > 0 && (!k->scode || !k->ssc || !k->U)) return HEADQ_ERR_NULL;
  if (c->value_mode == HEADQ_V_DENSE && !k->v) return HEADQ_ERR_NULL;
  if (c->value_mode == HEADQ_V_Q2 && (!k->vcode || !k->vmeta)) return HEADQ_ERR_NULL;
  if (c->value_protect && (!k->vdir || !k->vpidx || !k->vprot)) return HEADQ_ERR_NULL;
  const void* ptrs[] = {k->kcode, k->kmeta, k->scode, k->ssc, k->v,     k->vcode, k->vmeta,
                        k->U,     k->ktail, k->vtail, k->block_table, k->vdir, k->vpidx, k->vprot};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return HEADQ_ERR_ALIGN;
  return HEADQ_OK;
}

headq::CacheMap map_of(const headq_config* c, const headq_cache* k) {
  headq::CacheMap m{};
  m.block_table = k->block_table;
  m.max_pages = k->max_pages;
  m.n_pages = k->n_pages;
  m.hkv = c->n_kv_heads;
  m.groups_cap = c->capacity / headq::kGroup;
  return m;
}

}  // namespace

extern "C" const char* headq_status_string(headq_status s) {
  switch (s) {
    case HEADQ_OK: return "ok";
    case HEADQ_ERR_NULL: return "required pointer is NULL";
    case HEADQ_ERR_SHAPE: return "inconsistent or out-of-range dimensions";
    case HEADQ_ERR_ALIGN: return "buffer, stride or capacity not aligned (16 bytes; capacity a multiple of 32)";
    case HEADQ_ERR_CAPACITY: return "token range exceeds the cache capacity";
    case HEADQ_ERR_WORKSPACE: return "workspace too small";
    case HEADQ_ERR_NUMERIC: return "non-finite input";
    case HEADQ_ERR_UNSUPPORTED: return "setting not supported by libheadq";
    case HEADQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" headq_status headq_cache_append(const headq_config* cfg, const headq_cache* cache, const void* k,
                                           const int64_t k_strides[3], const void* v, const int64_t v_strides[3],
                                           int64_t start, int64_t n_new, const int32_t* row_start,
                                           void* stream) {
  headq_status st = check_config(cfg);
  if (st != HEADQ_OK) return st;
  if (!cache || !k || !k_strides) return HEADQ_ERR_NULL;
  if (v && !v_strides) return HEADQ_ERR_NULL;
  st = check_cache(cfg, cache);
  if (st != HEADQ_OK) return st;
  if (start < 0 || n_new < 0) return HEADQ_ERR_SHAPE;
  if ((row_start ? 0 : start) + n_new > cfg->capacity) return HEADQ_ERR_CAPACITY;
  // a range that starts or ends inside a group goes through the dense tails
  const bool group_aligned = !row_start && start % headq::kGroup == 0 && (start + n_new) % headq::kGroup == 0;
  if (!group_aligned && (!cache->ktail || (v && !cache->vtail))) return HEADQ_ERR_NULL;
  const int kes = cfg->key_dtype == HEADQ_F32 ? 4 : 2;
  const int ves = cfg->value_dtype == HEADQ_F32 ? 4 : 2;
  if (!aligned16(k)) return HEADQ_ERR_ALIGN;
  for (int i = 0; i < 3; ++i) {
    if (k_strides[i] < 0) return HEADQ_ERR_SHAPE;
    if ((k_strides[i] * kes) % 16) return HEADQ_ERR_ALIGN;
  }
  if (k_strides[2] < cfg->head_dim) return HEADQ_ERR_SHAPE;
  if (v) {
    if (!aligned16(v)) return HEADQ_ERR_ALIGN;
    for (int i = 0; i < 3; ++i) {
      if (v_strides[i] < 0) return HEADQ_ERR_SHAPE;
      if ((v_strides[i] * ves) % 16) return HEADQ_ERR_ALIGN;
    }
    if (v_strides[2] < cfg->head_dim) return HEADQ_ERR_SHAPE;
  }
  if (n_new == 0) return HEADQ_OK;

  headq::AppendArgs a{};
  a.d = cfg->head_dim;
  a.key_levels = (1 << cfg->base_bits) - 1;
  a.r = cfg->rank;
  a.hkv = cfg->n_kv_heads;
  a.batch = cfg->batch;
  a.cap = cfg->capacity;
  a.start = start;
  a.n_new = n_new;
  a.key_bf16 = cfg->key_dtype == HEADQ_BF16;
  a.value_bf16 = cfg->value_dtype == HEADQ_BF16;
  a.value_mode = cfg->value_mode;
  a.k = k;
  a.ks_b = k_strides[0];
  a.ks_h = k_strides[1];
  a.ks_t = k_strides[2];
  a.v = v;
  if (v) {
    a.vs_b = v_strides[0];
    a.vs_h = v_strides[1];
    a.vs_t = v_strides[2];
  }
  a.kcode = cache->kcode;
  a.kmeta = cache->kmeta;
  a.scode = cache->scode;
  a.ssc = cache->ssc;
  a.vdense = cache->v;
  a.vcode = cache->vcode;
  a.vmeta = cache->vmeta;
  a.U = cache->U;
  a.ktail = cache->ktail;
  a.vtail = cache->vtail;
  a.row_start = row_start;
  a.map = map_of(cfg, cache);
  a.value_protect = cfg->value_protect;
  a.prot_c2 = (float)(2.0 * 1.4426950408889634 / std::sqrt((double)cfg->head_dim));
  a.vdir = cache->vdir;
  a.vpidx = cache->vpidx;
  a.vprot = cache->vprot;
  hipStream_t s = (hipStream_t)stream;
  return finish(headq::launch_append(a, s), s);
}

namespace {

// The matrix-core kernel handles dense bf16 values and 2-bit values; HEADQ_DECODE_KERNEL=valu
// selects the plain vector kernel instead (kept as the measured comparison and for f32 values).
bool decode_uses_mfma(const headq_config* c) {
  static const bool force_valu = [] {
    const char* s = std::getenv("HEADQ_DECODE_KERNEL");
    return s && std::strcmp(s, "valu") == 0;
  }();
  return !force_valu && (c->value_mode == HEADQ_V_Q2 || c->value_dtype == HEADQ_BF16);
}

// With 2-bit values and g <= 8 heads per KV head the matrix-core kernel lets 16 / g groups share
// the 16 matrix columns; HEADQ_DECODE_PACK=0 keeps one group per product (the measured comparison).
bool decode_packs_columns() {
  static const bool off = [] {
    const char* s = std::getenv("HEADQ_DECODE_PACK");
    return s && std::strcmp(s, "0") == 0;
  }();
  return !off;
}

// Token splits per (b, h) stream. The matrix-core kernel aims at one wave per SIMD at d = 128
// (1024 waves over the 256 CUs: measured faster than two, which contend for the same issue slots
// and memory queues) and at two at d = 64, whose groups are half the work and whose registers
// leave room for two (TinyLlama-shaped decode: 20.4 us at 8 splits against 21.4 us at 4); the
// vector kernel aims at two. Every chunk (the groups one wave walks) stays at least 4 groups long
// so the partials remain a small fraction of the traffic.
int auto_splits(const headq_config* c, int64_t n_groups, int chunks, bool mfma) {
  const int64_t streams = (int64_t)c->batch * c->n_kv_heads;
  const int64_t target_waves = mfma && c->head_dim == 128 ? 1024 : 2048;
  int64_t s = (target_waves + streams * chunks - 1) / (streams * chunks);
  const int64_t min_groups_per_chunk = 4;
  if (s * chunks * min_groups_per_chunk > n_groups) s = n_groups / (chunks * min_groups_per_chunk);
  if (s < 1) s = 1;
  if (s > n_groups) s = n_groups;
  return (int)s;
}

}  // namespace

extern "C" headq_status headq_decode_attn(const headq_config* cfg, const headq_cache* cache, const void* q,
                                          int64_t n_ctx, const int32_t* row_len, void* out, int32_t out_dtype,
                                          float corr_scale,
                                          float* logits_dbg, int32_t n_splits, void* ws, size_t* ws_bytes,
                                          void* stream) {
  headq_status st = check_config(cfg);
  if (st != HEADQ_OK) return st;
  if (!ws_bytes) return HEADQ_ERR_NULL;
  if (n_ctx < 1) return HEADQ_ERR_SHAPE;

  if (n_ctx > cfg->capacity) return HEADQ_ERR_CAPACITY;
  if (out_dtype != HEADQ_F32 && out_dtype != HEADQ_BF16) return HEADQ_ERR_UNSUPPORTED;
  const int64_t n_groups = n_ctx / headq::kGroup;  // whole groups; the rest is in the tails
  // work units for the split: the whole groups plus the unfinished one held in the tails
  const int64_t n_units = n_groups + (n_ctx % headq::kGroup ? 1 : 0);
  if (n_splits < 0 || n_splits > n_units) return HEADQ_ERR_SHAPE;
  const bool mfma = decode_uses_mfma(cfg);
  if (cfg->value_protect && !mfma) return HEADQ_ERR_UNSUPPORTED;  // the policy is read by the matrix-core kernel
  const int chunks = mfma ? 4 : 1;
  const int S = n_splits ? n_splits : auto_splits(cfg, n_units, chunks, mfma);
  if (mfma && S > headq::kMaxSplitsMfma) return HEADQ_ERR_UNSUPPORTED;
  const size_t need = headq::decode_ws_bytes(cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, S);
  if (!ws) {
    *ws_bytes = need;
    return HEADQ_OK;
  }
  if (!cache || !q || !out) return HEADQ_ERR_NULL;
  st = check_cache(cfg, cache);
  if (st != HEADQ_OK) return st;
  if ((row_len || n_ctx % headq::kGroup) && (!cache->ktail || !cache->vtail)) return HEADQ_ERR_NULL;
  if (*ws_bytes < need) return HEADQ_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(out) || !aligned16(ws) || (logits_dbg && !aligned16(logits_dbg)))
    return HEADQ_ERR_ALIGN;

  headq::DecodeArgs a{};
  a.d = cfg->head_dim;
  a.key_nib = cfg->base_bits != 2;
  a.pack_columns = decode_packs_columns();
  a.r = cfg->rank;
  a.hq = cfg->n_q_heads;
  a.hkv = cfg->n_kv_heads;
  a.batch = cfg->batch;
  a.gqa = cfg->n_q_heads / cfg->n_kv_heads;
  a.cap = cfg->capacity;
  a.n_ctx = n_ctx;
  a.n_splits = S;
  a.chunks_per_split = chunks;
  a.use_mfma = mfma;
  a.groups_per_split = (int)((n_units + (int64_t)S * chunks - 1) / ((int64_t)S * chunks));
  a.query_bf16 = cfg->query_dtype == HEADQ_BF16;
  a.value_bf16 = cfg->value_dtype == HEADQ_BF16;
  a.value_mode = cfg->value_mode;
  a.out_bf16 = out_dtype == HEADQ_BF16;
  a.corr_scale = corr_scale;
  a.q = q;
  a.kcode = cache->kcode;
  a.kmeta = cache->kmeta;
  a.scode = cache->scode;
  a.ssc = cache->ssc;
  a.vdense = cache->v;
  a.vcode = cache->vcode;
  a.vmeta = cache->vmeta;
  a.U = cache->U;
  a.ktail = cache->ktail;
  a.vtail = cache->vtail;
  a.value_protect = cfg->value_protect;
  a.vpidx = cache->vpidx;
  a.vprot = cache->vprot;
  a.key_bf16 = cfg->key_dtype == HEADQ_BF16;
  a.row_len = row_len;
  a.map = map_of(cfg, cache);
  a.logits_dbg = logits_dbg;
  a.ws_count = (uint32_t*)ws;
  a.ws_o = (float*)((char*)ws + headq::decode_ws_counter_bytes(cfg->batch, cfg->n_kv_heads));
  a.ws_ml = a.ws_o + (size_t)cfg->batch * cfg->n_q_heads * S * cfg->head_dim;
  a.out = out;
  hipStream_t s = (hipStream_t)stream;
  return finish(headq::launch_decode(a, s), s);
}

extern "C" headq_status headq_score_diagnostics(const headq_config* cfg, const headq_cache* cache, const void* q,
                                                const void* k_ref, const int64_t k_strides[3], const void* v_ref,
                                                const int64_t v_strides[3], int64_t n_ctx, float corr_scale,
                                                double* stats, int32_t n_splits, void* ws, size_t* ws_bytes,
                                                void* stream) {
  headq_status st = check_config(cfg);
  if (st != HEADQ_OK) return st;
  if (!ws_bytes) return HEADQ_ERR_NULL;
  if (n_ctx < 1) return HEADQ_ERR_SHAPE;
  if (n_ctx > cfg->capacity) return HEADQ_ERR_CAPACITY;
  const int64_t n_chunks = (n_ctx + 63) / 64;  // 64-token chunks, one wave each at a time
  if (n_splits < 0 || n_splits > n_chunks) return HEADQ_ERR_SHAPE;
  // automatic: about two waves per SIMD over the whole launch, at least one chunk per wave
  int64_t S = n_splits;
  if (!S) {
    const int64_t streams = (int64_t)cfg->batch * cfg->n_kv_heads;
    S = (2048 + 4 * streams - 1) / (4 * streams);
    if (S * 4 > n_chunks) S = (n_chunks + 3) / 4;
    if (S < 1) S = 1;
  }
  const size_t need = headq::diag_ws_bytes(cfg->batch, cfg->n_q_heads, cfg->n_kv_heads, cfg->head_dim, cfg->rank,
                                           (int)S, n_ctx);
  if (!ws) {
    *ws_bytes = need;
    return HEADQ_OK;
  }
  if (!cache || !q || !k_ref || !k_strides || !stats) return HEADQ_ERR_NULL;
  if (v_ref && !v_strides) return HEADQ_ERR_NULL;
  st = check_cache(cfg, cache);
  if (st != HEADQ_OK) return st;
  if (n_ctx % headq::kGroup && (!cache->ktail || (v_ref && !cache->vtail))) return HEADQ_ERR_NULL;
  if (*ws_bytes < need) return HEADQ_ERR_WORKSPACE;
  const int kes = cfg->key_dtype == HEADQ_F32 ? 4 : 2;
  const int ves = cfg->value_dtype == HEADQ_F32 ? 4 : 2;
  if (!aligned16(q) || !aligned16(k_ref) || !aligned16(stats) || !aligned16(ws) || (v_ref && !aligned16(v_ref)))
    return HEADQ_ERR_ALIGN;
  for (int i = 0; i < 3; ++i) {
    if (k_strides[i] < 0 || (v_ref && v_strides[i] < 0)) return HEADQ_ERR_SHAPE;
    if ((k_strides[i] * kes) % 16 || (v_ref && (v_strides[i] * ves) % 16)) return HEADQ_ERR_ALIGN;
  }
  if (k_strides[2] < cfg->head_dim || (v_ref && v_strides[2] < cfg->head_dim)) return HEADQ_ERR_SHAPE;

  headq::DiagArgs a{};
  a.d = cfg->head_dim;
  a.key_nib = cfg->base_bits != 2;
  a.r = cfg->rank;
  a.hq = cfg->n_q_heads;
  a.hkv = cfg->n_kv_heads;
  a.batch = cfg->batch;
  a.gqa = cfg->n_q_heads / cfg->n_kv_heads;
  a.cap = cfg->capacity;
  a.n_ctx = n_ctx;
  a.n_splits = (int)S;
  a.key_bf16 = cfg->key_dtype == HEADQ_BF16;
  a.value_bf16 = cfg->value_dtype == HEADQ_BF16;
  a.value_mode = cfg->value_mode;
  a.query_bf16 = cfg->query_dtype == HEADQ_BF16;
  a.kappa = corr_scale;
  a.q = q;
  a.k_ref = k_ref;
  a.ks_b = k_strides[0];
  a.ks_h = k_strides[1];
  a.ks_t = k_strides[2];
  a.v_ref = v_ref;
  if (v_ref) {
    a.vs_b = v_strides[0];
    a.vs_h = v_strides[1];
    a.vs_t = v_strides[2];
  }
  a.kcode = cache->kcode;
  a.kmeta = cache->kmeta;
  a.scode = cache->scode;
  a.ssc = cache->ssc;
  a.vdense = cache->v;
  a.vcode = cache->vcode;
  a.vmeta = cache->vmeta;
  a.U = cache->U;
  a.ktail = cache->ktail;
  a.vtail = cache->vtail;
  a.value_protect = cfg->value_protect;
  a.vpidx = cache->vpidx;
  a.vprot = cache->vprot;
  a.map = map_of(cfg, cache);
  const int g = a.gqa;
  a.ws_q = (double*)ws;
  a.ws_qu = a.ws_q + headq::diag_ws_q_doubles(a.batch, a.hkv, g, a.d);
  a.ws_part = a.ws_qu + headq::diag_ws_qu_doubles(a.batch, a.hkv, g, a.r);
  a.ws_dv2 = a.ws_part + (size_t)a.batch * a.hq * S * headq::kDiagPart;
  a.stats = stats;
  hipStream_t s = (hipStream_t)stream;
  return finish(headq::launch_diagnostics(a, s), s);
}

extern "C" headq_status headq_prefill_attn(const headq_config* cfg, const headq_cache* cache, const void* q,
                                           int64_t start, int64_t n_q, void* out, int32_t out_dtype,
                                           float corr_scale, float* logits_dbg, void* stream) {
  headq_status st = check_config(cfg);
  if (st != HEADQ_OK) return st;
  if (!cache || !q || !out) return HEADQ_ERR_NULL;
  st = check_cache(cfg, cache);
  if (st != HEADQ_OK) return st;
  if (start < 0 || n_q < 1 || start + n_q > INT32_MAX) return HEADQ_ERR_SHAPE;  // positions are 32-bit in-kernel
  if (start + n_q > cfg->capacity) return HEADQ_ERR_CAPACITY;
  if (out_dtype != HEADQ_F32 && out_dtype != HEADQ_BF16) return HEADQ_ERR_UNSUPPORTED;
  // the matrix-core formats: dense bf16 or 2-bit values
  if (cfg->value_mode == HEADQ_V_DENSE && cfg->value_dtype != HEADQ_BF16) return HEADQ_ERR_UNSUPPORTED;
  if ((start + n_q) % headq::kGroup && (!cache->ktail || !cache->vtail)) return HEADQ_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || (logits_dbg && !aligned16(logits_dbg))) return HEADQ_ERR_ALIGN;

  headq::PrefillArgs a{};
  a.d = cfg->head_dim;
  a.key_nib = cfg->base_bits != 2;
  a.r = cfg->rank;
  a.hq = cfg->n_q_heads;
  a.hkv = cfg->n_kv_heads;
  a.batch = cfg->batch;
  a.gqa = cfg->n_q_heads / cfg->n_kv_heads;
  a.cap = cfg->capacity;
  a.start = start;
  a.n_q = n_q;
  a.query_bf16 = cfg->query_dtype == HEADQ_BF16;
  a.key_bf16 = cfg->key_dtype == HEADQ_BF16;
  a.value_bf16 = cfg->value_dtype == HEADQ_BF16;
  a.value_mode = cfg->value_mode;
  a.out_bf16 = out_dtype == HEADQ_BF16;
  a.corr_scale = corr_scale;
  a.q = q;
  a.kcode = cache->kcode;
  a.kmeta = cache->kmeta;
  a.scode = cache->scode;
  a.ssc = cache->ssc;
  a.vdense = cache->v;
  a.vcode = cache->vcode;
  a.vmeta = cache->vmeta;
  a.U = cache->U;
  a.ktail = cache->ktail;
  a.vtail = cache->vtail;
  a.value_protect = cfg->value_protect;
  a.vpidx = cache->vpidx;
  a.vprot = cache->vprot;
  a.map = map_of(cfg, cache);
  a.logits_dbg = logits_dbg;
  a.out = out;
  hipStream_t s = (hipStream_t)stream;
  return finish(headq::launch_prefill(a, s), s);
}
