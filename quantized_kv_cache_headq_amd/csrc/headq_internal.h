// headq_internal.h — launch descriptors shared by the host API and the HIP kernels of libheadq.
// Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "headq.h"

namespace headq {

constexpr int kGroup = 32;     // tokens per base-quantizer group
constexpr int kMaxGqa = 16;    // query heads per KV head supported by the decode kernels
constexpr int kMaxSplitsMfma = 128;  // splits per stream of the matrix-core decode (its in-kernel
                                     // merge stages 2 * splits * g floats in LDS)

// Packed 2-bit code layouts of the cache (the decode kernels turn a 32-bit word into eight f16 or
// bf16 operand pairs with one mask, one shift and byte-wise fp4 conversions):
//   keys   channel 16m + j of a token, j = 8q + 2b + e, at bit 8b + 4e + 2q of 32-bit word m
//   values per 32-token group, lane l = 16*(t/8) + c%16 owns d/8 bytes, two per 16-channel tile
//          c/16; token item i = t%8 = 4q + 2b + e sits in byte b of that pair at bit 4e + 2q
__host__ __device__ constexpr int kcode_bit(int j) { return 8 * ((j % 8) / 2) + 4 * (j % 2) + 2 * (j / 8); }
// 3- and 4-bit base codes, one per nibble: a token row is d/2 bytes, channel 8m + j at bit
// 4*(j/2) + 16*(j%2) of word m (channels 2i and 2i+1 share nibble i of the two 16-bit halves, which
// the matrix-core kernels turn into an f16 pair with one mask and one or)
__host__ __device__ constexpr int kcode4_bit(int j) { return 4 * (j / 2) + 16 * (j % 2); }
__host__ __device__ constexpr int kcode_row_bytes(int d, bool nib) { return nib ? d / 2 : d / 4; }
__host__ __device__ constexpr int vcode_pair_offset(int d, int c, int t) {  // byte offset of the 16-bit pair
  return ((16 * ((t % 32) / 8) + c % 16) * (d / 16) + c / 16) * 2;
}
__host__ __device__ constexpr int vcode_pair_bit(int t) {  // bit of token t inside its 16-bit pair
  return 8 * (((t % 8) % 4) / 2) + 4 * (t % 2) + 2 * ((t % 8) / 4);
}

// Where the block of one (batch row b, KV head h, 32-token group g) lives. Every cache array is a
// sequence of such blocks (kcode 32*d/4 bytes, kmeta 2*d halves, scode 32*r/2 bytes, ssc 32 halves,
// dense values d*32 elements, vcode d*8 bytes, vmeta 2*d halves; per-token rows of kcode, scode
// and ssc are block*32 + t). Contiguous caches: block = (b*Hkv + h)*groups_cap + g. Paged caches
// (block_table != null): block = page*Hkv + h with page = block_table[b*max_pages + g], from pools
// shared by all rows; an entry outside [0, n_pages) is clamped so a bad table cannot address
// outside the pools.
struct CacheMap {
  const int32_t* block_table;
  int64_t max_pages;
  int64_t n_pages;
  int hkv;
  int64_t groups_cap;
  __device__ __forceinline__ int64_t block(int b, int h, int64_t g) const {
    if (!block_table) return ((int64_t)b * hkv + h) * groups_cap + g;
    int64_t page = block_table[(int64_t)b * max_pages + g];
    page = page < 0 ? 0 : (page >= n_pages ? n_pages - 1 : page);
    return page * hkv + h;
  }
  __device__ __forceinline__ int64_t row(int b, int h, int64_t tok) const {
    return block(b, h, tok / 32) * 32 + tok % 32;
  }
};

struct AppendArgs {
  int d, r, hkv, batch;
  int64_t cap;                 // tokens per stream in the cache
  int64_t start, n_new;        // token range written (multiples of 32)
  int key_bf16, value_bf16, value_mode;
  int key_levels;              // base-code levels 2^bits - 1 (3, 7 or 15)
  const void* k;
  int64_t ks_b, ks_h, ks_t;    // key element strides
  const void* v;               // may be null: values untouched
  int64_t vs_b, vs_h, vs_t;
  uint8_t* kcode;
  uint16_t* kmeta;
  uint8_t* scode;
  uint16_t* ssc;
  void* vdense;
  uint8_t* vcode;
  uint16_t* vmeta;
  const float* U;
  void* ktail;                 // [B][Hkv][32][d] key_dtype: tokens of the unfinished last group
  void* vtail;                 // [B][Hkv][32][d] value_dtype
  const int32_t* row_start;    // [B] per-row append position, or null (all rows at `start`)
  CacheMap map;
  int value_protect;           // A^2 value policy: corrected tokens per group (0 = off)
  float prot_c2;               // its weight scale, f32(2 log2(e) / sqrt(d))
  const float* vdir;           // [Hkv][d] its direction
  uint32_t* vpidx;             // per group block: the corrected tokens' indices, one per byte
  uint16_t* vprot;             // per group block: [P][d] bf16 corrections
};

struct DecodeArgs {
  int d, r, hq, hkv, batch, gqa;
  int64_t cap, n_ctx;
  int n_splits;                // token splits (workgroups) per (b, h); one partial result each
  int groups_per_split;        // 32-token groups per chunk; a split has chunks_per_split chunks
  int chunks_per_split;        // 1 (VALU kernel) or 4 (MFMA kernel: one chunk per wave)
  int use_mfma;                // matrix-core kernel (dense bf16 or 2-bit values)
  int query_bf16, value_bf16, value_mode, out_bf16;
  int key_nib;                 // 3- or 4-bit base codes (one per nibble)
  int pack_columns;            // 2-bit values, g <= 8: several groups share the matrix columns
  float corr_scale;
  const void* q;
  const uint8_t* kcode;
  const uint16_t* kmeta;
  const uint8_t* scode;
  const uint16_t* ssc;
  const void* vdense;
  const uint8_t* vcode;
  const uint16_t* vmeta;
  const float* U;
  const void* ktail;           // tail of the unfinished group (n_ctx % 32 tokens), exact
  const void* vtail;
  const uint32_t* vpidx;       // A^2 value policy (value_protect > 0): indices per group block
  const uint16_t* vprot;       //   and [P][d] bf16 corrections per group block
  int value_protect;
  int key_bf16;                // dtype of ktail
  const int32_t* row_len;      // [B] per-row attended tokens (<= n_ctx), or null (all n_ctx)
  CacheMap map;
  float* logits_dbg;           // may be null
  uint32_t* ws_count;          // [B][Hkv] arrival counters (zero between calls)
  float* ws_o;                 // [B][Hq][S][d]
  float* ws_ml;                // [B][Hq][S][2]
  void* out;
};

struct DiagArgs {
  int d, r, hq, hkv, batch, gqa;
  int64_t cap, n_ctx;
  int n_splits;                // workgroups per (b, h); 4 waves each, 64-token chunks per wave
  int key_bf16, value_bf16, value_mode, query_bf16;
  int key_nib;                 // 3- or 4-bit base codes (one per nibble)
  double kappa;                // scale of the side correction in s_hat
  const void* q;
  const void* k_ref;           // reference keys (key dtype), element strides below
  int64_t ks_b, ks_h, ks_t;
  const void* v_ref;           // reference values (value dtype) or null: no A^2
  int64_t vs_b, vs_h, vs_t;
  const uint8_t* kcode;
  const uint16_t* kmeta;
  const uint8_t* scode;
  const uint16_t* ssc;
  const void* vdense;
  const uint8_t* vcode;
  const uint16_t* vmeta;
  const float* U;
  const void* ktail;
  const void* vtail;
  const uint32_t* vpidx;       // A^2 value policy (value_protect > 0): indices per group block
  const uint16_t* vprot;       //   and [P][d] bf16 corrections per group block
  int value_protect;
  CacheMap map;
  double* ws_q;                // [B][Hkv][padded g][d]   queries in f64 (zero rows past g)
  double* ws_qu;               // [B][Hkv][padded g][max(r, 1)]   U_h^T q in f64
  double* ws_part;             // [B][Hq][S][8]   split partials (max, six sums, max |ds|)
  double* ws_dv2;              // [B][Hkv][n_ctx]   |v_hat_j - v_j|^2 (with reference values)
  double* stats;               // [B][Hq][HEADQ_DIAG_NSTAT]
};

constexpr int kDiagPart = 8;        // doubles per split partial
constexpr int kDiagHeadBatch = 4;   // query heads per pass of the diagnostics stream kernel
__host__ __device__ constexpr int diag_padded_heads(int g) {
  return (g + kDiagHeadBatch - 1) / kDiagHeadBatch * kDiagHeadBatch;
}
// Workspace: queries [B][Hkv][padded g][d] and U_h^T q [B][Hkv][padded g][max(r, 1)] (f64), split
// partials [B][Hq][S][8], per-token value errors [B][Hkv][n_ctx].
inline size_t diag_ws_q_doubles(int batch, int hkv, int g, int d) {
  return (size_t)batch * hkv * diag_padded_heads(g) * d;
}
inline size_t diag_ws_qu_doubles(int batch, int hkv, int g, int r) {
  return (size_t)batch * hkv * diag_padded_heads(g) * (r > 0 ? r : 1);
}
inline size_t diag_ws_bytes(int batch, int hq, int hkv, int d, int r, int n_splits, int64_t n_ctx) {
  const int g = hq / hkv;
  return (diag_ws_q_doubles(batch, hkv, g, d) + diag_ws_qu_doubles(batch, hkv, g, r) +
          (size_t)batch * hq * n_splits * kDiagPart + (size_t)batch * hkv * (size_t)n_ctx) * sizeof(double);
}

struct PrefillArgs {
  int d, r, hq, hkv, batch, gqa;
  int64_t cap;
  int64_t start, n_q;          // query token t sits at position start + t; the cache holds
                               // tokens [0, start + n_q) (whole groups, the rest in the tails)
  int query_bf16, key_bf16, value_bf16, value_mode, out_bf16;
  int key_nib;                 // 3- or 4-bit base codes (one per nibble)
  float corr_scale;
  const void* q;               // [B][n_q][Hq][d]
  const uint8_t* kcode;
  const uint16_t* kmeta;
  const uint8_t* scode;
  const uint16_t* ssc;
  const void* vdense;
  const uint8_t* vcode;
  const uint16_t* vmeta;
  const float* U;
  const void* ktail;
  const void* vtail;
  const uint32_t* vpidx;       // A^2 value policy (value_protect > 0): indices per group block
  const uint16_t* vprot;       //   and [P][d] bf16 corrections per group block
  int value_protect;
  CacheMap map;
  float* logits_dbg;           // [B][n_q][Hq][start + n_q] or null
  void* out;                   // [B][n_q][Hq][d]
};

// Workspace of a decode: per-(b, h) arrival counters (rounded up to 256 bytes), then the split
// partials (unnormalised outputs, then running max and sum).
inline size_t decode_ws_counter_bytes(int batch, int hkv) {
  return ((size_t)batch * hkv * sizeof(uint32_t) + 255) / 256 * 256;
}
inline size_t decode_ws_bytes(int batch, int hq, int hkv, int d, int n_splits) {
  return decode_ws_counter_bytes(batch, hkv) + (size_t)batch * hq * n_splits * (size_t)(d + 2) * sizeof(float);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_mfma_split(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_diagnostics(const DiagArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// Host eigensolver used by headq_calibrate (fp64, symmetric). Returns false on non-convergence.
bool symmetric_eigen(int n, double* A, double* eigenvalues, double* eigenvectors);

}  // namespace headq
