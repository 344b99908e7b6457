/*
 * headq_oracle.h — C API of the CPU oracle for the HeadQ key-side KV cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library may include, link or call this.
 * Only the test suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 *
 * The oracle is written from the HeadQ description ("HeadQ: Model-Visible Distortion and
 * Score-Space Correction for KV-Cache Quantization"; the Dutch technical summary
 * "Technische Samenvatting", §3 "Algorithmisch Overzicht") and from the cache format that this
 * repository defines. It shares no code with the GPU library.
 *
 * Conventions shared by every function:
 *   - Half-precision numbers travel as their IEEE binary16 bit patterns (uint16_t), bfloat16 too.
 *   - Arrays are dense, row-major, in the shapes named in each comment.
 *   - Return value 0 = success, negative = invalid argument (the oracle never guesses).
 */
#ifndef HEADQ_ORACLE_H
#define HEADQ_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE-754 conversions (round to nearest, ties to even), written from the format definitions. */
uint16_t orc_f32_to_f16(float x);
float orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float x);
float orc_bf16_to_f32(uint16_t h);
void orc_f32_to_f16_array(const float* x, uint16_t* h, int64_t n);
void orc_f16_to_f32_array(const uint16_t* h, float* x, int64_t n);
void orc_f32_to_bf16_array(const float* x, uint16_t* h, int64_t n);

/* Calibration (summary §3 step 1): per KV head h, PCA of the pooled post-RoPE calibration queries
 * of the g = hq/hkv query heads that read it. Uncentered second moment, fp64 cyclic Jacobi.
 *   q_cal: f32 [hq][n_cal][d]   U: f32 [hkv][d][r] (out)   eig: f64 [hkv][r] (out, nullable)
 *   centered != 0 subtracts the pooled mean first (a variant, not the default reading). */
int orc_calibrate(int d, int hq, int hkv, int64_t n_cal, int r, int centered, const float* q_cal,
                  float* U, double* eig);

/* Key encode of one (batch, KV-head) stream of T tokens, T a multiple of 32 (summary §3 step 2),
 * in the kernel's f32 precision so that every integer decision matches bit for bit:
 *   k:     f32 [T][d]          keys (bf16 keys are widened exactly by the caller)
 *   U:     f32 [d][r]          side basis (ignored when r == 0)
 *   codes: u8  [T][d]          base codes 0..2^bits-1 (out)
 *   scale, zero: fp16 [T/32][d] per-(group, channel) step and offset (out)
 *   zc:    i8  [T][r]          side codes in -(2^(sb-1)-1) .. 2^(sb-1)-1 (out)
 *   sigma: fp16 [T]            per-token side step (out)
 *   resid: f32 [T][d]          residual e = k - k_base (out, nullable)
 *   proj:  f32 [T][r]          y = U^T e (out, nullable) */
int orc_encode_keys(int d, int r, int bits, int side_bits, int64_t T, const float* k, const float* U,
                    uint8_t* codes, uint16_t* scale, uint16_t* zero, int8_t* zc, uint16_t* sigma,
                    float* resid, float* proj);

/* Value 2-bit quantizer for one stream (full-KV composition): per token, per 32-channel group,
 * asymmetric min/max with the same numerics as the key base quantizer.
 *   v: f32 [T][d]   codes: u8 [T][d] (out)   scale, zero: fp16 [T][d/32] (out) */
int orc_quantize_values(int d, int bits, int64_t T, const float* v, uint8_t* codes, uint16_t* scale,
                        uint16_t* zero);

/* A^2 value policy (definition in headq_oracle.c): c2 = 2 log2(e) / sqrt(d) in f32; the mean
 * calibration query per KV head; the per-group choice of P corrected tokens and their bfloat16
 * corrections. */
float orc_policy_scale(int d);
int orc_mean_query(int d, int hq, int hkv, int64_t n_cal, const float* q_cal, float* a);
int orc_value_policy(int d, int P, int64_t T, const float* k, const float* v, const float* a,
                     const uint8_t* codes, const uint16_t* scale, const uint16_t* zero, uint8_t* idx,
                     uint16_t* delta, double* prio);

/* Packing into the cache format (one stream; offsets for (b, h) are the caller's).
 *   kcode [T][d/4] (d % 16 == 0): d/16 little-endian 32-bit words per token; channel 16m + j with
 *         j = 8q + 2b + e lies in word m, byte b, bits 4e + 2q (so masking a word with 0x33333333
 *         leaves channels 16m..16m+7 and the word shifted right by 2 leaves 16m+8..16m+15, two
 *         channels per byte in ascending order, one per nibble)
 *   kmeta [T/32][2][d]: row 0 = scale, row 1 = zero (fp16)
 *   scode [T][r/2]: byte i/2 holds (zc_i + 8) in the low nibble for even i, high nibble for odd i
 *   vdense [T/32][d][32]: element (token t, channel c) at group t/32, offset c*32 + t%32
 *   vcode [T/32][d*8] (d % 16 == 0): per group, lane l = 16*(t%32 / 8) + c%16 owns bytes
 *         [l*d/8, (l+1)*d/8), two per 16-channel tile c/16; token item i = t%8 = 4q + 2b + e lies
 *         in byte b of the tile's pair at bits 4e + 2q
 *   vmeta [T/32][2][d/32][32]: row 0 = scale, row 1 = zero, token-minor */
int orc_pack_kcode(int d, int64_t T, const uint8_t* codes, uint8_t* kcode);
/*   kcode4 [T][d/2] (d % 8 == 0), 3- and 4-bit base codes one per nibble: d/8 little-endian words
 *         per token; channel 8m + j in word m at bit 4*(j/2) + 16*(j%2) */
int orc_pack_kcode4(int d, int64_t T, const uint8_t* codes, uint8_t* kcode);
int orc_pack_kmeta(int d, int64_t T, const uint16_t* scale, const uint16_t* zero, uint16_t* kmeta);
int orc_pack_scode(int r, int64_t T, const int8_t* zc, uint8_t* scode);
int orc_pack_vdense(int d, int64_t T, int elem_bytes, const void* v, void* vdense);
int orc_pack_vcode(int d, int64_t T, const uint8_t* codes, uint8_t* vcode);
int orc_pack_vmeta(int d, int64_t T, const uint16_t* scale, const uint16_t* zero, uint16_t* vmeta);

/* Decode attention (summary §3 step 3 and §1/§2.2 readout) in fp64 from the packed cache.
 * Every (b, hq) with b in [b_begin, b_end): query head hq reads KV head hq / (hq_total / hkv).
 *   value_mode 0 = dense (value_dtype 0 = f32, 1 = bf16), 1 = 2-bit (vcode/vmeta)
 *   q: f32 [B][hq][d]  U: f32 [hkv][d][r]
 *   logits: f64 [B][hq][n_ctx] natural-log units (nullable)   out: f64 [B][hq][d]
 * Cache buffers are laid out [B][hkv][cap ...] as in the packing comments above. Tokens past the
 * last whole group (n_ctx % 32 of them) come from the dense tails ktail / vtail [B][hkv][32][d]
 * (row t % 32; f32, or bfloat16 bits when the dtype is 1) with exact keys and values: no base
 * code, no side code. The tails may be NULL when n_ctx is a multiple of 32. base_bits (2, 3 or 4)
 * selects the key-code packing: 2-bit words, or one code per nibble for 3 and 4 bits. n_prot > 0
 * (2-bit values only): the A^2 value policy's corrections, vpidx u8 [B][hkv][cap/32][4] and vprot
 * bf16 bits [B][hkv][cap/32][n_prot][d], added to the values of the tokens they name. */
int orc_decode(int d, int hq, int hkv, int r, int value_mode, int value_dtype, int B, int64_t cap,
               int64_t n_ctx, const uint8_t* kcode, const uint16_t* kmeta, const uint8_t* scode,
               const uint16_t* ssc, const void* vdense, const uint8_t* vcode, const uint16_t* vmeta,
               int key_dtype, const void* ktail, const void* vtail, const float* U, const float* q, double kappa,
               int b_begin, int b_end, double* logits, double* out, int base_bits, int n_prot,
               const uint8_t* vpidx, const uint16_t* vprot);

/* Value rows of stream (b, h) as the cache holds them, in fp64: out [n_ctx][d] (dense values as
 * stored, 2-bit values as code * s + z plus the policy's corrections, tokens past the last whole
 * group from vtail). Cache buffers as for orc_decode. */
int orc_value_rows(int d, int value_mode, int value_dtype, int hkv, int64_t cap, int64_t n_ctx,
                   const void* vdense, const uint8_t* vcode, const uint16_t* vmeta, const void* vtail, int b,
                   int h, double* out, int n_prot, const uint8_t* vpidx, const uint16_t* vprot);

#ifdef __cplusplus
}
#endif
#endif
