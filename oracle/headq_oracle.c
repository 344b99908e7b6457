/*
 * headq_oracle.c — plain, slow CPU oracle for the HeadQ key-side KV cache.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU-baseline leg of the
 * benchmark. The product library never includes or links it, and it shares no code with it.
 *
 * Sources (cited by page and section; the pages carry no code):
 *   [ABS]  "HeadQ: Model-Visible Distortion and Score-Space Correction for KV-Cache Quantization",
 *          abstract: key-side method, low-rank residual side code in a calibration-learned query
 *          basis, applied as an additive logit correction.
 *   [TS]   "Technische Samenvatting: HeadQ ..." (Dutch technical summary):
 *          §1 (readout sum p_j v_j), §2.1 (score perturbation, softmax-null shifts),
 *          §2.2 (value readout error), §3 "Algorithmisch Overzicht" steps 1-3.
 * Where the pages leave a step open, the reading is named inline ("reading: ...").
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared -lm
 * (no contraction: every fused multiply-add below is an explicit fmaf()).
 */
#include "headq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 32

/* ------------------------------------------------------------------------------------------ */
/* IEEE conversions, from the binary16 / bfloat16 definitions (round to nearest, ties to even). */

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* Round the non-negative integer `sig` right by `shift` bits, ties to even. */
static uint32_t shift_rne(uint32_t sig, int shift) {
  if (shift <= 0) return sig << (-shift);
  if (shift >= 32) return 0;
  uint32_t q = sig >> shift;
  uint32_t rem = sig & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1u;
  return q;
}

uint16_t orc_f32_to_f16(float x) {
  uint32_t u = f32_bits(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t e = (u >> 23) & 0xffu, m = u & 0x7fffffu;
  if (e == 0xffu) return (uint16_t)(sign | (m ? 0x7e00u : 0x7c00u)); /* NaN stays NaN (quiet) */
  if (e == 0 && m == 0) return sign;
  /* value = sig * 2^(exp2) with sig an integer */
  uint32_t sig = e ? (m | 0x800000u) : m;
  int exp2 = (e ? (int)e : 1) - 150;
  /* binary16 normal numbers: 2^-14 <= |x|; significand 11 bits; subnormal quantum 2^-24 */
  /* Try the normal path first: find the half exponent E with 2^E <= |x| < 2^(E+1). */
  int top = 31 - __builtin_clz(sig); /* position of leading one */
  int E = top + exp2;                /* floor(log2|x|) */
  if (E >= -14) {
    /* keep 11 significant bits: quantum 2^(E-10) */
    uint32_t q = shift_rne(sig, (E - 10) - exp2);
    /* q in [2^10, 2^11]; q == 2^11 means rounding carried into the next binade */
    if (q == 0x800u) { q = 0x400u; E += 1; }
    if (E > 15) return (uint16_t)(sign | 0x7c00u); /* overflow to infinity */
    return (uint16_t)(sign | ((uint32_t)(E + 15) << 10) | (q & 0x3ffu));
  }
  /* subnormal: quantum 2^-24 (the result may round up to the smallest normal, 0x0400) */
  uint32_t q = shift_rne(sig, -24 - exp2);
  return (uint16_t)(sign | q);
}

float orc_f16_to_f32(uint16_t h) {
  uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  if (e == 0x1fu) return bits_f32(sign | 0x7f800000u | (m << 13));
  if (e == 0) {
    /* zero or subnormal: m * 2^-24, exactly representable in binary32 */
    float v = (float)m * 0x1p-24f;
    return sign ? -v : v;
  }
  return bits_f32(sign | ((e + 112u) << 23) | (m << 13));
}

uint16_t orc_f32_to_bf16(float x) {
  uint32_t u = f32_bits(x);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t keep = u >> 16, rem = u & 0xffffu;
  if (rem > 0x8000u || (rem == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

float orc_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

void orc_f32_to_f16_array(const float* x, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = orc_f32_to_f16(x[i]);
}
void orc_f16_to_f32_array(const uint16_t* h, float* x, int64_t n) {
  for (int64_t i = 0; i < n; ++i) x[i] = orc_f16_to_f32(h[i]);
}
void orc_f32_to_bf16_array(const float* x, uint16_t* h, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = orc_f32_to_bf16(x[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* Calibration: [TS] §3 step 1 — a rank-r basis U_h per layer and head from PCA of post-RoPE
 * calibration queries. Readings: one basis per KV head, pooling the query heads that read it;
 * uncentered second moment E[q q^T] (the score error is q^T e with the raw query); eigenvectors
 * sorted by decreasing eigenvalue; each column signed so that its largest-magnitude entry (lowest
 * index on ties) is positive. */

/* Cyclic Jacobi eigen-decomposition of a symmetric n x n matrix A (destroyed). V receives the
 * eigenvectors as columns, w the eigenvalues. */
static void jacobi_eig(int n, double* A, double* V, double* w) {
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) V[i * n + j] = (i == j) ? 1.0 : 0.0;
  double total = 0.0;
  for (int i = 0; i < n * n; ++i) total += A[i] * A[i];
  for (int sweep = 0; sweep < 100; ++sweep) {
    double off = 0.0;
    for (int p = 0; p < n; ++p)
      for (int q = p + 1; q < n; ++q) off += A[p * n + q] * A[p * n + q];
    if (off <= 1e-30 * total || off == 0.0) break;
    for (int p = 0; p < n; ++p) {
      for (int q = p + 1; q < n; ++q) {
        double apq = A[p * n + q];
        if (apq == 0.0) continue;
        /* choose the rotation that annihilates A[p][q] */
        double theta = (A[q * n + q] - A[p * n + p]) / (2.0 * apq);
        double t = (theta >= 0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
        double c = 1.0 / sqrt(t * t + 1.0), s = t * c;
        for (int k = 0; k < n; ++k) { /* columns p, q */
          double akp = A[k * n + p], akq = A[k * n + q];
          A[k * n + p] = c * akp - s * akq;
          A[k * n + q] = s * akp + c * akq;
        }
        for (int k = 0; k < n; ++k) { /* rows p, q */
          double apk = A[p * n + k], aqk = A[q * n + k];
          A[p * n + k] = c * apk - s * aqk;
          A[q * n + k] = s * apk + c * aqk;
        }
        for (int k = 0; k < n; ++k) {
          double vkp = V[k * n + p], vkq = V[k * n + q];
          V[k * n + p] = c * vkp - s * vkq;
          V[k * n + q] = s * vkp + c * vkq;
        }
      }
    }
  }
  for (int i = 0; i < n; ++i) w[i] = A[i * n + i];
}

int orc_calibrate(int d, int hq, int hkv, int64_t n_cal, int r, int centered, const float* q_cal,
                  float* U, double* eig) {
  if (d <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || n_cal <= 0 || r < 0 || r > d || !q_cal || (r && !U))
    return -1;
  int g = hq / hkv;
  double* M = (double*)calloc((size_t)d * d, sizeof(double));
  double* V = (double*)malloc((size_t)d * d * sizeof(double));
  double* w = (double*)malloc((size_t)d * sizeof(double));
  double* mean = (double*)calloc((size_t)d, sizeof(double));
  int* order = (int*)malloc((size_t)d * sizeof(int));
  if (!M || !V || !w || !mean || !order) { free(M); free(V); free(w); free(mean); free(order); return -2; }
  for (int h = 0; h < hkv; ++h) {
    memset(M, 0, (size_t)d * d * sizeof(double));
    memset(mean, 0, (size_t)d * sizeof(double));
    double rows = (double)g * (double)n_cal;
    if (centered) {
      for (int a = h * g; a < (h + 1) * g; ++a)
        for (int64_t n = 0; n < n_cal; ++n)
          for (int i = 0; i < d; ++i) mean[i] += q_cal[((int64_t)a * n_cal + n) * d + i];
      for (int i = 0; i < d; ++i) mean[i] /= rows;
    }
    for (int a = h * g; a < (h + 1) * g; ++a)
      for (int64_t n = 0; n < n_cal; ++n) {
        const float* x = q_cal + ((int64_t)a * n_cal + n) * d;
        for (int i = 0; i < d; ++i)
          for (int j = 0; j < d; ++j) M[i * d + j] += ((double)x[i] - mean[i]) * ((double)x[j] - mean[j]);
      }
    for (int i = 0; i < d * d; ++i) M[i] /= rows;
    jacobi_eig(d, M, V, w);
    /* sort indices by decreasing eigenvalue (stable: lower index first on equal values) */
    for (int i = 0; i < d; ++i) order[i] = i;
    for (int i = 1; i < d; ++i) {
      int cur = order[i], j = i - 1;
      while (j >= 0 && w[order[j]] < w[cur]) { order[j + 1] = order[j]; --j; }
      order[j + 1] = cur;
    }
    for (int col = 0; col < r; ++col) {
      int src = order[col];
      int arg = 0;
      double best = -1.0;
      for (int i = 0; i < d; ++i) {
        double a = fabs(V[i * d + src]);
        if (a > best) { best = a; arg = i; }
      }
      double sgn = V[arg * d + src] < 0 ? -1.0 : 1.0;
      for (int i = 0; i < d; ++i) U[((int64_t)h * d + i) * r + col] = (float)(sgn * V[i * d + src]);
      if (eig) eig[(int64_t)h * r + col] = w[src];
    }
  }
  free(M); free(V); free(w); free(mean); free(order);
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Base quantizer B_b ([TS] §3 step 2, first bullet; KIVI-like per-channel asymmetric min/max
 * over groups of 32 tokens). Readings: scale and zero are stored in binary16 (round to nearest
 * even) and every code is taken against the stored grid; codes = clamp(rint((k - z)/s)) with the
 * quotient taken as (k - z) * (1/s) in f32 and 1/s = 0 when s == 0. */
static void minmax_grid(const float* x, int n, int stride, int levels, float* s_out, float* z_out,
                        uint16_t* s_bits, uint16_t* z_bits) {
  float lo = x[0], hi = x[0];
  for (int t = 1; t < n; ++t) {
    float v = x[(int64_t)t * stride];
    if (v < lo) lo = v;
    if (v > hi) hi = v;
  }
  float s = (hi - lo) / (float)levels;
  *s_bits = orc_f32_to_f16(s);
  *z_bits = orc_f32_to_f16(lo);
  *s_out = orc_f16_to_f32(*s_bits);
  *z_out = orc_f16_to_f32(*z_bits);
}

static int quant_code(float x, float s, float z, int levels) {
  float inv = (s == 0.0f) ? 0.0f : 1.0f / s;
  float c = nearbyintf((x - z) * inv);
  if (c < 0.0f) c = 0.0f;
  if (c > (float)levels) c = (float)levels;
  return (int)c;
}

int orc_encode_keys(int d, int r, int bits, int side_bits, int64_t T, const float* k, const float* U,
                    uint8_t* codes, uint16_t* scale, uint16_t* zero, int8_t* zc, uint16_t* sigma,
                    float* resid, float* proj) {
  if (d <= 0 || r < 0 || bits < 1 || bits > 8 || side_bits < 2 || side_bits > 8 || T <= 0 || T % GROUP ||
      !k || !codes || !scale || !zero || !sigma || (r && (!U || !zc)))
    return -1;
  const int levels = (1 << bits) - 1;
  const int zmax = (1 << (side_bits - 1)) - 1;
  float* e = (float*)malloc((size_t)d * sizeof(float));
  float* y = (float*)malloc((size_t)(r ? r : 1) * sizeof(float));
  float* s_f = (float*)malloc((size_t)d * sizeof(float));
  float* z_f = (float*)malloc((size_t)d * sizeof(float));
  if (!e || !y || !s_f || !z_f) { free(e); free(y); free(s_f); free(z_f); return -2; }
  for (int64_t g0 = 0; g0 < T; g0 += GROUP) {
    int64_t gi = g0 / GROUP;
    for (int c = 0; c < d; ++c)
      minmax_grid(k + g0 * d + c, GROUP, d, levels, &s_f[c], &z_f[c], &scale[gi * d + c], &zero[gi * d + c]);
    for (int64_t t = g0; t < g0 + GROUP; ++t) {
      const float* kt = k + t * d;
      /* B_b(k_j) and the residual e_j = k_j - k_base_j ([TS] §3 step 2, second bullet).
         Reading: the residual is taken against the stored grid with one fused multiply-add. */
      for (int c = 0; c < d; ++c) {
        int code = quant_code(kt[c], s_f[c], z_f[c], levels);
        codes[t * d + c] = (uint8_t)code;
        e[c] = kt[c] - fmaf((float)code, s_f[c], z_f[c]);
        if (resid) resid[t * d + c] = e[c];
      }
      /* y = U_h^T e_j ([TS] §3 step 2, third bullet). Reading: one f32 fused-multiply-add chain
         per component over channels 0..d-1 in order, starting from +0. */
      float amax = 0.0f;
      for (int i = 0; i < r; ++i) {
        float acc = 0.0f;
        for (int c = 0; c < d; ++c) acc = fmaf(U[(int64_t)c * r + i], e[c], acc);
        y[i] = acc;
        if (proj) proj[t * r + i] = acc;
        float a = fabsf(acc);
        if (a > amax) amax = a;
      }
      /* Q_q: low-bit side quantizer, symmetric, one scale per token. Readings: levels
         -zmax..zmax, scale = max|y| / zmax stored in binary16, codes taken against the stored
         scale, all codes 0 when the scale is 0. */
      uint16_t sb = orc_f32_to_f16(amax / (float)zmax);
      float sg = orc_f16_to_f32(sb);
      sigma[t] = sb;
      float inv = (sg == 0.0f) ? 0.0f : 1.0f / sg;
      for (int i = 0; i < r; ++i) {
        float q = nearbyintf(y[i] * inv);
        if (q < (float)-zmax) q = (float)-zmax;
        if (q > (float)zmax) q = (float)zmax;
        zc[t * r + i] = (int8_t)q;
      }
    }
  }
  free(e); free(y); free(s_f); free(z_f);
  return 0;
}

/* Value quantizer for the full-KV composition (abstract: HeadQ keys composed with a 2-bit value
 * cache). Reading: the plain per-token asymmetric min/max quantizer over groups of 32 channels,
 * with the same numerics as the key base quantizer; no value policy. */
int orc_quantize_values(int d, int bits, int64_t T, const float* v, uint8_t* codes, uint16_t* scale,
                        uint16_t* zero) {
  if (d <= 0 || d % GROUP || bits < 1 || bits > 8 || T <= 0 || !v || !codes || !scale || !zero) return -1;
  const int levels = (1 << bits) - 1;
  const int ng = d / GROUP;
  for (int64_t t = 0; t < T; ++t)
    for (int g = 0; g < ng; ++g) {
      float s, z;
      const float* x = v + t * d + g * GROUP;
      minmax_grid(x, GROUP, 1, levels, &s, &z, &scale[t * ng + g], &zero[t * ng + g]);
      for (int c = 0; c < GROUP; ++c) codes[t * d + g * GROUP + c] = (uint8_t)quant_code(x[c], s, z, levels);
    }
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* A^2 value policy ([TS] §2.2: values are read through the weighted sum, and their error is
 * measured by the A^2 surrogate sum_j p_j^2 |v_hat_j - v_j|^2; §5: the full-KV composition pairs
 * HeadQ keys with an A^2-weighted value policy). The pages define the surrogate, not the policy.
 * Reading: every token keeps its 2-bit value codes; per 32-token group, P of them also keep a
 * correction delta_j = v_j - v_hat_j in bfloat16 (the decoded value is then v_hat_j + delta_j):
 * the P tokens with the largest estimated reduction of the surrogate, w_j * e_j, where
 *   e_j = |v_j - v_hat_j|^2, v_hat = fma(code, s, z) per channel, summed by one f32 fma chain
 *         over channels 0..d-1 from +0;
 *   w_j = 2^n_j, n_j = clamp(rint(c2 * (a_h . k_j)), -64, 64): a power-of-two estimate of
 *         exp(2 a_h.k_j / sqrt(d)), to which E[p_j^2] is proportional within a group at first
 *         order in the query, a_h the mean post-RoPE calibration query of the KV head, a_h . k_j
 *         one f32 fma chain over channels 0..d-1 from +0, c2 = 2 log2(e) / sqrt(d) rounded to f32;
 *   w_j * e_j compared exactly (in double); ties go to the lower token index.
 * The chosen tokens fill the P slots in ascending token order. */
float orc_policy_scale(int d) { return (float)(2.0 * 1.4426950408889634 / sqrt((double)d)); }

/* Mean calibration query per KV head (the direction a_h above): f64 sums over the g query heads
 * of the KV head (in head order) and their n_cal queries (in order), divided by g * n_cal, rounded
 * to f32. q_cal: f32 [Hq][n_cal][d]; a: f32 [Hkv][d]. */
int orc_mean_query(int d, int hq, int hkv, int64_t n_cal, const float* q_cal, float* a) {
  if (d <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || n_cal <= 0 || !q_cal || !a) return -1;
  const int g = hq / hkv;
  for (int h = 0; h < hkv; ++h)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int hh = h * g; hh < (h + 1) * g; ++hh)
        for (int64_t n = 0; n < n_cal; ++n) acc += (double)q_cal[((int64_t)hh * n_cal + n) * d + c];
      a[(int64_t)h * d + c] = (float)(acc / ((double)g * (double)n_cal));
    }
  return 0;
}

/* The policy over whole groups of one stream. k, v: f32 [T][d] (keys and values as written);
 * a: f32 [d]; codes/scale/zero: the 2-bit value quantizer's output for v. Writes idx u8 [T/32][4]
 * (slot i < P: token index in the group; the other bytes 0) and delta bf16 bits [T/32][P][d];
 * prio (optional, f64 [T]): w_j * e_j. */
int orc_value_policy(int d, int P, int64_t T, const float* k, const float* v, const float* a,
                     const uint8_t* codes, const uint16_t* scale, const uint16_t* zero, uint8_t* idx,
                     uint16_t* delta, double* prio) {
  if (d <= 0 || d % GROUP || P < 1 || P > 4 || T <= 0 || T % GROUP || !k || !v || !a || !codes || !scale ||
      !zero || !idx || !delta)
    return -1;
  const int ng = d / GROUP;
  const float c2 = orc_policy_scale(d);
  double pr[GROUP];
  for (int64_t g0 = 0; g0 < T; g0 += GROUP) {
    const int64_t gi = g0 / GROUP;
    for (int t = 0; t < GROUP; ++t) {
      const int64_t row = g0 + t;
      float dot = 0.0f, e = 0.0f;
      for (int c = 0; c < d; ++c) dot = fmaf(a[c], k[row * d + c], dot);
      for (int c = 0; c < d; ++c) {
        const float s = orc_f16_to_f32(scale[row * ng + c / GROUP]);
        const float z = orc_f16_to_f32(zero[row * ng + c / GROUP]);
        const float diff = v[row * d + c] - fmaf((float)codes[row * d + c], s, z);
        e = fmaf(diff, diff, e);
      }
      float nf = nearbyintf(dot * c2);
      if (nf < -64.0f) nf = -64.0f;
      if (nf > 64.0f) nf = 64.0f;
      pr[t] = ldexp((double)e, (int)nf);
      if (prio) prio[row] = pr[t];
    }
    int slot = 0;
    for (int i = 0; i < 4; ++i) idx[gi * 4 + i] = 0;
    for (int t = 0; t < GROUP; ++t) {
      int rank = 0;
      for (int u = 0; u < GROUP; ++u)
        if (pr[u] > pr[t] || (pr[u] == pr[t] && u < t)) ++rank;
      if (rank >= P) continue;
      idx[gi * 4 + slot] = (uint8_t)t;
      const int64_t row = g0 + t;
      for (int c = 0; c < d; ++c) {
        const float s = orc_f16_to_f32(scale[row * ng + c / GROUP]);
        const float z = orc_f16_to_f32(zero[row * ng + c / GROUP]);
        delta[(gi * P + slot) * d + c] = orc_f32_to_bf16(v[row * d + c] - fmaf((float)codes[row * d + c], s, z));
      }
      ++slot;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Packing into the cache format (byte layouts are this repository's convention). */

/* Bit position of channel 16m + j inside the 32-bit little-endian word m of a token's key codes:
 * j = 8q + 2b + e sits in byte b at bit 4e + 2q. */
static int kcode_bit(int j) { return 8 * ((j % 8) / 2) + 4 * (j % 2) + 2 * (j / 8); }

int orc_pack_kcode(int d, int64_t T, const uint8_t* codes, uint8_t* kcode) {
  if (d % 16 || !codes || !kcode) return -1;
  for (int64_t t = 0; t < T; ++t)
    for (int m = 0; m < d / 16; ++m) {
      uint32_t word = 0;
      for (int j = 0; j < 16; ++j) word |= (uint32_t)(codes[t * d + 16 * m + j] & 3u) << kcode_bit(j);
      for (int k = 0; k < 4; ++k) kcode[t * (d / 4) + 4 * m + k] = (uint8_t)(word >> (8 * k));
    }
  return 0;
}

/* 3- and 4-bit base codes, one per nibble: a token row is d/2 bytes, d/8 little-endian words;
 * channel 8m + j sits in word m at bit 4*(j/2) + 16*(j%2) (channels 2i and 2i+1 at the same
 * nibble of the low and the high 16-bit half). */
static int kcode4_bit(int j) { return 4 * (j / 2) + 16 * (j % 2); }

int orc_pack_kcode4(int d, int64_t T, const uint8_t* codes, uint8_t* kcode) {
  if (d % 8 || !codes || !kcode) return -1;
  for (int64_t t = 0; t < T; ++t)
    for (int m = 0; m < d / 8; ++m) {
      uint32_t word = 0;
      for (int j = 0; j < 8; ++j) word |= (uint32_t)(codes[t * d + 8 * m + j] & 15u) << kcode4_bit(j);
      for (int k = 0; k < 4; ++k) kcode[t * (d / 2) + 4 * m + k] = (uint8_t)(word >> (8 * k));
    }
  return 0;
}

int orc_pack_kmeta(int d, int64_t T, const uint16_t* scale, const uint16_t* zero, uint16_t* kmeta) {
  if (T % GROUP || !scale || !zero || !kmeta) return -1;
  for (int64_t g = 0; g < T / GROUP; ++g)
    for (int c = 0; c < d; ++c) {
      kmeta[(g * 2 + 0) * d + c] = scale[g * d + c];
      kmeta[(g * 2 + 1) * d + c] = zero[g * d + c];
    }
  return 0;
}

int orc_pack_scode(int r, int64_t T, const int8_t* zc, uint8_t* scode) {
  if (r % 2 || (r && (!zc || !scode))) return -1;
  for (int64_t t = 0; t < T; ++t)
    for (int i = 0; i < r; i += 2) {
      unsigned lo = (unsigned)(zc[t * r + i] + 8) & 0xfu;
      unsigned hi = (unsigned)(zc[t * r + i + 1] + 8) & 0xfu;
      scode[t * (r / 2) + i / 2] = (uint8_t)(lo | (hi << 4));
    }
  return 0;
}

int orc_pack_vdense(int d, int64_t T, int elem_bytes, const void* v, void* vdense) {
  if (T % GROUP || (elem_bytes != 2 && elem_bytes != 4) || !v || !vdense) return -1;
  const uint8_t* src = (const uint8_t*)v;
  uint8_t* dst = (uint8_t*)vdense;
  for (int64_t t = 0; t < T; ++t)
    for (int c = 0; c < d; ++c) {
      int64_t g = t / GROUP, tt = t % GROUP;
      memcpy(dst + ((g * d + c) * GROUP + tt) * elem_bytes, src + (t * d + c) * elem_bytes, (size_t)elem_bytes);
    }
  return 0;
}

/* Byte and bit of (channel c, token tt of its group) inside a group's block of value codes:
 * lane = 16 * (tt / 8) + c % 16 owns d/8 consecutive bytes, two per 16-channel tile c / 16; token
 * item i = tt % 8 = 4q + 2b + e sits in byte b of the tile's pair at bit 4e + 2q. */
static int64_t vcode_byte(int d, int c, int tt) {
  const int lane = 16 * (tt / 8) + c % 16, i = tt % 8;
  return ((int64_t)lane * (d / 16) + c / 16) * 2 + (i % 4) / 2;
}
static int vcode_bit(int tt) {
  const int i = tt % 8;
  return 4 * (i % 2) + 2 * (i / 4);
}

int orc_pack_vcode(int d, int64_t T, const uint8_t* codes, uint8_t* vcode) {
  if (T % GROUP || d % 16 || !codes || !vcode) return -1;
  for (int64_t g = 0; g < T / GROUP; ++g) {
    uint8_t* blk = vcode + g * d * 8;
    memset(blk, 0, (size_t)d * 8);
    for (int tt = 0; tt < GROUP; ++tt)
      for (int c = 0; c < d; ++c)
        blk[vcode_byte(d, c, tt)] |= (uint8_t)((codes[(g * GROUP + tt) * d + c] & 3u) << vcode_bit(tt));
  }
  return 0;
}

int orc_pack_vmeta(int d, int64_t T, const uint16_t* scale, const uint16_t* zero, uint16_t* vmeta) {
  if (T % GROUP || d % GROUP || !scale || !zero || !vmeta) return -1;
  const int ng = d / GROUP;
  for (int64_t t = 0; t < T; ++t)
    for (int gc = 0; gc < ng; ++gc) {
      int64_t g = t / GROUP, tt = t % GROUP;
      vmeta[((g * 2 + 0) * ng + gc) * GROUP + tt] = scale[t * ng + gc];
      vmeta[((g * 2 + 1) * ng + gc) * GROUP + tt] = zero[t * ng + gc];
    }
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Decode in fp64 ([TS] §3 step 3): the corrected logit is q.k_base/sqrt(d) plus
 * q.(U_h z_hat)/sqrt(d); softmax over the cached tokens; readout sum_j p_j v_j ([TS] §1, §2.2).
 * Every quantity is unpacked from the cache bytes here, independently of any writer. Readings:
 * query head hq reads KV head hq / g; every one of the n_ctx cached tokens is attended (no mask);
 * kappa multiplies the correction (1 = HeadQ, 0 = base only, -1 = the wrong-sign control). */

static double k_hat(const uint8_t* kcode_t, const uint16_t* kmeta_g, int d, int c, int base_bits) {
  unsigned code;
  if (base_bits == 2) {
    const int m = c / 16, j = c % 16, bit = kcode_bit(j);
    code = (kcode_t[4 * m + bit / 8] >> (bit % 8)) & 3u;
  } else {  /* 3 or 4 bits, one code per nibble */
    const int m = c / 8, j = c % 8, bit = kcode4_bit(j);
    code = (kcode_t[4 * m + bit / 8] >> (bit % 8)) & 15u;
  }
  double s = orc_f16_to_f32(kmeta_g[c]);
  double z = orc_f16_to_f32(kmeta_g[d + c]);
  return (double)code * s + z;
}

/* The value of token t, channel c of one stream: dense as stored, or 2-bit code * s + z plus the
 * policy's correction when the token holds one of its group's n_prot slots (vpidx u8 [G][4],
 * vprot bf16 bits [G][n_prot][d] of the stream). */
static double v_hat(int value_mode, int value_dtype, const void* vdense, const uint8_t* vcode,
                    const uint16_t* vmeta, int d, int64_t t, int c, int n_prot, const uint8_t* vpidx,
                    const uint16_t* vprot) {
  int64_t g = t / GROUP, tt = t % GROUP;
  if (value_mode == 0) {
    int64_t idx = (g * d + c) * GROUP + tt;
    if (value_dtype == 0) return ((const float*)vdense)[idx];
    return orc_bf16_to_f32(((const uint16_t*)vdense)[idx]);
  }
  const int ng = d / GROUP;
  unsigned code = (vcode[g * d * 8 + vcode_byte(d, c, (int)tt)] >> vcode_bit((int)tt)) & 3u;
  double s = orc_f16_to_f32(vmeta[((g * 2 + 0) * ng + c / GROUP) * GROUP + tt]);
  double z = orc_f16_to_f32(vmeta[((g * 2 + 1) * ng + c / GROUP) * GROUP + tt]);
  double x = (double)code * s + z;
  for (int i = 0; i < n_prot; ++i)
    if (vpidx[g * 4 + i] == tt) x += orc_bf16_to_f32(vprot[(g * n_prot + i) * d + c]);
  return x;
}

/* An element of a dense tail row (f32, or bfloat16 bits when dtype == 1). */
static double tail_at(const void* tail, int dtype, int64_t idx) {
  if (dtype == 0) return ((const float*)tail)[idx];
  return orc_bf16_to_f32(((const uint16_t*)tail)[idx]);
}

int orc_decode(int d, int hq, int hkv, int r, int value_mode, int value_dtype, int B, int64_t cap,
               int64_t n_ctx, const uint8_t* kcode, const uint16_t* kmeta, const uint8_t* scode,
               const uint16_t* ssc, const void* vdense, const uint8_t* vcode, const uint16_t* vmeta,
               int key_dtype, const void* ktail, const void* vtail, const float* U, const float* q, double kappa,
               int b_begin, int b_end, double* logits, double* out, int base_bits, int n_prot,
               const uint8_t* vpidx, const uint16_t* vprot) {
  if (d <= 0 || d % 4 || hq <= 0 || hkv <= 0 || hq % hkv || r < 0 || r % 2 || cap % GROUP || n_ctx <= 0 ||
      n_ctx > cap || b_begin < 0 || b_end > B || b_begin > b_end || !kcode || !kmeta || !q || !out ||
      base_bits < 2 || base_bits > 4 || n_prot < 0 || n_prot > 4 ||
      (n_prot && (value_mode != 1 || !vpidx || !vprot)))
    return -1;
  const int row_bytes = base_bits == 2 ? d / 4 : d / 2;  /* packed key codes per token */
  /* tokens past the last whole group are the stream's dense tail: exact keys and values */
  const int64_t n_full = n_ctx / GROUP * GROUP;
  if (n_full < n_ctx && (!ktail || !vtail)) return -1;
  if (r && (!scode || !ssc || !U)) return -1;
  if (value_mode == 0 && !vdense) return -1;
  if (value_mode == 1 && (!vcode || !vmeta || d % GROUP)) return -1;
  const int g = hq / hkv;
  double* qd = (double*)malloc((size_t)d * sizeof(double));
  double* qu = (double*)malloc((size_t)(r ? r : 1) * sizeof(double));
  double* s = (double*)malloc((size_t)n_ctx * sizeof(double));
  double* o = (double*)malloc((size_t)d * sizeof(double));
  if (!qd || !qu || !s || !o) { free(qd); free(qu); free(s); free(o); return -2; }
  const double inv_sqrt_d = 1.0 / sqrt((double)d);
  for (int b = b_begin; b < b_end; ++b)
    for (int a = 0; a < hq; ++a) {
      const int h = a / g;
      const int64_t bh = (int64_t)b * hkv + h;
      for (int c = 0; c < d; ++c) qd[c] = q[((int64_t)b * hq + a) * d + c];
      /* U_h^T q: the runtime query decodes the side code ([TS] §3 step 3, first bullet) */
      for (int i = 0; i < r; ++i) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)U[((int64_t)h * d + c) * r + i] * qd[c];
        qu[i] = acc;
      }
      double smax = -INFINITY;
      for (int64_t j = n_full; j < n_ctx; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += qd[c] * tail_at(ktail, key_dtype, (bh * GROUP + j % GROUP) * d + c);
        s[j] = dot * inv_sqrt_d;
        if (s[j] > smax) smax = s[j];
      }
      for (int64_t j = 0; j < n_full; ++j) {
        const uint8_t* kt = kcode + (bh * cap + j) * row_bytes;
        const uint16_t* mg = kmeta + (bh * (cap / GROUP) + j / GROUP) * 2 * d;
        double base = 0.0;
        for (int c = 0; c < d; ++c) base += qd[c] * k_hat(kt, mg, d, c, base_bits);
        double corr = 0.0;
        if (r) {
          double sg = orc_f16_to_f32(ssc[bh * cap + j]);
          const uint8_t* st = scode + (bh * cap + j) * (r / 2);
          for (int i = 0; i < r; ++i) {
            int u = (st[i / 2] >> (4 * (i % 2))) & 0xf;
            corr += qu[i] * (sg * (double)(u - 8));
          }
        }
        s[j] = (base + kappa * corr) * inv_sqrt_d;
        if (s[j] > smax) smax = s[j];
      }
      /* per-(b, h) value stream */
      const int vb = (value_dtype == 0) ? 4 : 2;
      const void* vd = vdense ? (const void*)((const uint8_t*)vdense + bh * cap * d * vb) : NULL;
      const uint8_t* vc = vcode ? vcode + bh * (cap / GROUP) * d * 8 : NULL;
      const uint16_t* vm = vmeta ? vmeta + bh * (cap / GROUP) * 2 * d : NULL;
      const uint8_t* pi = n_prot ? vpidx + bh * (cap / GROUP) * 4 : NULL;
      const uint16_t* pv = n_prot ? vprot + bh * (cap / GROUP) * n_prot * d : NULL;
      double l = 0.0;
      for (int64_t j = 0; j < n_ctx; ++j) l += exp(s[j] - smax);
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      for (int64_t j = 0; j < n_ctx; ++j) {
        double p = exp(s[j] - smax) / l;
        if (j >= n_full)
          for (int c = 0; c < d; ++c) o[c] += p * tail_at(vtail, value_dtype, (bh * GROUP + j % GROUP) * d + c);
        else
          for (int c = 0; c < d; ++c)
            o[c] += p * v_hat(value_mode, value_dtype, vd, vc, vm, d, j, c, n_prot, pi, pv);
      }
      for (int c = 0; c < d; ++c) out[((int64_t)b * hq + a) * d + c] = o[c];
      if (logits)
        for (int64_t j = 0; j < n_ctx; ++j) logits[((int64_t)b * hq + a) * n_ctx + j] = s[j];
    }
  free(qd); free(qu); free(s); free(o);
  return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Value rows of one (b, h) stream as the cache holds them, in fp64 ([TS] §2.2: the operands v_j
 * of the readout): dense values as stored, 2-bit values unpacked as code * s + z, and the tokens
 * past the last whole group from the dense tail. out: f64 [n_ctx][d]. */
int orc_value_rows(int d, int value_mode, int value_dtype, int hkv, int64_t cap, int64_t n_ctx,
                   const void* vdense, const uint8_t* vcode, const uint16_t* vmeta, const void* vtail, int b,
                   int h, double* out, int n_prot, const uint8_t* vpidx, const uint16_t* vprot) {
  if (d <= 0 || cap % GROUP || n_ctx < 0 || n_ctx > cap || b < 0 || h < 0 || h >= hkv || !out || n_prot < 0 ||
      n_prot > 4 || (n_prot && (value_mode != 1 || !vpidx || !vprot)))
    return -1;
  const int64_t n_full = n_ctx / GROUP * GROUP;
  if (n_full < n_ctx && !vtail) return -1;
  if (value_mode == 0 && !vdense) return -1;
  if (value_mode == 1 && (!vcode || !vmeta || d % GROUP)) return -1;
  const int64_t bh = (int64_t)b * hkv + h;
  const int vb = (value_dtype == 0) ? 4 : 2;
  const void* vd = vdense ? (const void*)((const uint8_t*)vdense + bh * cap * d * vb) : NULL;
  const uint8_t* vc = vcode ? vcode + bh * (cap / GROUP) * d * 8 : NULL;
  const uint16_t* vm = vmeta ? vmeta + bh * (cap / GROUP) * 2 * d : NULL;
  const uint8_t* pi = n_prot ? vpidx + bh * (cap / GROUP) * 4 : NULL;
  const uint16_t* pv = n_prot ? vprot + bh * (cap / GROUP) * n_prot * d : NULL;
  for (int64_t j = 0; j < n_ctx; ++j)
    for (int c = 0; c < d; ++c)
      out[j * d + c] = j >= n_full ? tail_at(vtail, value_dtype, (bh * GROUP + j % GROUP) * d + c)
                                   : v_hat(value_mode, value_dtype, vd, vc, vm, d, j, c, n_prot, pi, pv);
  return 0;
}

