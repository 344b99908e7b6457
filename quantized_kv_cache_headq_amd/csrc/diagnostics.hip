// diagnostics.hip — headq_score_diagnostics on gfx950: score-space diagnostics of the cache.
//
// HeadQ technical summary ("Technische Samenvatting"), §2.1: a key error reaches the model only
// through the score error ds_j = s_hat_j - s_j, and the KL between the exact and the perturbed
// attention is locally the Fisher-weighted variance Var_p(ds); §2.2: for fixed attention the value
// distortion of token j is weighed by p_j^2 (the A^2 surrogate). For every (b, query head) over the
// first n_ctx tokens, with s_j = q.k_j/sqrt(d) from the reference keys and p = softmax(s):
//   Var_p(ds), KL = log E_p[exp(ds)] - E_p[ds], E_p[ds], max |ds|, sum_j p_j^2 |v_hat_j - v_j|^2,
//   and the entropy of p,
// where s_hat_j is the corrected logit of §3 step 3: q.k_base_j/sqrt(d) + kappa (U_h^T q).z_hat_j/sqrt(d).
//
// All arithmetic is f64 (full rate on this part's vector units). The score error is taken from
// the key error directly, ds_j = (q.(k_base_j - k_j) + kappa (U_h^T q).z_hat_j)/sqrt(d), with
// k_base_j = code*s + z exact in f64, so it carries no cancellation against s_j.
//
// Launches:
//   prep    queries and U_h^T q in f64 into the workspace (one workgroup per (b, query head))
//   value   (with reference values) |v_hat_j - v_j|^2 per token into the workspace
//   stream  grid (splits, KV heads, batch), 4 waves; a wave takes 64-token chunks (lane = token)
//           and the stream's query heads in batches of 4 (two or four batches: one wave group
//           each, walking the same chunks together). The queries are wave-uniform, so they
//           come through scalar loads and every fma takes them as a scalar operand. Each wave
//           keeps one running max per head, shared by its lanes, so a lane accumulates
//           e^{s - M}-weighted sums (rescaled when M grows); the wave, then the workgroup, reduce
//           them into one partial per (b, head, split).
//   merge   per (b, head): the splits combined by their maxima, then the six statistics.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>

#include <cmath>

#include "headq_internal.h"

namespace headq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kHB = kDiagHeadBatch;  // query heads per batch of the stream pass

typedef const __attribute__((address_space(4))) double* const_f64_ptr;  // read through scalar loads

__device__ __forceinline__ double bf16_bits(uint32_t h) { return (double)__uint_as_float(h << 16); }
__device__ __forceinline__ double f16_bits(uint32_t h) {
  return (double)(float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Element c of a row of key/value dtype (bf16 bits or f32), widened exactly.
__device__ __forceinline__ double elem(const void* row, int64_t c, bool bf16) {
  return bf16 ? bf16_bits(((const uint16_t*)row)[c]) : (double)((const float*)row)[c];
}

// Elements 8n .. 8n+7 of a 16-byte aligned row of key/value dtype, widened exactly.
__device__ __forceinline__ void load8(const char* row, int n, bool bf16, double* out) {
  if (bf16) {
    const uint4 u = *reinterpret_cast<const uint4*>(row + 16 * n);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_bits(w[i] & 0xffffu);
      out[2 * i + 1] = bf16_bits(w[i] >> 16);
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(row + 32 * n);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 u = p[i];
      out[4 * i] = (double)__uint_as_float(u.x);
      out[4 * i + 1] = (double)__uint_as_float(u.y);
      out[4 * i + 2] = (double)__uint_as_float(u.z);
      out[4 * i + 3] = (double)__uint_as_float(u.w);
    }
  }
}

// 8 binary16 values (16 bytes, 16-byte aligned) widened exactly.
__device__ __forceinline__ void load8_f16(const uint16_t* p, double* out) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = f16_bits(w[i] & 0xffffu);
    out[2 * i + 1] = f16_bits(w[i] >> 16);
  }
}

// The same double in every lane, said so to the compiler (a scalar register pair).
__device__ __forceinline__ double uniform(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double wave_max(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ---- prep: q (f64) and U_h^T q (f64, one sequential sum over channels per component), per KV
// head padded with zero queries to a whole number of head batches
__global__ __launch_bounds__(128) void diag_prep_kernel(DiagArgs a) {
  const int GP = diag_padded_heads(a.gqa);
  const int h = blockIdx.x / GP, hh = blockIdx.x % GP, b = blockIdx.y;
  const bool real = hh < a.gqa;
  const int64_t qrow = (int64_t)b * a.hq + h * a.gqa + hh;
  const int64_t wrow = ((int64_t)b * a.hkv + h) * GP + hh;
  __shared__ double qs[128];
  for (int c = threadIdx.x; c < a.d; c += blockDim.x) {
    const double x = real ? elem(a.q, qrow * a.d + c, a.query_bf16) : 0.0;
    qs[c] = x;
    a.ws_q[wrow * a.d + c] = x;
  }
  __syncthreads();
  const int RU = a.r > 0 ? a.r : 1;
  for (int i = threadIdx.x; i < a.r; i += blockDim.x) {
    const float* Uh = a.U + (int64_t)h * a.d * a.r;
    double acc = 0.0;
    for (int c = 0; c < a.d; ++c) acc = fma((double)Uh[c * a.r + i], qs[c], acc);
    a.ws_qu[wrow * RU + i] = acc;
  }
}

// ---- value pass: dv2[b][h][j] = |v_hat_j - v_j|^2 for the A^2 surrogate. A workgroup takes one
// 32-token group of one stream. Both tiles are staged in LDS with 16-byte loads in their own layout
// (reference rows [t][c]; the cache's group block [c][t], 2-bit codes and grid as stored, or the
// tail rows), bf16 values as their raw bits (half the LDS of widened ones, so twice the groups in
// flight per CU) and f32 values as they are; thread (part, t) then sums d/8 channels of token t
// exactly in f64, and the 8 partial sums are added in part order.
template <bool VBF> struct VTile { using T = float; };
template <> struct VTile<true> { using T = uint16_t; };
template <bool VBF>
__device__ __forceinline__ typename VTile<VBF>::T raw_of(const uint32_t* w, int e) {  // element e of a 16-byte chunk
  if constexpr (VBF) return (uint16_t)(e % 2 ? w[e / 2] >> 16 : w[e / 2] & 0xffffu);
  else return __uint_as_float(w[e]);
}
template <bool VBF>
__device__ __forceinline__ double wide(typename VTile<VBF>::T x) {
  if constexpr (VBF) return bf16_bits(x);
  else return (double)x;
}

template <int D, bool VBF>
__global__ __launch_bounds__(kThreads) void diag_value_kernel(DiagArgs a) {
  constexpr int CPT = D / 8;                  // channels per thread
  using ET = typename VTile<VBF>::T;
  // LDS pitches (elements): the column reads of ref_s (lane = token) hit 32 distinct banks
  constexpr int PR = VBF ? D + 2 : D + 1, PV = VBF ? kGroup + 2 : kGroup + 1;
  __shared__ ET ref_s[kGroup][PR];            // reference values [t][c]
  __shared__ ET val_s[D][PV];                 // the cache's values [c][t] (dense or tail)
  __shared__ __attribute__((aligned(16))) uint8_t code_s[D * 8];  // 2-bit: the code block as stored
  __shared__ __attribute__((aligned(16))) uint16_t meta_s[2 * D];  // 2-bit: step, zero [2][d/32][32]
  __shared__ __attribute__((aligned(16))) uint16_t prot_s[2 * D];  // the value policy's corrections [P][d]
  __shared__ double part_s[8][kGroup];
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int64_t g0 = (int64_t)blockIdx.x * kGroup;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t n_full = a.n_ctx / kGroup * kGroup;
  const int n_tok = (int)(a.n_ctx - g0 < kGroup ? a.n_ctx - g0 : kGroup);
  const bool tail = g0 >= n_full;
  constexpr int es = VBF ? 2 : 4, epc = 16 / es;  // element size, elements per 16-byte chunk
  constexpr int chunks_row = D / epc;

  // reference rows (and tail rows) [t][c] -> LDS
  for (int i = tid; i < kGroup * chunks_row; i += kThreads) {
    const int t = i / chunks_row, c0 = (i % chunks_row) * epc;
    ET x[8] = {0, 0, 0, 0, 0, 0, 0, 0}, y[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (t < n_tok) {
      const char* vr = (const char*)a.v_ref + ((int64_t)b * a.vs_b + (int64_t)h * a.vs_h + (g0 + t) * a.vs_t) * es;
      const uint4 u = *reinterpret_cast<const uint4*>(vr + c0 * es);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < epc; ++e) x[e] = raw_of<VBF>(w, e);
      if (tail) {
        const char* vt = (const char*)a.vtail + (bh * kGroup + t) * D * es;
        const uint4 v = *reinterpret_cast<const uint4*>(vt + c0 * es);
        const uint32_t z[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < epc; ++e) y[e] = raw_of<VBF>(z, e);
      }
    }
#pragma unroll
    for (int e = 0; e < epc; ++e) {
      ref_s[t][c0 + e] = x[e];
      if (tail) val_s[c0 + e][t] = y[e];
    }
  }
  if (!tail) {
    const int64_t blk = a.map.block(b, h, g0 / kGroup);
    if (a.value_mode == HEADQ_V_DENSE) {
      // group block [c][32 tokens]: a chunk is epc tokens of one channel
      const char* vg = (const char*)a.vdense + blk * D * kGroup * es;
      for (int i = tid; i < D * kGroup / epc; i += kThreads) {
        const int c = i / (kGroup / epc), t0 = (i % (kGroup / epc)) * epc;
        const uint4 u = reinterpret_cast<const uint4*>(vg)[i];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < epc; ++e) val_s[c][t0 + e] = raw_of<VBF>(w, e);
      }
    } else {
      for (int i = tid; i < D * 8 / 16; i += kThreads)
        reinterpret_cast<uint4*>(code_s)[i] = reinterpret_cast<const uint4*>(a.vcode + blk * D * 8)[i];
      for (int i = tid; i < 2 * D / 8; i += kThreads)
        reinterpret_cast<uint4*>(meta_s)[i] = reinterpret_cast<const uint4*>(a.vmeta + blk * 2 * D)[i];
      for (int i = tid; i < a.value_protect * D / 8; i += kThreads)
        reinterpret_cast<uint4*>(prot_s)[i] =
            reinterpret_cast<const uint4*>(a.vprot + blk * a.value_protect * D)[i];
    }
  }
  // the group's corrected tokens (A^2 value policy): the cache's value of token t is then
  // code * s + z + correction
  uint32_t pidx = 0;
  if (!tail && a.value_mode != HEADQ_V_DENSE && a.value_protect)
    pidx = a.vpidx[a.map.block(b, h, g0 / kGroup)];
  __syncthreads();

  const int t = tid % kGroup, part = tid / kGroup;
  const bool q2 = !tail && a.value_mode != HEADQ_V_DENSE;
  int pslot = -1;  // this token's correction slot, if any
  for (int k = 0; k < (q2 ? a.value_protect : 0); ++k)
    if ((int)((pidx >> (8 * k)) & 31u) == t) pslot = k;
  double e2 = 0.0;
  if (t < n_tok) {
    const int bit = vcode_pair_bit(t);
#pragma unroll 8
    for (int k = 0; k < CPT; ++k) {
      const int c = part * CPT + k;
      double vh;
      if (q2) {
        const uint32_t pair = *reinterpret_cast<const uint16_t*>(code_s + vcode_pair_offset(D, c, t));
        const int gc = c / 32;
        vh = (double)((pair >> bit) & 3u) * f16_bits(meta_s[gc * kGroup + t]) +
             f16_bits(meta_s[(D / 32 + gc) * kGroup + t]);
        if (pslot >= 0) vh += bf16_bits(prot_s[pslot * D + c]);
      } else {
        vh = wide<VBF>(val_s[c][t]);
      }
      const double dv = vh - wide<VBF>(ref_s[t][c]);
      e2 = fma(dv, dv, e2);
    }
  }
  part_s[part][t] = e2;
  __syncthreads();
  if (tid < n_tok) {
    double sum = 0.0;
    for (int p = 0; p < 8; ++p) sum += part_s[p][tid];
    a.ws_dv2[bh * a.n_ctx + g0 + tid] = sum;
  }
}

// One f64 element of 32 channels held as raw 32-bit words: bf16 pairs or f32.
template <bool BF16>
__device__ __forceinline__ double raw_elem(const uint32_t* w, int c) {
  if constexpr (BF16) return bf16_bits(c % 2 ? w[c / 2] >> 16 : w[c / 2] & 0xffffu);
  else return (double)__uint_as_float(w[c]);
}

// ---- stream pass
template <int D, int R, bool KBF, bool NB>
__global__ __launch_bounds__(kThreads) void diag_stream_kernel(DiagArgs a) {
  constexpr int RU = R > 0 ? R : 1;
  constexpr int KW = KBF ? 16 : 32;  // 32-bit words of 32 reference-key channels
  constexpr int kes = KBF ? 2 : 4;
  __shared__ double part_s[kWaves][kHB][kDiagPart];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  const int g = a.gqa, hq0 = h * g;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t n_ctx = a.n_ctx, n_full = n_ctx / kGroup * kGroup;
  const int64_t n_chunks = (n_ctx + 63) / 64;
  const double inv_sqrt_d = 1.0 / sqrt((double)D);
  // Head batches: with 2 or 4 of them the waves split into groups, one batch per group, that walk
  // the same chunks together (the second read of a chunk hits the caches); with 1 or 3 every wave
  // runs the batches in turn.
  const int nb = (g + kHB - 1) / kHB;
  const int wpb = kWaves % nb == 0 ? kWaves / nb : kWaves;  // waves per batch
  const int n_rounds = wpb == kWaves ? nb : 1;
  const int slot = wave % wpb, W = a.n_splits * wpb;

  for (int round = 0; round < n_rounds; ++round) {
    const int hb = (wpb == kWaves ? round : wave / wpb) * kHB;
    // padded heads (past g) have zero queries: every batch runs all kHB heads unconditionally
    const int64_t wrow = ((int64_t)b * a.hkv + h) * diag_padded_heads(g) + hb;
    const const_f64_ptr qh = (const_f64_ptr)(a.ws_q + wrow * D);
    const const_f64_ptr quh = (const_f64_ptr)(a.ws_qu + wrow * RU);
    double M[kHB], S0[kHB], S1[kHB], S2[kHB], S3[kHB], S4[kHB], S5[kHB], MX[kHB];
#pragma unroll
    for (int i = 0; i < kHB; ++i) {
      M[i] = -INFINITY;
      S0[i] = S1[i] = S2[i] = S3[i] = S4[i] = S5[i] = MX[i] = 0.0;
    }
    for (int64_t k = (int64_t)split * wpb + slot; k < n_chunks; k += W) {
      const int64_t j = k * 64 + lane;
      const bool valid = j < n_ctx, tail = j >= n_full;
      double acc_s[kHB], acc_d[kHB];
#pragma unroll
      for (int i = 0; i < kHB; ++i) acc_s[i] = acc_d[i] = 0.0;
      if (valid) {
        const char* kr = (const char*)a.k_ref + ((int64_t)b * a.ks_b + (int64_t)h * a.ks_h + j * a.ks_t) * kes;
        if (!tail) {
          // 32 channels at a time: reference keys, codes, steps and zeros; k_base = code*s + z
          // is exact in f64, and so is the key error dk = k_base - k
          const int64_t row = a.map.row(b, h, j);
          const uint16_t* meta = a.kmeta + a.map.block(b, h, j / kGroup) * 2 * D;
#pragma unroll 1
          for (int blk = 0; blk < D / 32; ++blk) {
            uint32_t kw[KW], sw[16], zw[16];
#pragma unroll
            for (int i = 0; i < KW / 4; ++i) {
              const uint4 u = reinterpret_cast<const uint4*>(kr + blk * 32 * kes)[i];
              kw[4 * i] = u.x, kw[4 * i + 1] = u.y, kw[4 * i + 2] = u.z, kw[4 * i + 3] = u.w;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint4 u = reinterpret_cast<const uint4*>(meta + 32 * blk)[i];
              sw[4 * i] = u.x, sw[4 * i + 1] = u.y, sw[4 * i + 2] = u.z, sw[4 * i + 3] = u.w;
              const uint4 v = reinterpret_cast<const uint4*>(meta + D + 32 * blk)[i];
              zw[4 * i] = v.x, zw[4 * i + 1] = v.y, zw[4 * i + 2] = v.z, zw[4 * i + 3] = v.w;
            }
            // the block's packed codes: 2 words of 2-bit codes, or 4 nibble words
            uint32_t cw[NB ? 4 : 2];
            if constexpr (NB) {
              const uint4 u = *reinterpret_cast<const uint4*>(a.kcode + row * (D / 2) + 16 * blk);
              cw[0] = u.x, cw[1] = u.y, cw[2] = u.z, cw[3] = u.w;
            } else {
              const uint2 u = *reinterpret_cast<const uint2*>(a.kcode + row * (D / 4) + 8 * blk);
              cw[0] = u.x, cw[1] = u.y;
            }
#pragma unroll
            for (int cc = 0; cc < 32; ++cc) {
              // keep the scheduler from converting all 32 channels at once (register pressure)
              if (cc % 8 == 0) __builtin_amdgcn_sched_barrier(0);
              const double code = NB ? (double)((cw[cc / 8] >> kcode4_bit(cc % 8)) & 15u)
                                     : (double)((cw[cc / 16] >> kcode_bit(cc % 16)) & 3u);
              const double sv = f16_bits(cc % 2 ? sw[cc / 2] >> 16 : sw[cc / 2] & 0xffffu);
              const double zv = f16_bits(cc % 2 ? zw[cc / 2] >> 16 : zw[cc / 2] & 0xffffu);
              const double kk = raw_elem<KBF>(kw, cc);
              const double dk = (code * sv + zv) - kk;
#pragma unroll
              for (int i = 0; i < kHB; ++i) {
                const double qc = qh[i * D + 32 * blk + cc];
                acc_s[i] = fma(qc, kk, acc_s[i]);
                acc_d[i] = fma(qc, dk, acc_d[i]);
              }
            }
          }
          if constexpr (R > 0) {
            // side correction kappa (U_h^T q).z_hat_j with z_hat_j = sigma_j * (nibble - 8)
            const double sg = f16_bits(a.ssc[row]);
            const uint8_t* sc = a.scode + row * (R / 2);
            double corr[kHB];
#pragma unroll
            for (int i = 0; i < kHB; ++i) corr[i] = 0.0;
#pragma unroll 4
            for (int r = 0; r < R; ++r) {
              const double z = sg * (double)((int)((sc[r / 2] >> (4 * (r % 2))) & 0xfu) - 8);
#pragma unroll
              for (int i = 0; i < kHB; ++i)
                corr[i] = fma(quh[i * RU + r], z, corr[i]);
            }
#pragma unroll
            for (int i = 0; i < kHB; ++i) acc_d[i] = fma(a.kappa, corr[i], acc_d[i]);
          }
        } else {
          // the unfinished group: exact keys from the dense tail, no side code
          const char* kt = (const char*)a.ktail + (bh * kGroup + j % kGroup) * D * kes;
#pragma unroll 1
          for (int n = 0; n < D / 8; ++n) {
            double kk8[8], kh8[8];
            load8(kr, n, KBF, kk8);
            load8(kt, n, KBF, kh8);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const double dk = kh8[jj] - kk8[jj];
#pragma unroll
              for (int i = 0; i < kHB; ++i) {
                const double qc = qh[i * D + 8 * n + jj];
                acc_s[i] = fma(qc, kk8[jj], acc_s[i]);
                acc_d[i] = fma(qc, dk, acc_d[i]);
              }
            }
          }
        }
      }
      const double dv2 = a.v_ref && valid ? a.ws_dv2[bh * n_ctx + j] : 0.0;
      // online statistics: one running max per head, shared by the lanes of the wave
#pragma unroll
      for (int i = 0; i < kHB; ++i) {
        {
          const double s = acc_s[i] * inv_sqrt_d, ds = acc_d[i] * inv_sqrt_d;
          const double mc = uniform(wave_max(valid ? s : -INFINITY));
          if (mc > M[i]) {
            const double f = M[i] == -INFINITY ? 0.0 : exp(M[i] - mc);
            S0[i] *= f;
            S1[i] *= f;
            S2[i] *= f;
            S3[i] *= f;
            S4[i] *= f * f;
            S5[i] *= f;
            M[i] = mc;
          }
          if (valid) {
            const double w = exp(s - M[i]);
            S0[i] += w;
            S1[i] = fma(w, ds, S1[i]);
            S2[i] = fma(w * ds, ds, S2[i]);
            S3[i] = fma(w, expm1(ds), S3[i]);
            S4[i] = fma(w * w, dv2, S4[i]);
            S5[i] = fma(w, s, S5[i]);
            MX[i] = fmax(MX[i], fabs(ds));
          }
        }
      }
    }
    // the wave's lanes share M: plain sums over lanes
#pragma unroll
    for (int i = 0; i < kHB; ++i) {
      {
        const double v0 = wave_sum(S0[i]), v1 = wave_sum(S1[i]), v2 = wave_sum(S2[i]);
        const double v3 = wave_sum(S3[i]), v4 = wave_sum(S4[i]), v5 = wave_sum(S5[i]);
        double mx = MX[i];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o));
        if (lane == 0) {
          part_s[wave][i][0] = M[i];
          part_s[wave][i][1] = v0;
          part_s[wave][i][2] = v1;
          part_s[wave][i][3] = v2;
          part_s[wave][i][4] = v3;
          part_s[wave][i][5] = v4;
          part_s[wave][i][6] = v5;
          part_s[wave][i][7] = mx;
        }
      }
    }
    __syncthreads();
    // one thread per (wave group, head): merge the group's waves into the split partial
    const int grp = threadIdx.x / kHB, i = threadIdx.x % kHB;
    const int hb_t = (wpb == kWaves ? round : grp) * kHB;
    if (grp < kWaves / wpb && hb_t + i < g) {
      double Mx = -INFINITY;
      for (int w = grp * wpb; w < (grp + 1) * wpb; ++w) Mx = fmax(Mx, part_s[w][i][0]);
      double acc[6] = {0, 0, 0, 0, 0, 0}, mx = 0.0;
      for (int w = grp * wpb; w < (grp + 1) * wpb; ++w) {
        mx = fmax(mx, part_s[w][i][7]);
        if (part_s[w][i][0] == -INFINITY) continue;
        const double f = exp(part_s[w][i][0] - Mx);
        for (int k = 0; k < 6; ++k) acc[k] = fma(part_s[w][i][1 + k], k == 4 ? f * f : f, acc[k]);
      }
      double* out = a.ws_part + (((int64_t)b * a.hq + hq0 + hb_t + i) * a.n_splits + split) * kDiagPart;
      out[0] = Mx;
      for (int k = 0; k < 6; ++k) out[1 + k] = acc[k];
      out[7] = mx;
    }
    __syncthreads();
  }
}

// ---- merge the splits of every (b, query head) and finish the statistics
__global__ __launch_bounds__(64) void diag_merge_kernel(DiagArgs a) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= (int64_t)a.batch * a.hq) return;
  const double* p = a.ws_part + row * a.n_splits * kDiagPart;
  double Mx = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) Mx = fmax(Mx, p[s * kDiagPart]);
  double S[6] = {0, 0, 0, 0, 0, 0}, mx = 0.0;
  for (int s = 0; s < a.n_splits; ++s) {
    const double* q = p + s * kDiagPart;
    mx = fmax(mx, q[7]);
    if (q[0] == -INFINITY) continue;
    const double f = exp(q[0] - Mx);
    for (int k = 0; k < 6; ++k) S[k] = fma(q[1 + k], k == 4 ? f * f : f, S[k]);
  }
  const double mean = S[1] / S[0];
  double* o = a.stats + row * HEADQ_DIAG_NSTAT;
  o[HEADQ_DIAG_FISHER_VAR] = S[2] / S[0] - mean * mean;
  o[HEADQ_DIAG_KL] = log1p(S[3] / S[0]) - mean;
  o[HEADQ_DIAG_MEAN_DS] = mean;
  o[HEADQ_DIAG_MAX_ABS_DS] = mx;
  o[HEADQ_DIAG_A2] = a.v_ref ? S[4] / (S[0] * S[0]) : NAN;
  o[HEADQ_DIAG_ENTROPY] = log(S[0]) + Mx - S[5] / S[0];
}

template <int D, bool KBF, bool NB>
hipError_t launch_dk(const DiagArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.n_splits, (unsigned)a.hkv, (unsigned)a.batch);
  switch (a.r) {
    case 0: hipLaunchKernelGGL((diag_stream_kernel<D, 0, KBF, NB>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((diag_stream_kernel<D, 4, KBF, NB>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((diag_stream_kernel<D, 8, KBF, NB>), grid, dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((diag_stream_kernel<D, 16, KBF, NB>), grid, dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((diag_stream_kernel<D, 32, KBF, NB>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DiagArgs& a, hipStream_t s) {
  if (a.v_ref) {
    dim3 grid((unsigned)((a.n_ctx + kGroup - 1) / kGroup), (unsigned)a.hkv, (unsigned)a.batch);
    if (a.value_bf16)
      hipLaunchKernelGGL((diag_value_kernel<D, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((diag_value_kernel<D, false>), grid, dim3(kThreads), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.key_nib) return a.key_bf16 ? launch_dk<D, true, true>(a, s) : launch_dk<D, false, true>(a, s);
  return a.key_bf16 ? launch_dk<D, true, false>(a, s) : launch_dk<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_diagnostics(const DiagArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(diag_prep_kernel, dim3((unsigned)(a.hkv * diag_padded_heads(a.gqa)), (unsigned)a.batch), dim3(128), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = a.d == 64 ? launch_d<64>(a, s) : a.d == 128 ? launch_d<128>(a, s) : hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  const int rows = a.batch * a.hq;
  hipLaunchKernelGGL(diag_merge_kernel, dim3((unsigned)((rows + 63) / 64)), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace headq
