// prefill_mfma.hip — headq_prefill_attn on gfx950 matrix cores: chunked-prefill attention over
// the HeadQ cache.
//
// HeadQ technical summary ("Technische Samenvatting"), §3 step 3 (Cache Uitlezen), read once per
// query token: token t of a chunk, at position start + t, attends the cached tokens 0 .. start + t
// with the corrected logit
//     s_j = q.k_base_j / sqrt(d) + (U_h^T q).z_hat_j / sqrt(d)
// and the softmax readout sum_j p_j v_j (§1, §2.2).
//
// With many query tokens the cache reads are shared. A workgroup owns 64 (query token, head)
// columns of one (b, h) stream, 16 per wave, and walks the stream's 32-token groups once: the
// whole workgroup stages each group in LDS with 16-byte loads (two LDS buffers; the next three
// groups' loads are in flight in registers while a group is computed) and every wave contracts it
// against its 16 columns on the matrix cores, as the decode does with its 16 heads:
//   scores^T [32 tok x 16 cols] = codes . (q o s)^T  (+ q.z)  + zc . (U^T q)^T scaled by sigma_j
//   out^T    [d x 16 cols]     += V^T . P^T
// with the decode's operand precision (the f32 factors split into high and low half-precision
// parts, f32 accumulation) and its per-column power-of-two query scale. Causality is a token limit
// per column: a wave skips the groups past its last column and masks only the groups that reach
// past its first one. The tokens of the cache's unfinished group come from the exact tails, on
// the vector units.
#include <hip/hip_runtime.h>

#include "headq_internal.h"
#include "mfma_common.h"

namespace headq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = 16 * kWaves;        // (query token, head) columns per workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;          // rescale only when the max grows by more than 2^8

// Bytes of one 32-token group as staged in LDS (each array of a group is one contiguous block of
// the cache): packed key codes 32 x d/4 | key step/zero rows 2 x d x 2 | side codes 32 x r/2 |
// sigma 32 x 2 | (2-bit values) value step/zero rows 2 x d/32 x 32 x 2 | values (dense bf16
// [d][32], or 2-bit codes d x 8 in matrix-operand order) | (A^2 value policy) corrections
// [P][d] bf16 | their token-index word, padded to 16 bytes.
template <int D, int R, bool VQ2, bool NB, int VP = 0>
struct Tile {
  static constexpr int KC = kGroup * D / (NB ? 2 : 4), KM = 4 * D, SC = kGroup * R / 2, SG = R > 0 ? kGroup * 2 : 0;
  static constexpr int VM = VQ2 ? 4 * D : 0, VB = VQ2 ? D * 8 : D * kGroup * 2;
  static constexpr int VPB = VP * D * 2, VIB = VP > 0 ? 16 : 0;  // A^2 value policy: corrections, index word
  static constexpr int OFF_KM = KC, OFF_SC = OFF_KM + KM, OFF_SG = OFF_SC + SC, OFF_VM = OFF_SG + SG;
  static constexpr int OFF_V = OFF_VM + VM, OFF_VP = OFF_V + VB, OFF_VI = OFF_VP + VPB, BYTES = OFF_VI + VIB;
  static constexpr int CHUNKS = BYTES / 16;
  static_assert(BYTES % 16 == 0 && OFF_V % 16 == 0, "16-byte staging");
};

// Staging plan of a group: every array of the group's block is fetched in pieces of 64 16-byte
// chunks, one piece per wave instruction, so a piece never mixes arrays and its source is one
// wave-uniform buffer resource (a lane's offset is its chunk). Piece q of the group (in array
// order) goes to wave q % 4, into its register q / 4. Arrays: key codes, key step/zero, side
// codes, sigma, 2-bit value step/zero, values, the value policy's corrections (its index word,
// 4 bytes per group, is loaded on its own).
template <int D, int R, bool VQ2, bool NB, int VP>
struct Stage {
  using TL = Tile<D, R, VQ2, NB, VP>;
  static constexpr int NARR = 7;
  static constexpr int BYTES[NARR] = {TL::KC, TL::KM, TL::SC, TL::SG, TL::VM, TL::VB, TL::VPB};
  static constexpr int OFF[NARR] = {0, TL::OFF_KM, TL::OFF_SC, TL::OFF_SG, TL::OFF_VM, TL::OFF_V, TL::OFF_VP};
  static constexpr int chunks(int A) { return BYTES[A] / 16; }
  static constexpr int pieces(int A) { return (chunks(A) + 63) / 64; }
  static constexpr int first(int A) {
    int q = 0;
    for (int i = 0; i < A; ++i) q += pieces(i);
    return q;
  }
  static constexpr int KV = (first(NARR) + 3) / 4;  // pieces (16-byte registers) per lane
  static_assert(TL::KC % 16 == 0 && TL::KM % 16 == 0 && TL::SC % 16 == 0 && TL::SG % 16 == 0 &&
                    TL::VM % 16 == 0 && TL::VB % 16 == 0 && TL::VPB % 16 == 0,
                "16-byte chunks");
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stage_rsrc(const void* base, int64_t bytes) {
  const uint32_t nbytes = bytes > 0x7fffffff ? 0x7fffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

// Per-lane operands fixed for the whole kernel (column n of the wave).
template <int D, int R>
struct Fixed {
  static constexpr int NKT = D / 32;
  half8_t bq_hi[NKT], bq_lo[NKT];  // scaled query at this lane's channels, hi/lo f16
  half4_t bu_hi4, bu_lo4;          // U^T q at ranks 4*quad + j (16x16x16 path)
  half8_t bu_hi8, bu_lo8;          // U^T q at ranks 8*quad + j (16x16x32 path, r = 32)
  float inv_scale;                 // 2^e: undoes the per-column query scale
};

// o += p_t * correction_t for the group's corrected tokens t (A^2 value policy; rows at `prow`,
// [VP][d] bf16): token t's probability for this column is held by the lane of the same column
// with quad t / 8, slot t % 8.
template <int D, int VP>
__device__ __forceinline__ void add_corrections(const uint8_t* prow, uint32_t idx, const float* p, int n, int quad,
                                                floatx4* o_acc) {
  constexpr int NCT = D / 16;
#pragma unroll
  for (int k = 0; k < VP; ++k) {
    const int t = (idx >> (8 * k)) & 31;
    float pt = p[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) pt = (t & 7) == j ? p[j] : pt;
    pt = __shfl(pt, n + 16 * (t >> 3));
    const uint16_t* row = reinterpret_cast<const uint16_t*>(prow + k * D * 2);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(row + 16 * ct + 4 * quad);  // channels 16ct + 4quad ..+3
      o_acc[ct][0] = fmaf(pt, __uint_as_float(w[0] << 16), o_acc[ct][0]);
      o_acc[ct][1] = fmaf(pt, __uint_as_float(w[0] & 0xffff0000u), o_acc[ct][1]);
      o_acc[ct][2] = fmaf(pt, __uint_as_float(w[1] << 16), o_acc[ct][2]);
      o_acc[ct][3] = fmaf(pt, __uint_as_float(w[1] & 0xffff0000u), o_acc[ct][3]);
    }
  }
}

// One staged group against the wave's 16 columns: scores, causal mask, online softmax, P.V (and
// the value policy's corrections when VP > 0).
template <int D, int R, bool VQ2, bool NB, int VP>
__device__ __forceinline__ void group_step(const uint8_t* T, const Fixed<D, R>& f, int tok0,
                                           bool masked, int n_att, float* lg_row, int n, int quad, int lane,
                                           floatx4* o_acc, float* z_acc, float& m_run, float& l_run) {
  using TL = Tile<D, R, VQ2, NB, VP>;
  constexpr int NKT = D / 32, NCT = D / 16, NG = D / 32;
  const _Float16* km_h = reinterpret_cast<const _Float16*>(T + TL::OFF_KM);
  const int row_tok0 = 8 * (n / 4) + (n % 4);  // token of this lane's row in tile 0 (tile 1: +4)
  // packed codes of the row tokens, this lane's piece (channels (d/4)*quad .. +d/4): d/64 words
  // of 2-bit codes, or d/32 nibble words (3- and 4-bit base codes)
  constexpr int KW = NB ? D / 32 : D / 64;
  uint32_t kcw[2][KW];
#pragma unroll
  for (int Ti = 0; Ti < 2; ++Ti) {
    const uint8_t* p = T + (row_tok0 + 4 * Ti) * (TL::KC / 32) + 4 * KW * quad;
#pragma unroll
    for (int w = 0; w < KW; ++w) kcw[Ti][w] = reinterpret_cast<const uint32_t*>(p)[w];
  }
  // zero term q.z (the same for every token row), then codes . (q o s) on top of it
  floatx4 cz = (floatx4){0.f, 0.f, 0.f, 0.f};
  half8_t st[NKT];
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    const int c0 = (D / 4) * quad + 8 * t;
    st[t] = *reinterpret_cast<const half8_t*>(km_h + c0);
    const half8_t zt = *reinterpret_cast<const half8_t*>(km_h + D + c0);
    cz = mfma_f16(zt, f.bq_hi[t], cz);
    cz = mfma_f16(zt, f.bq_lo[t], cz);
  }
  floatx4 acc[2] = {cz, cz};
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    // (q o s) as hi + lo f16: the exact product error by fma, plus the low part of q times s
    const half8_t p_hi = f.bq_hi[t] * st[t];
    const half8_t e = __builtin_elementwise_fma(f.bq_hi[t], st[t], -p_hi);
    const half8_t p_lo = __builtin_elementwise_fma(f.bq_lo[t], st[t], e);
#pragma unroll
    for (int Ti = 0; Ti < 2; ++Ti) {
      half8_t ac;
      if constexpr (NB) {
        ac = key_codes8_nib(kcw[Ti][t]);
      } else {
        const uint32_t w = kcw[Ti][(D == 128) ? (t >> 1) : 0];
        ac = key_codes8((t & 1) ? odd_codes(w) : even_codes(w));
      }
      acc[Ti] = mfma_f16(ac, p_hi, acc[Ti]);
      acc[Ti] = mfma_f16(ac, p_lo, acc[Ti]);
    }
  }
  // scores of tokens 8*quad + j for column n, in log2 units before the column's power-of-two
  // scale (applied in the softmax; the correction scale is folded into U^T q)
  float sv[8];
  if constexpr (R > 0) {
    floatx4 cr[2];
#pragma unroll
    for (int Ti = 0; Ti < 2; ++Ti) {
      cr[Ti] = (floatx4){0.f, 0.f, 0.f, 0.f};
      const uint8_t* srow = T + TL::OFF_SC + (row_tok0 + 4 * Ti) * (R / 2);
      if constexpr (R == 32) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(srow + 4 * quad);
        const half4_t lo4 = nibbles4_f16(w & 0xffffu), hi4 = nibbles4_f16(w >> 16);
        const half8_t az = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        cr[Ti] = mfma_f16(az, f.bu_hi8, cr[Ti]);
        cr[Ti] = mfma_f16(az, f.bu_lo8, cr[Ti]);
      } else {
        // ranks 4*quad .. 4*quad+3; quads past the rank multiply zero operands
        const uint32_t w = (2 * quad < R / 2) ? *reinterpret_cast<const uint16_t*>(srow + 2 * quad) : 0x8888u;
        const half4_t az = nibbles4_f16(w);
        cr[Ti] = mfma_f16k16(az, f.bu_hi4, cr[Ti]);
        cr[Ti] = mfma_f16k16(az, f.bu_lo4, cr[Ti]);
      }
    }
    const half8_t sg = *reinterpret_cast<const half8_t*>(T + TL::OFF_SG + 16 * quad);
#pragma unroll
    for (int Ti = 0; Ti < 2; ++Ti)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sv[4 * Ti + j] = fmaf((float)sg[4 * Ti + j], cr[Ti][j], acc[Ti][j]);
  } else {
#pragma unroll
    for (int Ti = 0; Ti < 2; ++Ti)
#pragma unroll
      for (int j = 0; j < 4; ++j) sv[4 * Ti + j] = acc[Ti][j];
  }
  if (masked) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (tok0 + 8 * quad + j >= n_att) sv[j] = -INFINITY;
  }
  if (lg_row) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (tok0 + 8 * quad + j < n_att) lg_row[tok0 + 8 * quad + j] = f.inv_scale * sv[j] * kLn2;
  }

  // online softmax (lazy maximum); masked tokens weigh 0. The scale is a power of two, so scaling
  // the maximum, or each score inside the exponent's fma, rounds exactly as scaling first would.
  float mx = sv[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
  mx = f.inv_scale * quad_max(mx);
  const bool grow = mx > m_run + kLazyMax;  // true on a column's first unmasked group
  if (__any(grow)) {
    const float m_new = grow ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first group, 1 if unchanged
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) o_acc[ct] *= alpha;
    if constexpr (VQ2)
#pragma unroll
      for (int cg = 0; cg < NG; ++cg) z_acc[cg] *= alpha;
  }
  float p[8];
  if (masked) {  // a column whose limit falls in this group may see only masked scores (m_run = -inf)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      p[j] = sv[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(fmaf(f.inv_scale, sv[j], -m_run));
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(f.inv_scale, sv[j], -m_run));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) l_run += p[j];
  if constexpr (VQ2) {
    // v_hat = code * s + z per (token, 32-channel group): the code part is a matrix product with
    // p o s as the second operand (one per channel group); the zero part sum_j p_j z_j per column
    // and group is accumulated per lane and summed over the quads at the end
    const _Float16* vm_h = reinterpret_cast<const _Float16*>(T + TL::OFF_VM);
    const uint32_t* vcw = reinterpret_cast<const uint32_t*>(T + TL::OFF_V + lane * (D / 8));
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) {
      const uint32_t x = vcw[cg];
      const uint32_t ve = even_codes(x), vo = odd_codes(x);
      const half8_t s8 = *reinterpret_cast<const half8_t*>(vm_h + cg * kGroup + 8 * quad);
      const half8_t z8 = *reinterpret_cast<const half8_t*>(vm_h + (NG + cg) * kGroup + 8 * quad);
      u32x4 xh, xl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h2, l2;
        split_bf16_pair(__builtin_fmaf(p[2 * i], (float)s8[2 * i], 0.0f),
                        __builtin_fmaf(p[2 * i + 1], (float)s8[2 * i + 1], 0.0f), h2, l2);
        xh[i] = h2;
        xl[i] = l2;
      }
      float za = z_acc[cg];
#pragma unroll
      for (int j = 0; j < 8; ++j) za = fmaf(p[j], (float)z8[j], za);
      z_acc[cg] = za;
      const bf16x8_t bh = bitcast<bf16x8_t>(xh), bl = bitcast<bf16x8_t>(xl);
      const bf16x8_t a0 = value_codes8<0>(ve, vo);
      const bf16x8_t a1 = value_codes8<1>(ve, vo);
      o_acc[2 * cg] = mfma_bf16(a0, bh, o_acc[2 * cg]);
      o_acc[2 * cg] = mfma_bf16(a0, bl, o_acc[2 * cg]);
      o_acc[2 * cg + 1] = mfma_bf16(a1, bh, o_acc[2 * cg + 1]);
      o_acc[2 * cg + 1] = mfma_bf16(a1, bl, o_acc[2 * cg + 1]);
    }
    if constexpr (VP > 0)
      add_corrections<D, VP>(T + TL::OFF_VP, *reinterpret_cast<const uint32_t*>(T + TL::OFF_VI), p, n, quad, o_acc);
  } else {
    bf16x8_t p_hi, p_lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 ph = (__bf16)p[j];
      p_hi[j] = ph;
      p_lo[j] = (__bf16)(p[j] - (float)ph);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      // channel 16*ct + n, tokens 8*quad .. +7 of the channel-major value block
      const bf16x8_t av =
          *reinterpret_cast<const bf16x8_t*>(T + TL::OFF_V + ((16 * ct + n) * kGroup + 8 * quad) * 2);
      o_acc[ct] = mfma_bf16(av, p_hi, o_acc[ct]);
      o_acc[ct] = mfma_bf16(av, p_lo, o_acc[ct]);
    }
  }
}

// Tokens of the cache's unfinished group (exact, from the tails) for the wave's columns, on the
// vector units: lane (n, quad) scores tail rows 8*quad .. +7 for column n (rows past the column's
// limit weigh 0), takes the same online-softmax step, and adds p . v to its output channels
// 16*ct + 4*quad + j with the other quads' probabilities fetched by lane shuffles.
template <int D>
__device__ __forceinline__ void tail_step(const PrefillArgs& a, int64_t bh, int64_t n_full, int tail_len,
                                          int64_t n_att, const float* qcol, float inv_scale, float* lg_row, int n,
                                          int quad, floatx4* o_acc, float* z_acc, int n_z, float& m_run,
                                          float& l_run) {
  constexpr int NCT = D / 16;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll 1
  for (int c = 0; c < D; c += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = 8 * quad + j;
      if (t >= tail_len) continue;
      const int64_t row = (bh * kGroup + t) * D + c;
      float k[8];
      if (a.key_bf16) {
        const u32x4 w = *reinterpret_cast<const u32x4*>((const uint16_t*)a.ktail + row);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          k[2 * i] = __uint_as_float(w[i] << 16);
          k[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
        const floatx4 w0 = *reinterpret_cast<const floatx4*>((const float*)a.ktail + row);
        const floatx4 w1 = *reinterpret_cast<const floatx4*>((const float*)a.ktail + row + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          k[i] = w0[i];
          k[4 + i] = w1[i];
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[j] = fmaf(qcol[c + i], k[i], acc[j]);
    }
  }
  float sv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = 8 * quad + j;
    const bool live = t < tail_len && n_full + t < n_att;
    sv[j] = live ? inv_scale * acc[j] : -INFINITY;
    if (live && lg_row) lg_row[n_full + t] = sv[j] * kLn2;
  }
  float mx = sv[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
  mx = quad_max(mx);
  const bool grow = mx > m_run + kLazyMax;
  if (__any(grow)) {
    const float m_new = grow ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) o_acc[ct] *= alpha;
    for (int cg = 0; cg < n_z; ++cg) z_acc[cg] *= alpha;
  }
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = sv[j] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sv[j] - m_run);
    l_run += p[j];
  }
#pragma unroll 1
  for (int t = 0; t < tail_len; ++t) {
    // row t's probability for column n lives in lane n + 16 * (t / 8), slot t % 8
    const int js = t % 8;
    float pj = p[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) pj = js == j ? p[j] : pj;
    const float pt = __shfl(pj, n + 16 * (t / 8));
    const int64_t row = (bh * kGroup + t) * D + 4 * quad;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float v[4];
      if (a.value_bf16) {
        const u32x2 w = *reinterpret_cast<const u32x2*>((const uint16_t*)a.vtail + row + 16 * ct);
        v[0] = __uint_as_float(w[0] << 16);
        v[1] = __uint_as_float(w[0] & 0xffff0000u);
        v[2] = __uint_as_float(w[1] << 16);
        v[3] = __uint_as_float(w[1] & 0xffff0000u);
      } else {
        const floatx4 w = *reinterpret_cast<const floatx4*>((const float*)a.vtail + row + 16 * ct);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = w[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) o_acc[ct][i] = fmaf(pt, v[i], o_acc[ct][i]);
    }
  }
}

template <int D, int R, bool VQ2, bool NB, int VP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(PrefillArgs a) {
  static_assert(VP == 0 || (VQ2 && !NB), "the value policy is built for 2-bit values and 2-bit keys");
  using TL = Tile<D, R, VQ2, NB, VP>;
  constexpr int RU = R > 0 ? R : 1;
  constexpr int NKT = D / 32, NCT = D / 16, NG = D / 32;
  using ST = Stage<D, R, VQ2, NB, VP>;
  __shared__ u32x4 tile_s[2][TL::CHUNKS];
  __shared__ float qs[kCols][D];        // scaled queries of the workgroup's columns
  __shared__ float qu_s[kCols][RU];     // U^T q (scaled)
  __shared__ float inv_scale_s[kCols];  // 2^e undoing the per-column query scale

  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64), n = lane % 16, quad = lane / 16;
  const int g = a.gqa, hq0 = h * g;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t n_cols = a.n_q * g, col0 = (int64_t)blockIdx.x * kCols;
  const int64_t L = a.start + a.n_q, n_full = L / kGroup * kGroup, Lrow = L;
  // tokens attended by column c (query token c / g at position start + c / g); 0 past the columns
  auto n_att_of = [&](int64_t c) -> int64_t { return c < n_cols ? a.start + c / g + 1 : 0; };

  // ---- prologue: queries of the workgroup's columns (in log2 units: times log2(e)/sqrt(d)),
  // per-column power-of-two scale, U^T q
  const float qscale = kLog2e / sqrtf((float)D);
  for (int i = tid; i < kCols * D; i += kThreads) {
    const int cl = i / D, c = i % D;
    const int64_t col = col0 + cl;
    float x = 0.0f;
    if (col < n_cols) {
      const int64_t qi = (((int64_t)b * a.n_q + col / g) * a.hq + hq0 + col % g) * D + c;
      x = a.query_bf16 ? __uint_as_float((uint32_t)((const uint16_t*)a.q)[qi] << 16) : ((const float*)a.q)[qi];
    }
    qs[cl][c] = x * qscale;
  }
  __syncthreads();
  {
    const int cl = tid / 4, k = tid % 4;  // 4 threads per column
    float mx = 0.0f;
    for (int c = k; c < D; c += 4) mx = fmaxf(mx, fabsf(qs[cl][c]));
    mx = fmaxf(mx, __shfl_xor(mx, 1, 4));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 4));
    int e = 0;
    if (mx > 0.0f) frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
    for (int c = k; c < D; c += 4) qs[cl][c] = ldexpf(qs[cl][c], -e);
    if (k == 0) inv_scale_s[cl] = ldexpf(1.0f, e);
  }
  __syncthreads();
  if constexpr (R > 0) {
    const float* Uh = a.U + (int64_t)h * D * R;
    for (int i = tid; i < kCols * R; i += kThreads) {
      const int cl = i / R, r = i % R;
      float acc = 0.0f;
      for (int c = 0; c < D; ++c) acc = fmaf(Uh[c * R + r], qs[cl][c], acc);
      qu_s[cl][r] = a.corr_scale * acc;  // the correction's scale rides on U^T q
    }
  }
  __syncthreads();

  const int cl = 16 * wave + n;  // this lane's column
  const int64_t col = col0 + cl;
  const int64_t n_att = n_att_of(col);
  Fixed<D, R> f;
#pragma unroll
  for (int t = 0; t < NKT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = qs[cl][(D / 4) * quad + 8 * t + j];
      f.bq_hi[t][j] = f16_hi(x);
      f.bq_lo[t][j] = f16_lo(x);
    }
  f.inv_scale = inv_scale_s[cl];
  if constexpr (R == 32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f.bu_hi8[j] = f16_hi(qu_s[cl][8 * quad + j]);
      f.bu_lo8[j] = f16_lo(qu_s[cl][8 * quad + j]);
    }
  } else if constexpr (R > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * quad + j;
      const float x = r < R ? qu_s[cl][r] : 0.0f;
      f.bu_hi4[j] = f16_hi(x);
      f.bu_lo4[j] = f16_lo(x);
    }
  }
  float* lg_row = nullptr;
  if (a.logits_dbg && col < n_cols)
    lg_row = a.logits_dbg + (((int64_t)b * a.n_q + col / g) * a.hq + hq0 + col % g) * Lrow;

  // the wave's and the workgroup's token limits (columns are in token order)
  const int64_t wc0 = col0 + 16 * wave;
  const int64_t wc1 = (wc0 + 15 < n_cols ? wc0 + 15 : n_cols - 1);
  const int64_t att_min_w = n_att_of(wc0), att_max_w = wc0 < n_cols ? n_att_of(wc1) : 0;
  const int64_t wg_last = col0 + kCols - 1 < n_cols ? col0 + kCols - 1 : n_cols - 1;
  const int64_t att_max_wg = n_att_of(wg_last);
  int64_t G = (att_max_wg + kGroup - 1) / kGroup;  // groups any column of the workgroup reaches
  if (G > n_full / kGroup) G = n_full / kGroup;     // whole groups only; the rest is in the tails

  floatx4 o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o_acc[ct] = (floatx4){0.f, 0.f, 0.f, 0.f};
  float z_acc[NG];
#pragma unroll
  for (int cg = 0; cg < NG; ++cg) z_acc[cg] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // ---- the stream's whole groups, staged by the workgroup (double-buffered)
  // groups in flight in registers: a ring of PD sets, so a group's loads have PD - 1 group steps
  // to arrive before it is staged
  constexpr int PD = 3;
  u32x4 pf[PD][ST::KV];
  uint32_t pidx[PD];  // VP > 0: each group's index word (one uniform load)
  // the arrays of this stream: byte base and size of the region the group offsets index
  const int64_t groups_cap = a.cap / kGroup;
  auto arr_base = [&](int i) -> const char* {  // i is a compile-time constant at every use
    switch (i) {
      case 0: return (const char*)a.kcode;
      case 1: return (const char*)a.kmeta;
      case 2: return (const char*)a.scode;
      case 3: return (const char*)a.ssc;
      case 4: return (const char*)a.vmeta;
      case 5: return VQ2 ? (const char*)a.vcode : (const char*)a.vdense;
      default: return (const char*)a.vprot;
    }
  };
  // piece 4 * j + wave of a group: its array A (wave-uniform, by scalar compares) and chunk
  auto piece_array = [&](int q) {
    int A = 0;
#pragma unroll
    for (int i = 1; i < ST::NARR; ++i) A = (ST::pieces(i) > 0 && q >= ST::first(i)) ? i : A;
    return A;
  };
  auto fetch_into = [&](u32x4* dst, uint32_t& idx, int64_t gi) {
    // contiguous caches: one resource per stream and array, the group by offset; paged caches:
    // the group's block (page * Hkv + h) as its own resource
    const bool paged = a.map.block_table != nullptr;
    const int64_t blk = paged ? a.map.block(b, h, gi) : bh * groups_cap;
#pragma unroll
    for (int j = 0; j < ST::KV; ++j) {
      const int q = 4 * j + wave, A = piece_array(q);
      const char* base = arr_base(0);
      int bytes = ST::BYTES[0], first = 0;
#pragma unroll
      for (int i = 1; i < ST::NARR; ++i)
        if (A == i) {
          base = arr_base(i);
          bytes = ST::BYTES[i];
          first = ST::first(i);
        }
      const __amdgpu_buffer_rsrc_t rs = stage_rsrc(base + blk * bytes, paged ? bytes : groups_cap * bytes);
      const int soff = __builtin_amdgcn_readfirstlane(paged ? 0 : (int)(gi * bytes));
      // every lane loads (a chunk past the array's end, or a piece past the group's, reads beyond
      // the group and is not staged), so each step issues the same loads and its waits count exactly
      dst[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (64 * (q - first) + lane), soff, 0);
    }
    if constexpr (VP > 0) {
      const __amdgpu_buffer_rsrc_t ri = stage_rsrc(a.vpidx + blk, paged ? 4 : groups_cap * 4);
      idx = __builtin_amdgcn_raw_buffer_load_b32(ri, 0, __builtin_amdgcn_readfirstlane(paged ? 0 : (int)(gi * 4)), 0);
    }
  };
  auto stage_from = [&](const u32x4* src, uint32_t idx, int buf) {
#pragma unroll
    for (int j = 0; j < ST::KV; ++j) {
      const int q = 4 * j + wave, A = piece_array(q);
      int off = ST::OFF[0], chunks = ST::chunks(0), first = 0;
#pragma unroll
      for (int i = 1; i < ST::NARR; ++i)
        if (A == i) {
          off = ST::OFF[i];
          chunks = ST::chunks(i);
          first = ST::first(i);
        }
      const int chunk = 64 * (q - first) + lane;
      if (q < ST::first(ST::NARR) && chunk < chunks) tile_s[buf][off / 16 + chunk] = src[j];
    }
    if constexpr (VP > 0)
      if (tid == 0) reinterpret_cast<uint32_t*>(tile_s[buf])[TL::OFF_VI / 4] = idx;
  };
  // Requests are unconditional (indices past the last group read the last group again, unused),
  // so every step issues the same loads in the same order and each wait counts exactly.
  auto clamp_g = [&](int64_t x) { return x < G ? x : G - 1; };
  if (G > 0) {
#pragma unroll
    for (int k = 0; k < PD; ++k) fetch_into(pf[k], pidx[k], clamp_g(k));
    stage_from(pf[0], pidx[0], 0);
  }
  __syncthreads();
  for (int64_t g0 = 0; g0 < G; g0 += PD) {
#pragma unroll
    for (int k = 0; k < PD; ++k) {
      const int64_t gi = g0 + k;
      if (gi >= G) break;
      fetch_into(pf[k], pidx[k], clamp_g(gi + PD));  // set k held group gi, staged in the step before
      const int64_t tok0 = gi * kGroup;
      if (tok0 < att_max_w)
        group_step<D, R, VQ2, NB, VP>(reinterpret_cast<const uint8_t*>(tile_s[gi & 1]), f, (int)tok0,
                                  tok0 + kGroup > att_min_w, (int)n_att, lg_row, n, quad, lane, o_acc, z_acc, m_run,
                                  l_run);
      stage_from(pf[(k + 1) % PD], pidx[(k + 1) % PD], (int)((gi + 1) & 1));  // group gi + 1 (past the end: unused)
      __syncthreads();
    }
  }

  // ---- the cache's unfinished group, for the columns that reach it
  const int tail_len = (int)(L - n_full);
  if (tail_len > 0 && att_max_w > n_full)
    tail_step<D>(a, bh, n_full, tail_len, n_att, qs[cl], f.inv_scale, lg_row, n, quad, o_acc, z_acc,
                 VQ2 ? NG : 0, m_run, l_run);

  if constexpr (VQ2) {
    // zero part of the 2-bit values: sum over the four token quads, added to every channel of
    // its group (channel 16*ct + 4*quad + j lies in group ct/2)
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) {
      float z = z_acc[cg];
      z = quad_sum(z);
      o_acc[2 * cg] += z;
      o_acc[2 * cg + 1] += z;
    }
  }
  l_run = quad_sum(l_run);
  if (col < n_cols) {
    const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    const int64_t orow = (((int64_t)b * a.n_q + col / g) * a.hq + hq0 + col % g) * D;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float o = o_acc[ct][j] * inv_l;
        const int c = 16 * ct + 4 * quad + j;
        if (a.out_bf16)
          ((__bf16*)a.out)[orow + c] = (__bf16)o;
        else
          ((float*)a.out)[orow + c] = o;
      }
  }
}

template <int D, bool VQ2, bool NB, int VP>
hipError_t launch_rp(const PrefillArgs& a, hipStream_t s) {
  const int64_t n_cols = a.n_q * a.gqa;
  dim3 grid((unsigned)((n_cols + kCols - 1) / kCols), (unsigned)a.hkv, (unsigned)a.batch);
  switch (a.r) {
    case 0: hipLaunchKernelGGL((prefill_mfma_kernel<D, 0, VQ2, NB, VP>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((prefill_mfma_kernel<D, 4, VQ2, NB, VP>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((prefill_mfma_kernel<D, 8, VQ2, NB, VP>), grid, dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((prefill_mfma_kernel<D, 16, VQ2, NB, VP>), grid, dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((prefill_mfma_kernel<D, 32, VQ2, NB, VP>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool VQ2, bool NB>
hipError_t launch_r(const PrefillArgs& a, hipStream_t s) {
  if constexpr (VQ2 && !NB) {
    if (a.value_protect == 1) return launch_rp<D, true, false, 1>(a, s);
    if (a.value_protect == 2) return launch_rp<D, true, false, 2>(a, s);
  }
  if (a.value_protect) return hipErrorInvalidValue;
  return launch_rp<D, VQ2, NB, 0>(a, s);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  const bool q2 = a.value_mode == HEADQ_V_Q2;
  if (a.key_nib) {
    if (a.d == 64) return q2 ? launch_r<64, true, true>(a, s) : launch_r<64, false, true>(a, s);
    if (a.d == 128) return q2 ? launch_r<128, true, true>(a, s) : launch_r<128, false, true>(a, s);
  } else {
    if (a.d == 64) return q2 ? launch_r<64, true, false>(a, s) : launch_r<64, false, false>(a, s);
    if (a.d == 128) return q2 ? launch_r<128, true, false>(a, s) : launch_r<128, false, false>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace headq
