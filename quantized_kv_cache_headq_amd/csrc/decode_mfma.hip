// decode_mfma.hip — headq_decode_attn on gfx950 matrix cores (dense bf16 values).
//
// HeadQ technical summary ("Technische Samenvatting"), §3 step 3 (Cache Uitlezen): the runtime
// query decodes the side code through U_h^T q, the logit is corrected additively,
//     s_j = q.k_base_j / sqrt(d) + (U_h^T q).z_hat_j / sqrt(d),
// and the output is the softmax readout sum_j p_j v_j (§1, §2.2).
//
// The g = Hq/Hkv query heads of a KV head share every cached row, so both contractions of a
// 32-token group are GQA-grouped matrix products and run on MFMA:
//   scores^T [32 tok x 16 heads] = codes [tok x d] . (q o s)^T [d x heads]     (+ q.z per head)
//                                  + zc [tok x r] . (U^T q)^T [r x heads] scaled by sigma_j
//   out^T    [d x 16 heads]     += V^T [d x 32 tok] . P^T [tok x heads]
// Operand precision: the 2-bit codes, the offset-binary side codes and the binary16 zeros are
// exact in f16; bf16 values are exact in bf16. The f32 factors (q o s, q, U^T q, p) are split
// into a high and a low half-precision part and contracted twice, which keeps ~22 bits (f16)
// or ~16 bits (bf16) of each factor; accumulation is f32. The query is scaled per head by a
// power of two so that |q| <= 1, which keeps q o s inside the f16 range for any valid cache.
//
// Layouts (lane L of a wave64, n = L % 16, quad = L / 16):
//   A operand of 16x16x32: row L%16, k = 8*quad + j (j = 0..7); B: column L%16, same k;
//   result D[row][col]: column L%16, rows 4*quad + j (j = 0..3).
//   QK rows are tokens: tile T row i <-> token 8*(i/4) + 4*T + i%4, so lane L ends up holding
//   the 8 scores of tokens 8*quad .. 8*quad+7 for head n, exactly the B operand of the P.V
//   product; the channel order inside a K-step is 32*quad + 8*t + j (d = 128) so every lane
//   reads one contiguous 8-byte piece of each packed key row.
//   Dense values are stored channel-major within a group, so the V^T operand of a lane is one
//   16-byte load.
// Online softmax per head in log2 units with a lazy maximum (rescaling only when the group max
// exceeds the running max by more than 8), per-lane partial sums, and a 4-wave merge in LDS.
#include <hip/hip_runtime.h>

#include "headq_internal.h"

namespace headq {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;  // rescale only when the max grows by more than 2^8

template <class T, class S>
__device__ __forceinline__ T bitcast(const S& s) {
  static_assert(sizeof(T) == sizeof(S), "size");
  return __builtin_bit_cast(T, s);
}

// 8 two-bit codes (bits 2j..2j+1 of the low 16 bits of x) -> 8 exact f16 values 0..3.
__device__ __forceinline__ half8_t codes8_f16(uint32_t x16) {
  const uint32_t y = x16 | (x16 << 14);  // code 2p at bits 4p, code 2p+1 at bits 4p+16
  u32x4 w;
  w[0] = (y & 0x00030003u) | 0x64006400u;  // f16 1024 + code
  w[1] = ((y >> 4) & 0x00030003u) | 0x64006400u;
  w[2] = ((y >> 8) & 0x00030003u) | 0x64006400u;
  w[3] = ((y >> 12) & 0x00030003u) | 0x64006400u;
  return bitcast<half8_t>(w) - (half8_t)(_Float16)1024.0f;
}

// 4 offset-binary nibbles (low 16 bits of x, component i at bits 4i) -> 4 exact f16 values u - 8.
__device__ __forceinline__ half4_t nibbles4_f16(uint32_t x16) {
  const uint32_t y = x16 | (x16 << 12);  // nibble 0 at 0, 1 at 16, 2 at 8, 3 at 24
  u32x2 w;
  w[0] = (y & 0x000F000Fu) | 0x64006400u;
  w[1] = ((y >> 8) & 0x000F000Fu) | 0x64006400u;
  return bitcast<half4_t>(w) - (half4_t)(_Float16)1032.0f;
}

// x ~ hi + lo with both halves in f16 (hi rounded to nearest, lo the rounded remainder).
__device__ __forceinline__ _Float16 f16_hi(float x) { return (_Float16)x; }
__device__ __forceinline__ _Float16 f16_lo(float x) { return (_Float16)(x - (float)(_Float16)x); }

__device__ __forceinline__ floatx4 mfma_f16(const half8_t& a, const half8_t& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8_t& a, const bf16x8_t& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma_f16k16(const half4_t& a, const half4_t& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Raw bytes of one 32-token group as one lane needs them (filled one group ahead).
template <int D, int R>
struct GroupRaw {
  static constexpr int NKT = D / 32;   // K-steps of 32 channels
  static constexpr int NCT = D / 16;   // channel tiles of the P.V product
  static constexpr int KB = D / 16;    // key-code bytes per lane per token (8 at d=128, 4 at d=64)
  uint32_t kc[2][KB / 4];              // packed codes of the lane's row token, tiles 0 and 1
  u32x4 s[NKT];                        // binary16 steps of the lane's channels
  u32x4 z[NKT];                        // binary16 zeros of the lane's channels
  uint32_t sc[2];                      // side-code bits of the row token, tiles 0 and 1
  u32x4 sig;                           // binary16 sigma of tokens 8*quad .. 8*quad+7
  u32x4 v[NCT];                        // values: channel 16*ct + n, tokens 8*quad .. +7
};

template <int D, int R>
__device__ __forceinline__ void load_group(GroupRaw<D, R>& g, const DecodeArgs& a, int64_t bh, int64_t gi, int n,
                                           int quad) {
  constexpr int NKT = D / 32, NCT = D / 16, KB = D / 16;
  const int row_tok0 = 8 * (n / 4) + (n % 4);  // token of this lane's row in tile 0 (tile 1: +4)
  const int64_t tok_base = bh * a.cap + gi * kGroup;
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const uint8_t* row = a.kcode + (tok_base + row_tok0 + 4 * T) * (D / 4) + KB * quad;
    if constexpr (KB == 8) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(row);
      g.kc[T][0] = w[0];
      g.kc[T][1] = w[1];
    } else {
      g.kc[T][0] = *reinterpret_cast<const uint32_t*>(row);
    }
  }
  const uint16_t* meta = a.kmeta + (bh * (a.cap / kGroup) + gi) * 2 * D;
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    const int c0 = (D / 4) * quad + 8 * t;  // first channel of this K-step in this lane
    g.s[t] = *reinterpret_cast<const u32x4*>(meta + c0);
    g.z[t] = *reinterpret_cast<const u32x4*>(meta + D + c0);
  }
  if constexpr (R > 0) {
    constexpr int SB = R / 2;  // side-code bytes per token
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const uint8_t* srow = a.scode + (tok_base + row_tok0 + 4 * T) * SB;
      if constexpr (R == 32)
        g.sc[T] = *reinterpret_cast<const uint32_t*>(srow + 4 * quad);
      else if constexpr (R == 16)
        g.sc[T] = *reinterpret_cast<const uint16_t*>(srow + 2 * quad);
      else  // R == 8 (quads 0,1) or R == 4 (quad 0)
        g.sc[T] = (2 * quad < SB) ? *reinterpret_cast<const uint16_t*>(srow + 2 * quad) : 0u;
    }
    g.sig = *reinterpret_cast<const u32x4*>(a.ssc + tok_base + 8 * quad);
  }
  const uint16_t* vg = (const uint16_t*)a.vdense + (bh * (a.cap / kGroup) + gi) * (int64_t)D * kGroup;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) g.v[ct] = *reinterpret_cast<const u32x4*>(vg + (16 * ct + n) * kGroup + 8 * quad);
}

// One 32-token group: scores, online-softmax update, P.V accumulation.
template <int D, int R>
__device__ __forceinline__ void process_group(const GroupRaw<D, R>& cur, const DecodeArgs& a, int64_t gi, int b,
                                              int hq0, int g, int n, int quad, const half8_t* bq_hi,
                                              const half8_t* bq_lo, const half4_t& bu_hi4, const half4_t& bu_lo4,
                                              const half8_t& bu_hi8, const half8_t& bu_lo8, float inv_scale,
                                              float kappa, floatx4* o_acc, float& m_run, float& l_run) {
  constexpr int NKT = D / 32, NCT = D / 16;
  // scores^T tiles: start from the zero term q.z (same for every token row), add codes.(q o s)
  floatx4 cz = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    const half8_t zt = bitcast<half8_t>(cur.z[t]);
    cz = mfma_f16(zt, bq_hi[t], cz);
    cz = mfma_f16(zt, bq_lo[t], cz);
  }
  floatx4 acc[2] = {cz, cz};
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    const half8_t st = bitcast<half8_t>(cur.s[t]);
    // (q o s) as hi + lo f16: exact product error by fma, plus the low part of q times s
    const half8_t p_hi = bq_hi[t] * st;
    const half8_t e = __builtin_elementwise_fma(bq_hi[t], st, -p_hi);
    const half8_t p_lo = __builtin_elementwise_fma(bq_lo[t], st, e);
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      uint32_t x16;
      if constexpr (D == 128)
        x16 = (t & 1) ? (cur.kc[T][t >> 1] >> 16) : (cur.kc[T][t >> 1] & 0xffffu);
      else
        x16 = (t & 1) ? (cur.kc[T][0] >> 16) : (cur.kc[T][0] & 0xffffu);
      const half8_t ac = codes8_f16(x16);
      acc[T] = mfma_f16(ac, p_hi, acc[T]);
      acc[T] = mfma_f16(ac, p_lo, acc[T]);
    }
  }
  float sv[8];  // scores (log2 units) of tokens 8*quad + j for head n
  if constexpr (R > 0) {
    floatx4 cr[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      cr[T] = (floatx4){0.f, 0.f, 0.f, 0.f};
      if constexpr (R == 32) {
        const uint32_t w = cur.sc[T];
        const half4_t lo4 = nibbles4_f16(w & 0xffffu), hi4 = nibbles4_f16(w >> 16);
        const half8_t az = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        cr[T] = mfma_f16(az, bu_hi8, cr[T]);
        cr[T] = mfma_f16(az, bu_lo8, cr[T]);
      } else {
        const half4_t az = nibbles4_f16(cur.sc[T]);
        cr[T] = mfma_f16k16(az, bu_hi4, cr[T]);
        cr[T] = mfma_f16k16(az, bu_lo4, cr[T]);
      }
    }
    const half8_t sg = bitcast<half8_t>(cur.sig);
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sv[4 * T + j] = inv_scale * fmaf(kappa * (float)sg[4 * T + j], cr[T][j], acc[T][j]);
  } else {
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j) sv[4 * T + j] = inv_scale * acc[T][j];
  }
  if (a.logits_dbg && n < g) {
    float* dst = a.logits_dbg + ((int64_t)b * a.hq + hq0 + n) * a.n_ctx + gi * kGroup + 8 * quad;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = sv[j] * kLn2;
  }

  // online softmax (lazy maximum)
  float mx = sv[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const bool grow = mx > m_run + kLazyMax;  // true on the first group (m_run = -inf)
  if (__any(grow)) {
    const float m_new = grow ? mx : m_run;
    const float alpha = exp2f(m_run - m_new);  // 0 on the first group, 1 if unchanged
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) o_acc[ct] *= alpha;
  }
  bf16x8_t p_hi, p_lo;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float p = exp2f(sv[j] - m_run);
    l_run += p;
    const __bf16 ph = (__bf16)p;
    p_hi[j] = ph;
    p_lo[j] = (__bf16)(p - (float)ph);
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const bf16x8_t av = bitcast<bf16x8_t>(cur.v[ct]);
    o_acc[ct] = mfma_bf16(av, p_hi, o_acc[ct]);
    o_acc[ct] = mfma_bf16(av, p_lo, o_acc[ct]);
  }
}

template <int D, int R>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NKT = D / 32, NCT = D / 16;
  constexpr int RU = R > 0 ? R : 1;
  __shared__ float qs[kMaxGqa][D];            // scaled queries
  __shared__ float qu_s[kMaxGqa][RU];         // U^T q (scaled)
  __shared__ float inv_scale_s[kMaxGqa];      // 2^e undoing the per-head query scale
  __shared__ float m_w[kWaves][kMaxGqa], l_w[kWaves][kMaxGqa];
  __shared__ float o_w[kWaves][kMaxGqa][D];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int n = lane % 16, quad = lane / 16;
  const int g = a.gqa;
  const int hq0 = h * g;
  const int64_t bh = (int64_t)b * a.hkv + h;

  // ---- prologue (whole workgroup): q_bar = q * log2(e)/sqrt(d), per-head power-of-two scale, U^T q
  const float qscale = kLog2e / sqrtf((float)D);
  for (int i = tid; i < kMaxGqa * D; i += kThreads) {
    const int hh = i / D, c = i % D;
    float x = 0.0f;
    if (hh < g) {
      const int64_t qi = ((int64_t)b * a.hq + hq0 + hh) * D + c;
      x = a.query_bf16 ? __uint_as_float((uint32_t)((const uint16_t*)a.q)[qi] << 16) : ((const float*)a.q)[qi];
    }
    qs[hh][c] = x * qscale;
  }
  __syncthreads();
  {
    const int hh = tid / 16, k = tid % 16;  // 16 lanes per head
    float mx = 0.0f;
    for (int c = k; c < D; c += 16) mx = fmaxf(mx, fabsf(qs[hh][c]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
    int e = 0;
    if (mx > 0.0f) frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
    for (int c = k; c < D; c += 16) qs[hh][c] = ldexpf(qs[hh][c], -e);
    if (k == 0) inv_scale_s[hh] = ldexpf(1.0f, e);
  }
  __syncthreads();
  if constexpr (R > 0) {
    const float* Uh = a.U + (int64_t)h * D * R;
    for (int i = tid; i < kMaxGqa * R; i += kThreads) {
      const int hh = i / R, r = i % R;
      float acc = 0.0f;
      if (hh < g)
        for (int c = 0; c < D; ++c) acc = fmaf(Uh[c * R + r], qs[hh][c], acc);
      qu_s[hh][r] = acc;
    }
  }
  __syncthreads();

  // ---- per-lane fixed operands
  half8_t bq_hi[NKT], bq_lo[NKT];  // q_bar (scaled) of head n, lane channels, hi/lo f16
#pragma unroll
  for (int t = 0; t < NKT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = qs[n][(D / 4) * quad + 8 * t + j];
      bq_hi[t][j] = f16_hi(x);
      bq_lo[t][j] = f16_lo(x);
    }
  const float inv_scale = inv_scale_s[n];
  half4_t bu_hi4, bu_lo4;  // U^T q for ranks 4*quad + j (16x16x16 path: r = 4, 8, 16)
  half8_t bu_hi8, bu_lo8;  // ranks 8*quad + j (16x16x32 path: r = 32)
  if constexpr (R == 32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bu_hi8[j] = f16_hi(qu_s[n][8 * quad + j]);
      bu_lo8[j] = f16_lo(qu_s[n][8 * quad + j]);
    }
  } else if constexpr (R > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * quad + j;
      const float x = r < R ? qu_s[n][r] : 0.0f;
      bu_hi4[j] = f16_hi(x);
      bu_lo4[j] = f16_lo(x);
    }
  }
  const float kappa = a.corr_scale;

  floatx4 o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o_acc[ct] = (floatx4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  // ---- this wave's groups
  const int64_t n_groups = a.n_ctx / kGroup;
  const int64_t chunk = (int64_t)split * kWaves + wave;
  const int64_t g_begin = chunk * a.groups_per_split;
  int64_t g_end = g_begin + a.groups_per_split;
  if (g_end > n_groups) g_end = n_groups;

  GroupRaw<D, R> ga, gb;  // ping-pong register sets: one group computed while the next loads
  if (g_begin < g_end) load_group<D, R>(ga, a, bh, g_begin, n, quad);
  for (int64_t gi = g_begin; gi < g_end; gi += 2) {
    if (gi + 1 < g_end) load_group<D, R>(gb, a, bh, gi + 1, n, quad);
    process_group<D, R>(ga, a, gi, b, hq0, g, n, quad, bq_hi, bq_lo, bu_hi4, bu_lo4, bu_hi8, bu_lo8, inv_scale, kappa,
                        o_acc, m_run, l_run);
    if (gi + 1 >= g_end) break;
    if (gi + 2 < g_end) load_group<D, R>(ga, a, bh, gi + 2, n, quad);
    process_group<D, R>(gb, a, gi + 1, b, hq0, g, n, quad, bq_hi, bq_lo, bu_hi4, bu_lo4, bu_hi8, bu_lo8, inv_scale,
                        kappa, o_acc, m_run, l_run);
  }

  // ---- merge the 4 waves of this workgroup, write the split partial
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (quad == 0) {
    m_w[wave][n] = m_run;
    l_w[wave][n] = l_run;
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) o_w[wave][n][16 * ct + 4 * quad + j] = o_acc[ct][j];
  __syncthreads();
  for (int i = tid; i < g * D; i += kThreads) {
    const int hh = i / D, c = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_w[w][hh]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (m_w[w][hh] == -INFINITY) continue;
        const float f = exp2f(m_w[w][hh] - M);
        L = fmaf(l_w[w][hh], f, L);
        O = fmaf(o_w[w][hh][c], f, O);
      }
    }
    const int64_t row = ((int64_t)b * a.hq + hq0 + hh) * a.n_splits + split;
    a.ws_o[row * D + c] = O;
    if (c == 0) {
      a.ws_ml[row * 2] = M;
      a.ws_ml[row * 2 + 1] = L;
    }
  }
}

template <int D>
hipError_t launch_r(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.n_splits, (unsigned)a.hkv, (unsigned)a.batch);
  switch (a.r) {
    case 0: hipLaunchKernelGGL((decode_mfma_kernel<D, 0>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<D, 4>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<D, 8>), grid, dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<D, 16>), grid, dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((decode_mfma_kernel<D, 32>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma_split(const DecodeArgs& a, hipStream_t s) {
  if (a.d == 64) return launch_r<64>(a, s);
  if (a.d == 128) return launch_r<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace headq
