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
// exact f16 values, bf16 values are exact. (Feeding the codes as f16 subnormals, code * 2^-24,
// would save two instructions per operand register but measurably loses accumulation precision
// on the matrix cores: mean logit error 5e-5 instead of 4e-7 relative.) The f32 factors
// (q o s, q, U^T q, p) are split into a high and a low half-precision part and contracted
// twice, which keeps ~22 bits (f16) or ~16 bits (bf16) of each factor; accumulation is f32.
// The query is scaled per head by a power of two so that |q| <= 1, which keeps q o s inside
// the f16 range for any valid cache.
//
// Layouts (lane L of a wave64, n = L % 16, quad = L / 16):
//   A operand of 16x16x32: row L%16, k = 8*quad + j (j = 0..7); B: column L%16, same k;
//   result D[row][col]: column L%16, rows 4*quad + j (j = 0..3).
//   QK rows are tokens: tile T row i <-> token 8*(i/4) + 4*T + i%4, so lane L ends up holding
//   the 8 scores of tokens 8*quad .. 8*quad+7 for head n, exactly the B operand of the P.V
//   product; the channel order inside a K-step is (d/4)*quad + 8*t + j so every lane reads one
//   contiguous piece of each packed key row.
//   Dense values are stored channel-major within a group, so the V^T operand of a lane is one
//   16-byte load.
// Memory: every load is a buffer load with the (b, h) stream base in SGPRs, the lane offset in
// a VGPR fixed for the whole kernel and the group offset in an SGPR. A wave prefetches the next
// group into registers while it computes the current one; the per-group step/zero row (read by
// 16 lanes each) goes through a wave-private LDS slot instead of 16 redundant loads.
// Online softmax per head in log2 units with a lazy maximum (rescaling only when the group max
// exceeds the running max by more than 8), per-lane partial sums, and a 4-wave merge in LDS.
// Splits of a stream are merged in the same launch: each workgroup publishes its partial,
// fences, and counts itself in on the stream's workspace counter; the last one merges by
// log-sum-exp, writes the output and zeroes the counter again.
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
constexpr float kLazyMax = 8.0f;          // rescale only when the max grows by more than 2^8
constexpr int kBufferConfig = 0x00020000; // raw buffer resource, dword 3
constexpr int kStream = 2;                 // cache policy "nt": the cache is read once per call

template <class T, class S>
__device__ __forceinline__ T bitcast(const S& s) {
  static_assert(sizeof(T) == sizeof(S), "size");
  return __builtin_bit_cast(T, s);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > 0x7fffffff ? 0x7fffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kBufferConfig);
}

// 8 two-bit codes laid out as "code 2p at bit 4p, code 2p+1 at bit 4p+16" -> 8 exact f16
// values 0..3 (built as the f16 1024 + code, then 1024 subtracted in packed f16).
__device__ __forceinline__ half8_t codes8_f16(uint32_t y) {
  u32x4 w;
  w[0] = (y & 0x00030003u) | 0x64006400u;
  w[1] = ((y >> 4) & 0x00030003u) | 0x64006400u;
  w[2] = ((y >> 8) & 0x00030003u) | 0x64006400u;
  w[3] = ((y >> 12) & 0x00030003u) | 0x64006400u;
  return bitcast<half8_t>(w) - (half8_t)(_Float16)1024.0f;
}
// Rearrange one 32-bit word of packed codes (code j at bits 2j) for codes8_f16: low and high
// 16-bit halves, each with its odd codes moved up by 14 bits.
__device__ __forceinline__ uint32_t spread_lo(uint32_t w) { return (w & 0xffffu) | ((w << 14) & 0xffff0000u); }
__device__ __forceinline__ uint32_t spread_hi(uint32_t w) { return (w >> 16) | ((w >> 2) & 0xffff0000u); }

// 4 offset-binary nibbles (low 16 bits of x, component i at bits 4i) -> 4 exact f16 values u - 8.
__device__ __forceinline__ half4_t nibbles4_f16(uint32_t x16) {
  const uint32_t y = x16 | (x16 << 12);  // nibble 0 at 0, 1 at 16, 2 at 8, 3 at 24
  u32x2 w;
  w[0] = (y & 0x000F000Fu) | 0x64006400u;  // f16 1024 + u
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

// Split partials cross workgroups (and XCDs, each with its own L2). They are written with
// agent-scope stores (write-through to the device coherence point) and read with agent-scope
// loads, so no L2-wide write-back or invalidate is needed; a workgroup counts itself in on the
// stream's counter only after its stores have completed (s_waitcnt on the memory counter).
__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fetch(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0): every store acknowledged
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ void lds_wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Wave-uniform view of one (b, h) stream of the cache.
struct Stream {
  __amdgpu_buffer_rsrc_t kcode, kmeta, scode, ssc, v;
};

// Key-side bytes of one 32-token group, staged per wave in LDS in this order:
//   packed codes 32 x d/4 | step/zero rows 2 x d x 2 | side codes 32 x r/2 | sigma 32 x 2.
// Every array of a group is contiguous in the cache, so each is fetched with one load
// instruction in which lane L takes bytes [L*w, L*w + w) (w = 16, 8, 4, 2 or 1): fully
// coalesced, whatever pieces the matrix operands need afterwards.
template <int D, int R>
struct KSide {
  static constexpr int KC = kGroup * D / 4, KM = 4 * D, SC = kGroup * R / 2, SG = R > 0 ? kGroup * 2 : 0;
  static constexpr int OFF_KM = KC, OFF_SC = KC + KM, OFF_SG = KC + KM + SC;
  static constexpr int BYTES = (KC + KM + SC + SG + 15) / 16 * 16;
};

template <int N>
struct Bytes;  // N bytes held by one lane
template <> struct Bytes<16> { using T = u32x4; };
template <> struct Bytes<8> { using T = u32x2; };
template <> struct Bytes<4> { using T = uint32_t; };
template <> struct Bytes<2> { using T = uint16_t; };
template <> struct Bytes<1> { using T = uint8_t; };

template <int N>
__device__ __forceinline__ typename Bytes<N>::T load_piece(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  if constexpr (N == 16) return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStream);
  if constexpr (N == 8) return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStream);
  if constexpr (N == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStream);
  if constexpr (N == 2) return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kStream);
  if constexpr (N == 1) return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, kStream);
}

// Raw bytes of one 32-token group as one lane holds them (filled one group ahead).
template <int D, int R>
struct GroupRaw {
  static constexpr int NCT = D / 16;            // channel tiles of the P.V product
  typename Bytes<D / 8>::T kc;                  // lane's share of the packed codes
  typename Bytes<D / 16>::T km;                 // lane's share of the step/zero rows
  typename Bytes<(R > 0 ? R / 4 : 1)>::T sc;    // lane's share of the side codes
  uint8_t sg;                                   // lane's share of the sigmas
  u32x4 v[NCT];                                 // values: channel 16*ct + n, tokens 8*quad .. +7
};

template <int D, int R>
__device__ __forceinline__ void load_group(GroupRaw<D, R>& g, const Stream& s, int lane, int n, int quad,
                                           int64_t gi) {
  constexpr int NCT = D / 16;
  g.kc = load_piece<D / 8>(s.kcode, lane * (D / 8), (int)(gi * KSide<D, R>::KC));
  g.km = load_piece<D / 16>(s.kmeta, lane * (D / 16), (int)(gi * KSide<D, R>::KM));
  if constexpr (R > 0) {
    g.sc = load_piece<R / 4>(s.scode, lane * (R / 4), (int)(gi * KSide<D, R>::SC));
    g.sg = load_piece<1>(s.ssc, lane, (int)(gi * KSide<D, R>::SG));
  }
  const int v0 = (n * kGroup + 8 * quad) * 2;  // channel n (+16*ct), tokens 8*quad .. +7
  const int v_goff = (int)(gi * (D * kGroup * 2));
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int off = (ct & 3) * 1024;  // 16 channels x 32 tokens x 2 bytes per tile
    g.v[ct] = __builtin_amdgcn_raw_buffer_load_b128(s.v, ct < 4 ? v0 : v0 + 4096, v_goff + off, kStream);
  }
}

// Per-lane operands fixed for the whole kernel.
template <int D, int R>
struct Fixed {
  static constexpr int NKT = D / 32;
  half8_t bq_hi[NKT], bq_lo[NKT];  // scaled q_bar of head n at this lane's channels, hi/lo f16
  half4_t bu_hi4, bu_lo4;          // U^T q at ranks 4*quad + j (16x16x16 path)
  half8_t bu_hi8, bu_lo8;          // U^T q at ranks 8*quad + j (16x16x32 path, r = 32)
  float inv_scale;                 // 2^e: undoes the per-head query scale
  float kappa;                     // corr_scale
};

// One 32-token group: scores, online-softmax update, P.V accumulation.
template <int D, int R>
__device__ __forceinline__ void process_group(const GroupRaw<D, R>& cur, const Fixed<D, R>& f, uint8_t* slot,
                                              const DecodeArgs& a, int64_t gi, int b, int hq0, int g, int lane, int n,
                                              int quad, floatx4* o_acc, float& m_run, float& l_run) {
  constexpr int NKT = D / 32, NCT = D / 16;
  using KS = KSide<D, R>;
  // Key side through the wave's LDS slot. Lanes read what other lanes wrote, so the accesses
  // are ordered by wave-scope fences (the wave executes its LDS operations in order; the fences
  // stop the compiler from moving reads across the writes, in either direction).
  lds_wave_fence();
  *reinterpret_cast<typename Bytes<D / 8>::T*>(slot + lane * (D / 8)) = cur.kc;
  *reinterpret_cast<typename Bytes<D / 16>::T*>(slot + KS::OFF_KM + lane * (D / 16)) = cur.km;
  if constexpr (R > 0) {
    *reinterpret_cast<typename Bytes<R / 4>::T*>(slot + KS::OFF_SC + lane * (R / 4)) = cur.sc;
    slot[KS::OFF_SG + lane] = cur.sg;
  }
  lds_wave_fence();
  const _Float16* km_h = reinterpret_cast<const _Float16*>(slot + KS::OFF_KM);
  const int row_tok0 = 8 * (n / 4) + (n % 4);  // token of this lane's row in tile 0 (tile 1: +4)
  uint32_t kcw[2][D / 64];                      // packed codes of the row tokens, this lane's piece
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const uint8_t* p = slot + (row_tok0 + 4 * T) * (D / 4) + (D / 16) * quad;
    if constexpr (D == 128) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(p);
      kcw[T][0] = w[0];
      kcw[T][1] = w[1];
    } else {
      kcw[T][0] = *reinterpret_cast<const uint32_t*>(p);
    }
  }

  // zero term q.z (identical for every token row), then codes . (q o s) on top of it
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
    // (q o s) as hi + lo f16: exact product error by fma, plus the low part of q times s
    const half8_t p_hi = f.bq_hi[t] * st[t];
    const half8_t e = __builtin_elementwise_fma(f.bq_hi[t], st[t], -p_hi);
    const half8_t p_lo = __builtin_elementwise_fma(f.bq_lo[t], st[t], e);
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      const uint32_t w = kcw[T][(D == 128) ? (t >> 1) : 0];
      const half8_t ac = codes8_f16((t & 1) ? spread_hi(w) : spread_lo(w));
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
      const uint8_t* srow = slot + KS::OFF_SC + (row_tok0 + 4 * T) * (R / 2);
      if constexpr (R == 32) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(srow + 4 * quad);
        const half4_t lo4 = nibbles4_f16(w & 0xffffu), hi4 = nibbles4_f16(w >> 16);
        const half8_t az = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
        cr[T] = mfma_f16(az, f.bu_hi8, cr[T]);
        cr[T] = mfma_f16(az, f.bu_lo8, cr[T]);
      } else {
        // ranks 4*quad .. 4*quad+3; quads past the rank multiply zero operands
        const uint32_t w = (2 * quad < R / 2) ? *reinterpret_cast<const uint16_t*>(srow + 2 * quad) : 0x8888u;
        const half4_t az = nibbles4_f16(w);
        cr[T] = mfma_f16k16(az, f.bu_hi4, cr[T]);
        cr[T] = mfma_f16k16(az, f.bu_lo4, cr[T]);
      }
    }
    const half8_t sg = *reinterpret_cast<const half8_t*>(slot + KS::OFF_SG + 16 * quad);
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sv[4 * T + j] = f.inv_scale * fmaf(f.kappa * (float)sg[4 * T + j], cr[T][j], acc[T][j]);
  } else {
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j) sv[4 * T + j] = f.inv_scale * acc[T][j];
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
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int NKT = D / 32, NCT = D / 16;
  constexpr int RU = R > 0 ? R : 1;
  __shared__ float qs[kMaxGqa][D];            // scaled queries
  __shared__ float qu_s[kMaxGqa][RU];         // U^T q (scaled)
  __shared__ float inv_scale_s[kMaxGqa];      // 2^e undoing the per-head query scale
  __shared__ u32x4 kslot[kWaves][KSide<D, R>::BYTES / 16];  // per-wave key-side staging
  __shared__ float m_w[kWaves][kMaxGqa], l_w[kWaves][kMaxGqa];
  __shared__ float o_w[kWaves][kMaxGqa][D];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform per wave: keeps group offsets scalar
  const int n = lane % 16, quad = lane / 16;
  const int g = a.gqa;
  const int hq0 = h * g;
  const int64_t bh = (int64_t)b * a.hkv + h;

  // ---- query and U_h first (small; their latency is then hidden behind the group loads below)
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
  if constexpr (R > 0) {
    // U_h staged in LDS with one coalesced pass (the merge buffer is idle until the epilogue)
    static_assert(D * R <= kWaves * kMaxGqa * D, "U_h must fit the merge buffer");
    const float* Uh = a.U + (int64_t)h * D * R;
    float* U_s = &o_w[0][0][0];
    for (int i = tid; i < D * R; i += kThreads) U_s[i] = Uh[i];
  }

  // ---- stream view and schedule: the W = 4 * splits waves of a stream interleave its groups
  // (wave c takes group slots c, c + W, c + 2W, ...), so the waves reading a stream touch
  // adjacent memory at any moment; each stream starts at its own rotation so that streams are
  // not at the same relative offset together. The first two groups are requested before the
  // prologue so that their latency overlaps it.
  Stream s;
  const int64_t groups_cap = a.cap / kGroup;
  s.kcode = make_rsrc(a.kcode + bh * a.cap * (D / 4), a.cap * (D / 4));
  s.kmeta = make_rsrc(a.kmeta + bh * groups_cap * 2 * D, groups_cap * 4 * D);
  s.scode = make_rsrc(R > 0 ? a.scode + bh * a.cap * (R / 2) : a.kcode, R > 0 ? a.cap * (R / 2) : 0);
  s.ssc = make_rsrc(R > 0 ? a.ssc + bh * a.cap : a.kmeta, R > 0 ? a.cap * 2 : 0);
  s.v = make_rsrc((const uint16_t*)a.vdense + bh * a.cap * D, a.cap * D * 2);
  const int64_t n_groups = a.n_ctx / kGroup;
  const int64_t W = (int64_t)a.n_splits * kWaves;
  const int64_t rot = (bh * 40503) % n_groups;
  auto group_at = [&](int64_t j) { const int64_t x = j + rot; return x >= n_groups ? x - n_groups : x; };
  const int64_t j_begin = (int64_t)split * kWaves + wave;
  GroupRaw<D, R> ga, gb;  // ping-pong register sets: one group computed while the next loads
  if (j_begin < n_groups) load_group<D, R>(ga, s, lane, n, quad, group_at(j_begin));
  if (j_begin + W < n_groups) load_group<D, R>(gb, s, lane, n, quad, group_at(j_begin + W));
  __syncthreads();

  // ---- prologue (whole workgroup): per-head power-of-two query scale, U^T q
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
    const float* U_s = &o_w[0][0][0];
    for (int i = tid; i < kMaxGqa * R; i += kThreads) {
      const int hh = i / R, r = i % R;
      float acc = 0.0f;
      if (hh < g)
        for (int c = 0; c < D; ++c) acc = fmaf(U_s[c * R + r], qs[hh][c], acc);
      qu_s[hh][r] = acc;
    }
  }
  __syncthreads();

  // ---- per-lane fixed operands
  Fixed<D, R> f;
#pragma unroll
  for (int t = 0; t < NKT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = qs[n][(D / 4) * quad + 8 * t + j];
      f.bq_hi[t][j] = f16_hi(x);
      f.bq_lo[t][j] = f16_lo(x);
    }
  f.inv_scale = inv_scale_s[n];
  f.kappa = a.corr_scale;
  if constexpr (R == 32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f.bu_hi8[j] = f16_hi(qu_s[n][8 * quad + j]);
      f.bu_lo8[j] = f16_lo(qu_s[n][8 * quad + j]);
    }
  } else if constexpr (R > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * quad + j;
      const float x = r < R ? qu_s[n][r] : 0.0f;
      f.bu_hi4[j] = f16_hi(x);
      f.bu_lo4[j] = f16_lo(x);
    }
  }

  floatx4 o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o_acc[ct] = (floatx4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  // ---- this wave's groups
  uint8_t* slot = reinterpret_cast<uint8_t*>(kslot[wave]);
  for (int64_t j = j_begin; j < n_groups; j += 2 * W) {
    process_group<D, R>(ga, f, slot, a, group_at(j), b, hq0, g, lane, n, quad, o_acc, m_run, l_run);
    if (j + W >= n_groups) break;
    if (j + 2 * W < n_groups) load_group<D, R>(ga, s, lane, n, quad, group_at(j + 2 * W));
    process_group<D, R>(gb, f, slot, a, group_at(j + W), b, hq0, g, lane, n, quad, o_acc, m_run, l_run);
    if (j + 3 * W < n_groups) load_group<D, R>(gb, s, lane, n, quad, group_at(j + 3 * W));
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
  // one partial per workgroup: merge the waves, keep it in LDS (o_w[0], m_w[0], l_w[0]) and in
  // the workspace for the other workgroups of this stream
  __shared__ int last_s;
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
        const float fct = exp2f(m_w[w][hh] - M);
        L = fmaf(l_w[w][hh], fct, L);
        O = fmaf(o_w[w][hh][c], fct, O);
      }
    }
    const int64_t row = ((int64_t)b * a.hq + hq0 + hh) * a.n_splits + split;
    publish(a.ws_o + row * D + c, O);
    if (c == 0) {
      publish(a.ws_ml + row * 2, M);
      publish(a.ws_ml + row * 2 + 1, L);
    }
  }
  // Last workgroup of the stream to arrive merges all splits (log-sum-exp) and writes the
  // normalised output; it then returns the stream's counter to zero for the next call.
  wait_stores_done();
  __syncthreads();
  if (tid == 0) last_s = atomicAdd(a.ws_count + bh, 1u) == (uint32_t)(a.n_splits - 1);
  __syncthreads();
  if (!last_s) return;
  // (max, sum) of every split and head into LDS with one round of loads, then the weights
  // 2^(m_s - M) per head, then every split's output with independent loads per element
  const int S = a.n_splits;
  float* ml_s = &o_w[0][0][0];            // reuse: S * g pairs fit easily (S <= n_groups)
  for (int i = tid; i < S * g; i += kThreads) {
    const int hh = i / S, sp = i % S;
    const int64_t row = ((int64_t)b * a.hq + hq0 + hh) * S + sp;
    ml_s[2 * i] = fetch(a.ws_ml + row * 2);
    ml_s[2 * i + 1] = fetch(a.ws_ml + row * 2 + 1);
  }
  __syncthreads();
  if (tid < g) {
    float M = -INFINITY;
    for (int sp = 0; sp < S; ++sp) M = fmaxf(M, ml_s[2 * (tid * S + sp)]);
    float L = 0.0f;
    for (int sp = 0; sp < S; ++sp) {
      const float ms = ml_s[2 * (tid * S + sp)];
      const float wgt = ms == -INFINITY ? 0.0f : exp2f(ms - M);  // a split without tokens weighs 0
      ml_s[2 * (tid * S + sp)] = wgt;
      L = fmaf(ml_s[2 * (tid * S + sp) + 1], wgt, L);
    }
    m_w[0][tid] = 1.0f / L;
  }
  __syncthreads();
  for (int i = tid; i < g * D; i += kThreads) {
    const int hh = i / D, c = i % D;
    const int64_t row0 = ((int64_t)b * a.hq + hq0 + hh) * S;
    float O = 0.0f;
    int sp = 0;
    for (; sp + 4 <= S; sp += 4) {
      const float o0 = fetch(a.ws_o + (row0 + sp) * D + c), o1 = fetch(a.ws_o + (row0 + sp + 1) * D + c);
      const float o2 = fetch(a.ws_o + (row0 + sp + 2) * D + c), o3 = fetch(a.ws_o + (row0 + sp + 3) * D + c);
      O = fmaf(o0, ml_s[2 * (hh * S + sp)], O);
      O = fmaf(o1, ml_s[2 * (hh * S + sp + 1)], O);
      O = fmaf(o2, ml_s[2 * (hh * S + sp + 2)], O);
      O = fmaf(o3, ml_s[2 * (hh * S + sp + 3)], O);
    }
    for (; sp < S; ++sp) O = fmaf(fetch(a.ws_o + (row0 + sp) * D + c), ml_s[2 * (hh * S + sp)], O);
    const float o = O * m_w[0][hh];
    const int64_t orow = ((int64_t)b * a.hq + hq0 + hh) * D + c;
    if (a.out_bf16)
      ((__bf16*)a.out)[orow] = (__bf16)o;
    else
      ((float*)a.out)[orow] = o;
  }
  if (tid == 0) atomicExch(a.ws_count + bh, 0u);
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
