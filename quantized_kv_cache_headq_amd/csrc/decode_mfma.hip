// decode_mfma.hip — headq_decode_attn on gfx950 matrix cores (dense bf16 or 2-bit values).
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
// With 2-bit values and g <= 8, J groups share the 16 columns (process_block); with the A^2
// value policy, each group's corrections are staged with it and added after the P.V product.
#include <hip/hip_runtime.h>

#include "headq_internal.h"
#include "mfma_common.h"

namespace headq {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.0f;          // rescale only when the max grows by more than 2^8
constexpr int kBufferConfig = 0x00020000; // raw buffer resource, dword 3
constexpr int kStream = 2;                 // cache policy "nt": the cache is read once per call

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes > 0x7fffffff ? 0x7fffffffu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kBufferConfig);
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
  __amdgpu_buffer_rsrc_t kcode, kmeta, scode, ssc, v, vmeta;
  __amdgpu_buffer_rsrc_t vprot, vpidx;  // A^2 value policy (VP > 0)
};

// Bytes of one 32-token group staged per wave in LDS, in this order:
//   packed key codes 32 x d/4 | key step/zero rows 2 x d x 2 | side codes 32 x r/2 |
//   sigma 32 x 2 | (2-bit values) value step/zero rows 2 x d/32 x 32 x 2.
// Every array of a group is contiguous in the cache, so each is fetched with one load
// instruction in which lane L takes bytes [L*w, L*w + w) (w = 16, 8, 4, 2 or 1): fully
// coalesced, whatever pieces the matrix operands need afterwards.
template <int D, int R, bool VQ2, bool NB>
struct KSide {
  // key codes: 2 bits (4 per byte) or one per nibble (3- and 4-bit base codes, NB)
  static constexpr int KC = kGroup * D / (NB ? 2 : 4), KM = 4 * D, SC = kGroup * R / 2, SG = R > 0 ? kGroup * 2 : 0;
  static constexpr int VM = VQ2 ? 4 * D : 0;
  static constexpr int OFF_KM = KC, OFF_SC = KC + KM, OFF_SG = KC + KM + SC, OFF_VM = KC + KM + SC + SG;
  static constexpr int BYTES = (KC + KM + SC + SG + VM + 15) / 16 * 16;
};

template <int N>
struct Bytes;  // N bytes held by one lane
template <> struct Bytes<32> { using T = u32x8; };
template <> struct Bytes<16> { using T = u32x4; };
template <> struct Bytes<8> { using T = u32x2; };
template <> struct Bytes<4> { using T = uint32_t; };
template <> struct Bytes<2> { using T = uint16_t; };
template <> struct Bytes<1> { using T = uint8_t; };

template <int N>
__device__ __forceinline__ typename Bytes<N>::T load_piece(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  if constexpr (N == 32) {
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStream);
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, kStream);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  if constexpr (N == 16) return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStream);
  if constexpr (N == 8) return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStream);
  if constexpr (N == 4) return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStream);
  if constexpr (N == 2) return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kStream);
  if constexpr (N == 1) return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, kStream);
}

// Word w of a lane's piece (N bytes, N/4 words).
template <int N>
__device__ __forceinline__ uint32_t word_of(const typename Bytes<N>::T& x, int w) {
  if constexpr (N == 4) return x;
  else return x[w];
}

// Raw bytes of one 32-token group as one lane holds them (filled one group ahead).
template <int D, int R, bool VQ2, bool NB>
struct GroupRaw {
  static constexpr int NCT = D / 16;            // channel tiles of the P.V product
  typename Bytes<KSide<D, R, VQ2, NB>::KC / 64>::T kc;  // lane's share of the packed key codes
  typename Bytes<D / 16>::T km;                 // lane's share of the key step/zero rows
  typename Bytes<(R > 0 ? R / 4 : 1)>::T sc;    // lane's share of the side codes
  uint8_t sg;                                   // lane's share of the sigmas
  u32x4 v[VQ2 ? 1 : NCT];                       // dense: channel 16*ct + n, tokens 8*quad .. +7
  typename Bytes<D / 8>::T vc;                  // 2-bit: the lane's value codes (all tiles)
  typename Bytes<D / 16>::T vm;                 // 2-bit: lane's share of the value step/zero rows
};

template <int D, int R, bool VQ2, bool NB>
__device__ __forceinline__ void load_group(GroupRaw<D, R, VQ2, NB>& g, const Stream& s_stream, const DecodeArgs& a, int h,
                                           int page_v, int lane, int n, int quad, int gi_in) {
  using KS = KSide<D, R, VQ2, NB>;
  // the group index is wave-uniform; saying so keeps every group offset in a scalar register
  // (a per-lane offset would make the compiler loop over the lanes around each buffer load)
  int gi = __builtin_amdgcn_readfirstlane(gi_in);
  Stream s = s_stream;
  if (a.map.block_table) {
    // paged cache: this group's block in the pools (page_v from request_page), one buffer
    // resource per array from its own 64-bit base (pools may exceed the 32-bit offset range of a
    // single resource)
    int64_t page = __builtin_amdgcn_readfirstlane(page_v);
    page = page < 0 ? 0 : (page >= a.map.n_pages ? a.map.n_pages - 1 : page);
    const int64_t blk = page * a.hkv + h;
    s.kcode = make_rsrc(a.kcode + blk * KS::KC, KS::KC);
    s.kmeta = make_rsrc(a.kmeta + blk * 2 * D, KS::KM);
    if constexpr (R > 0) {
      s.scode = make_rsrc(a.scode + blk * KS::SC, KS::SC);
      s.ssc = make_rsrc(a.ssc + blk * kGroup, KS::SG);
    }
    if constexpr (VQ2) {
      s.v = make_rsrc(a.vcode + blk * (D * 8), D * 8);
      s.vmeta = make_rsrc(a.vmeta + blk * 2 * D, 4 * D);
    } else {
      s.v = make_rsrc((const uint16_t*)a.vdense + blk * D * kGroup, D * kGroup * 2);
    }
    gi = 0;
  }
  g.kc = load_piece<KS::KC / 64>(s.kcode, lane * (KS::KC / 64), gi * KS::KC);
  g.km = load_piece<D / 16>(s.kmeta, lane * (D / 16), gi * KS::KM);
  if constexpr (R > 0) {
    g.sc = load_piece<R / 4>(s.scode, lane * (R / 4), gi * KS::SC);
    g.sg = load_piece<1>(s.ssc, lane, gi * KS::SG);
  }
  if constexpr (VQ2) {
    g.vc = load_piece<D / 8>(s.v, lane * (D / 8), gi * (D * 8));
    g.vm = load_piece<D / 16>(s.vmeta, lane * (D / 16), gi * (4 * D));
  } else {
    constexpr int NCT = D / 16;
    const int v0 = (n * kGroup + 8 * quad) * 2;  // channel n (+16*ct), tokens 8*quad .. +7
    const int v_goff = gi * (D * kGroup * 2);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int off = (ct & 3) * 1024;  // 16 channels x 32 tokens x 2 bytes per tile
      g.v[ct] = __builtin_amdgcn_raw_buffer_load_b128(s.v, ct < 4 ? v0 : v0 + 4096, v_goff + off, kStream);
    }
  }
}

// Page of group gi in this row's block table (paged caches; 0 otherwise), requested one group pair
// ahead as a vector load: the wait for it then falls after the group loads issued before it (the
// vector memory counter is in order) instead of stalling the next group's requests.
__device__ __forceinline__ int request_page(const DecodeArgs& a, __amdgpu_buffer_rsrc_t table_row, int gi) {
  const int off = __builtin_amdgcn_readfirstlane(gi * 4);  // wave-uniform: no loop over the lanes
  return a.map.block_table ? (int)__builtin_amdgcn_raw_buffer_load_b32(table_row, 0, off, 0) : 0;
}

// A^2 value policy, VP corrected tokens per group (2-bit values): the lane's share of the group's
// [VP][d] bfloat16 corrections (staged in LDS like the key side) and the group's token indices.
template <int D, int VP>
struct ProtRaw {
  typename Bytes<(VP > 0 ? VP * D / 32 : 4)>::T vp;
  uint32_t idx;  // slot k: bits 8k .. 8k+7
};

template <int D, int R, bool NB, int VP>
__device__ __forceinline__ void load_prot(ProtRaw<D, VP>& p, const Stream& s_stream, const DecodeArgs& a, int h,
                                          int page_v, int lane, int gi_in) {
  constexpr int BYTES = VP * D * 2;
  int gi = __builtin_amdgcn_readfirstlane(gi_in);
  __amdgpu_buffer_rsrc_t rp = s_stream.vprot, ri = s_stream.vpidx;
  if (a.map.block_table) {
    int64_t page = __builtin_amdgcn_readfirstlane(page_v);
    page = page < 0 ? 0 : (page >= a.map.n_pages ? a.map.n_pages - 1 : page);
    const int64_t blk = page * a.hkv + h;
    rp = make_rsrc(a.vprot + blk * VP * D, BYTES);
    ri = make_rsrc(a.vpidx + blk, 4);
    gi = 0;
  }
  p.vp = load_piece<VP * D / 32>(rp, lane * (VP * D / 32), gi * BYTES);
  p.idx = __builtin_amdgcn_raw_buffer_load_b32(ri, 0, gi * 4, kStream);
}

// o += p_t * correction_t for the corrected tokens t of the lane's group (rows staged at `prow`,
// [VP][d] bf16). Token t's probability for this column is held by the lane of the same column
// with quad t / 8, slot t % 8; every lane of a column shares the group, hence the token list.
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

// Per-lane operands fixed for the whole kernel.
template <int D, int R>
struct Fixed {
  static constexpr int NKT = D / 32;
  half8_t bq_hi[NKT], bq_lo[NKT];  // scaled q_bar of head n at this lane's channels, hi/lo f16
  half4_t bu_hi4, bu_lo4;          // U^T q at ranks 4*quad + j (16x16x16 path)
  half8_t bu_hi8, bu_lo8;          // U^T q at ranks 8*quad + j (16x16x32 path, r = 32)
  float inv_scale;                 // 2^e: undoes the per-head query scale
};

// Stage the lane's raw bytes of one group into a wave's LDS slot (the caller orders the slot's
// accesses with wave fences: lanes read what other lanes wrote).
template <int D, int R, bool VQ2, bool NB>
__device__ __forceinline__ void stage_group(const GroupRaw<D, R, VQ2, NB>& cur, uint8_t* slot, int lane) {
  using KS = KSide<D, R, VQ2, NB>;
  *reinterpret_cast<typename Bytes<KS::KC / 64>::T*>(slot + lane * (KS::KC / 64)) = cur.kc;
  *reinterpret_cast<typename Bytes<D / 16>::T*>(slot + KS::OFF_KM + lane * (D / 16)) = cur.km;
  if constexpr (R > 0) {
    *reinterpret_cast<typename Bytes<R / 4>::T*>(slot + KS::OFF_SC + lane * (R / 4)) = cur.sc;
    slot[KS::OFF_SG + lane] = cur.sg;
  }
  if constexpr (VQ2) *reinterpret_cast<typename Bytes<D / 16>::T*>(slot + KS::OFF_VM + lane * (D / 16)) = cur.vm;
}

// (q o s) at this lane's channels as hi + lo f16 operands (exact product error by fma, plus the
// low part of q times s), s the key step row of the group staged in `slot`.
template <int D, int R, bool VQ2, bool NB>
__device__ __forceinline__ void query_times_step(const uint8_t* slot, const Fixed<D, R>& f, int quad, half8_t* p_hi,
                                                 half8_t* p_lo) {
  using KS = KSide<D, R, VQ2, NB>;
  const _Float16* km_h = reinterpret_cast<const _Float16*>(slot + KS::OFF_KM);
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    const half8_t st = *reinterpret_cast<const half8_t*>(km_h + (D / 4) * quad + 8 * t);
    p_hi[t] = f.bq_hi[t] * st;
    const half8_t e = __builtin_elementwise_fma(f.bq_hi[t], st, -p_hi[t]);
    p_lo[t] = __builtin_elementwise_fma(f.bq_lo[t], st, e);
  }
}

// Raw logit parts of the 32 tokens of the group staged in `slot` against the B operands of this
// lane's column: acc = q.z + codes.(q o s) and cr = zc.(U^T q), token tiles T = 0, 1. PRE: q o s
// is given (p_hi/p_lo, from query_times_step); otherwise it is formed here, k-tile by k-tile, from
// the step row of the same group.
template <int D, int R, bool VQ2, bool NB, bool PRE>
__device__ __forceinline__ void group_logits(const uint8_t* slot, const Fixed<D, R>& f, const half8_t* p_hi,
                                             const half8_t* p_lo, int n, int quad, floatx4* acc, floatx4* cr) {
  constexpr int NKT = D / 32;
  using KS = KSide<D, R, VQ2, NB>;
  const _Float16* km_h = reinterpret_cast<const _Float16*>(slot + KS::OFF_KM);
  const int row_tok0 = 8 * (n / 4) + (n % 4);  // token of this lane's row in tile 0 (tile 1: +4)
  // packed codes of the row tokens, this lane's piece (channels (d/4)*quad .. +d/4): d/64 words
  // of 2-bit codes, or d/32 nibble words
  constexpr int KW = NB ? D / 32 : D / 64;
  uint32_t kcw[2][KW];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    const uint8_t* p = slot + (row_tok0 + 4 * T) * (KS::KC / 32) + 4 * KW * quad;
#pragma unroll
    for (int w = 0; w < KW; ++w) kcw[T][w] = reinterpret_cast<const uint32_t*>(p)[w];
  }
  // zero term q.z (identical for every token row), then codes . (q o s) on top of it
  floatx4 cz = (floatx4){0.f, 0.f, 0.f, 0.f};
  half8_t st[NKT];
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    const int c0 = (D / 4) * quad + 8 * t;
    if constexpr (!PRE) st[t] = *reinterpret_cast<const half8_t*>(km_h + c0);
    const half8_t zt = *reinterpret_cast<const half8_t*>(km_h + D + c0);
    cz = mfma_f16(zt, f.bq_hi[t], cz);
    cz = mfma_f16(zt, f.bq_lo[t], cz);
  }
  acc[0] = cz;
  acc[1] = cz;
#pragma unroll
  for (int t = 0; t < NKT; ++t) {
    half8_t ph, pl;
    if constexpr (PRE) {
      ph = p_hi[t];
      pl = p_lo[t];
    } else {
      ph = f.bq_hi[t] * st[t];
      const half8_t e = __builtin_elementwise_fma(f.bq_hi[t], st[t], -ph);
      pl = __builtin_elementwise_fma(f.bq_lo[t], st[t], e);
    }
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      // k-tile t covers channels (d/4)*quad + 8t .. +7: the even (t even) or odd (t odd) run of
      // the lane's word t/2
      half8_t ac;
      if constexpr (NB) {
        ac = key_codes8_nib(kcw[T][t]);  // nibble word t: channels (d/4)*quad + 8t .. +7
      } else {
        const uint32_t w = kcw[T][(D == 128) ? (t >> 1) : 0];
        ac = key_codes8((t & 1) ? odd_codes(w) : even_codes(w));
      }
      acc[T] = mfma_f16(ac, ph, acc[T]);
      acc[T] = mfma_f16(ac, pl, acc[T]);
    }
  }
  if constexpr (R > 0) {
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
  }
}

// Scores of tokens 8*quad + j for this lane's column before the head's power-of-two scale (log2
// units once scaled): acc + sigma_j * cr, sigma from the group staged in `slot` (the correction
// scale kappa is folded into U^T q).
template <int D, int R, bool VQ2, bool NB>
__device__ __forceinline__ void group_scores(const uint8_t* slot, const Fixed<D, R>& f, int quad, const floatx4* acc,
                                             const floatx4* cr, float* sv) {
  using KS = KSide<D, R, VQ2, NB>;
  if constexpr (R > 0) {
    const half8_t sg = *reinterpret_cast<const half8_t*>(slot + KS::OFF_SG + 16 * quad);
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sv[4 * T + j] = fmaf((float)sg[4 * T + j], cr[T][j], acc[T][j]);
  } else {
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j) sv[4 * T + j] = acc[T][j];
  }
}

// Online-softmax step (lazy maximum) over this lane's 8 scores s = inv_scale * sv; p = 2^(s - m_run),
// with live = false giving p = 0 and no update (a column whose group does not exist in this step).
// inv_scale is a power of two, so scaling the maximum, or each score inside the exponent's fma,
// rounds exactly as scaling the scores first would.
template <int NCT, int NG, bool VQ2>
__device__ __forceinline__ void softmax_step(const float* sv, float inv_scale, bool live, float* p, floatx4* o_acc,
                                             float* z_acc, float& m_run, float& l_run) {
  float mx = sv[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
  mx = inv_scale * quad_max(mx);
  const bool grow = live && mx > m_run + kLazyMax;  // true on the first group (m_run = -inf)
  if (__any(grow)) {
    // alpha: 0 on a column's first group; exactly 1 for the columns that keep their maximum
    // (also those still at -inf, whose state is all zero)
    const float m_new = grow ? mx : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) o_acc[ct] *= alpha;
    if constexpr (VQ2)
#pragma unroll
      for (int cg = 0; cg < NG; ++cg) z_acc[cg] *= alpha;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = live ? __builtin_amdgcn_exp2f(fmaf(inv_scale, sv[j], -m_run)) : 0.0f;  // below 2^-126 flushes to 0
    l_run += p[j];
  }
}

// 2-bit values, the B side of this lane's column: p o s as bf16 hi/lo pairs per 32-channel group
// (the code part of v_hat = code * s + z is a matrix product with p o s as second operand), and
// the zero part sum_j p_j z_j per channel group accumulated per lane (tokens 8*quad .. +7; the
// quads are summed at the end). s and z come from the group staged in `slot`.
template <int D, int R, bool NB>
__device__ __forceinline__ void value_operands(const uint8_t* slot, const float* p, int quad, bf16x8_t* bh,
                                               bf16x8_t* bl, float* z_acc) {
  constexpr int NG = D / 32;
  using KS = KSide<D, R, true, NB>;
  const _Float16* vm_h = reinterpret_cast<const _Float16*>(slot + KS::OFF_VM);
#pragma unroll
  for (int cg = 0; cg < NG; ++cg) {
    const half8_t s8 = *reinterpret_cast<const half8_t*>(vm_h + cg * kGroup + 8 * quad);
    const half8_t z8 = *reinterpret_cast<const half8_t*>(vm_h + (NG + cg) * kGroup + 8 * quad);
    u32x4 xh, xl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h2, l2;
      // fma with a zero addend maps to one mixed-precision fma (the f16 step read directly)
      split_bf16_pair(__builtin_fmaf(p[2 * i], (float)s8[2 * i], 0.0f),
                      __builtin_fmaf(p[2 * i + 1], (float)s8[2 * i + 1], 0.0f), h2, l2);
      xh[i] = h2;
      xl[i] = l2;
    }
    float za = z_acc[cg];
#pragma unroll
    for (int j = 0; j < 8; ++j) za = fmaf(p[j], (float)z8[j], za);
    z_acc[cg] = za;
    bh[cg] = bitcast<bf16x8_t>(xh);
    bl[cg] = bitcast<bf16x8_t>(xl);
  }
}

// One 32-token group: scores, online-softmax update, P.V accumulation (VP > 0: plus the A^2 value
// policy's corrections, staged at `pslot`).
template <int D, int R, bool VQ2, bool NB, int VP>
__device__ __forceinline__ void process_group(const GroupRaw<D, R, VQ2, NB>& cur, const ProtRaw<D, VP>& pr,
                                              const Fixed<D, R>& f, uint8_t* slot, uint8_t* pslot,
                                              const DecodeArgs& a, int gi, int b, int hq0, int g, int lane, int n,
                                              int quad, floatx4* o_acc, float* z_acc, float& m_run, float& l_run) {
  constexpr int NKT = D / 32, NCT = D / 16, NG = D / 32;
  lds_wave_fence();
  stage_group<D, R, VQ2, NB>(cur, slot, lane);
  if constexpr (VP > 0) *reinterpret_cast<typename Bytes<VP * D / 32>::T*>(pslot + lane * (VP * D / 32)) = pr.vp;
  lds_wave_fence();
  floatx4 acc[2], cr[2];
  group_logits<D, R, VQ2, NB, false>(slot, f, nullptr, nullptr, n, quad, acc, cr);
  float sv[8];  // scores (log2 units) of tokens 8*quad + j for head n
  group_scores<D, R, VQ2, NB>(slot, f, quad, acc, cr, sv);
  if (a.logits_dbg && n < g) {
    float* dst = a.logits_dbg + ((int64_t)b * a.hq + hq0 + n) * a.n_ctx + (int64_t)gi * kGroup + 8 * quad;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = f.inv_scale * sv[j] * kLn2;
  }
  float p[8];
  softmax_step<NCT, NG, VQ2>(sv, f.inv_scale, true, p, o_acc, z_acc, m_run, l_run);
  if constexpr (VQ2) {
    bf16x8_t bh[NG], bl[NG];
    value_operands<D, R, NB>(slot, p, quad, bh, bl, z_acc);
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) {
      // tiles 2cg and 2cg+1 = the low and high halves of the lane's code word cg
      const uint32_t x = word_of<D / 8>(cur.vc, cg);
      const uint32_t ve = even_codes(x), vo = odd_codes(x);
      const bf16x8_t a0 = value_codes8<0>(ve, vo);
      const bf16x8_t a1 = value_codes8<1>(ve, vo);
      o_acc[2 * cg] = mfma_bf16(a0, bh[cg], o_acc[2 * cg]);
      o_acc[2 * cg] = mfma_bf16(a0, bl[cg], o_acc[2 * cg]);
      o_acc[2 * cg + 1] = mfma_bf16(a1, bh[cg], o_acc[2 * cg + 1]);
      o_acc[2 * cg + 1] = mfma_bf16(a1, bl[cg], o_acc[2 * cg + 1]);
    }
    if constexpr (VP > 0) add_corrections<D, VP>(pslot, pr.idx, p, n, quad, o_acc);
  } else {
    bf16x8_t p_hi8, p_lo8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 ph = (__bf16)p[j];
      p_hi8[j] = ph;
      p_lo8[j] = (__bf16)(p[j] - (float)ph);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const bf16x8_t av = bitcast<bf16x8_t>(cur.v[ct]);
      o_acc[ct] = mfma_bf16(av, p_hi8, o_acc[ct]);
      o_acc[ct] = mfma_bf16(av, p_lo8, o_acc[ct]);
    }
  }
}

// J groups of one step (2-bit values, g <= 16 / J) share the 16 matrix columns: column n = lane
// % 16 belongs to block jl = n / g, head hd = n % g, and follows group jl of the step. Each
// group's products run over all 16 columns and every lane keeps the result of its own group, so
// the per-column work (q o s, the softmax step, p o s and its split) is done once per step
// instead of once per group; the matrix products per group are unchanged. The columns of a head
// are separate online-softmax partials, merged with the waves' partials at the end. `nv` groups
// of the step exist (the last step of a wave may hold fewer); the others' columns stay idle: the
// products of all J groups run unconditionally (straight-line code the scheduler can interleave),
// a missing group's results are only ever selected by idle columns, whose scores are replaced and
// whose probabilities are 0, and its value operand meets zero columns only.
template <int D, int R, bool NB, int J, int VP>
__device__ __forceinline__ void process_block(const typename Bytes<D / 8>::T* vcs, const uint32_t* pidx,
                                              const int* gis, int nv, const Fixed<D, R>& f, const uint8_t* slots,
                                              const uint8_t* pslots, const DecodeArgs& a, int b, int hq0, int g,
                                              int jl, int hd, int n, int quad, floatx4* o_acc, float* z_acc,
                                              float& m_run, float& l_run) {
  constexpr int NKT = D / 32, NCT = D / 16, NG = D / 32;
  using KS = KSide<D, R, true, NB>;
  const bool live = jl < nv;
  // the lane's own group (idle columns read the last existing one: finite bytes, weight 0)
  const uint8_t* own = slots + (live ? jl : nv - 1) * KS::BYTES;
  half8_t p_hi[NKT], p_lo[NKT];
  query_times_step<D, R, true, NB>(own, f, quad, p_hi, p_lo);
  floatx4 A[2], C[2];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    floatx4 acc[2], cr[2];
    group_logits<D, R, true, NB, true>(slots + j * KS::BYTES, f, p_hi, p_lo, n, quad, acc, cr);
#pragma unroll
    for (int T = 0; T < 2; ++T) {
      A[T] = (j == 0 || jl == j) ? acc[T] : A[T];
      if constexpr (R > 0) C[T] = (j == 0 || jl == j) ? cr[T] : C[T];
    }
  }
  float sv[8];
  group_scores<D, R, true, NB>(own, f, quad, A, C, sv);
  if (a.logits_dbg && live && hd < g) {
    int gi = gis[0];
#pragma unroll
    for (int j = 1; j < J; ++j) gi = jl == j ? gis[j] : gi;
    float* dst = a.logits_dbg + ((int64_t)b * a.hq + hq0 + hd) * a.n_ctx + (int64_t)gi * kGroup + 8 * quad;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = f.inv_scale * sv[j] * kLn2;
  }
  float p[8];
  softmax_step<NCT, NG, true>(sv, f.inv_scale, live, p, o_acc, z_acc, m_run, l_run);
  bf16x8_t bh[NG], bl[NG];
  value_operands<D, R, NB>(own, p, quad, bh, bl, z_acc);
  const bf16x8_t zero8 = bitcast<bf16x8_t>((u32x4){0u, 0u, 0u, 0u});
#pragma unroll
  for (int j = 0; j < J; ++j) {
#pragma unroll
    for (int cg = 0; cg < NG; ++cg) {
      // group j's value codes against the columns of block j only
      const bf16x8_t bhj = jl == j ? bh[cg] : zero8, blj = jl == j ? bl[cg] : zero8;
      const uint32_t x = word_of<D / 8>(vcs[j], cg);
      const uint32_t ve = even_codes(x), vo = odd_codes(x);
      const bf16x8_t a0 = value_codes8<0>(ve, vo);
      const bf16x8_t a1 = value_codes8<1>(ve, vo);
      o_acc[2 * cg] = mfma_bf16(a0, bhj, o_acc[2 * cg]);
      o_acc[2 * cg] = mfma_bf16(a0, blj, o_acc[2 * cg]);
      o_acc[2 * cg + 1] = mfma_bf16(a1, bhj, o_acc[2 * cg + 1]);
      o_acc[2 * cg + 1] = mfma_bf16(a1, blj, o_acc[2 * cg + 1]);
    }
  }
  if constexpr (VP > 0) {
    // the corrections of the lane's own group (idle columns: p = 0 against finite rows)
    const int jo = live ? jl : nv - 1;
    uint32_t idx = pidx[0];
#pragma unroll
    for (int j = 1; j < J; ++j) idx = jo == j ? pidx[j] : idx;
    add_corrections<D, VP>(pslots + jo * (VP * D * 2), idx, p, n, quad, o_acc);
  }
}

// The unfinished last group: n_ctx % 32 tokens whose keys and values are held exactly in the
// tails (no base or side code). On the vector units, once per stream: lane (column n, quad)
// scores tokens 8*quad .. +7 for its head hd with the scaled query, takes the same online-softmax
// step as a group, and adds p . v to its own output channels 16*ct + 4*quad + j, fetching the
// other quads' probabilities by lane shuffles. Columns with act = false (the other blocks of a
// packed layout, whose heads the first block already covers) take no part.
template <int D>
__device__ __forceinline__ void process_tail(const DecodeArgs& a, int64_t n_ctx, int64_t bh, int b, int hq0, int g,
                                             int n, int hd, bool act, int quad, const float (*qs)[D],
                                             float inv_scale, floatx4* o_acc, float* z_acc, int n_z, float& m_run,
                                             float& l_run) {
  constexpr int NCT = D / 16;
  const int64_t n_full = n_ctx / kGroup * kGroup;
  const int tail_len = (int)(n_ctx - n_full);
  const int own_len = act ? tail_len : 0;  // rows this lane scores
  // scores of rows 8*quad + j: channels in steps of 8 (one 16-byte or two 16-byte loads per row)
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll 1
  for (int c = 0; c < D; c += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = 8 * quad + j;
      if (t >= own_len) continue;
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
      for (int i = 0; i < 8; ++i) acc[j] = fmaf(qs[hd][c + i], k[i], acc[j]);
    }
  }
  float sv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = 8 * quad + j;
    sv[j] = t < own_len ? inv_scale * acc[j] : -INFINITY;
    if (t < own_len && a.logits_dbg && hd < g)
      a.logits_dbg[((int64_t)b * a.hq + hq0 + hd) * a.n_ctx + n_full + t] = sv[j] * kLn2;
  }
  // online softmax step (as for a group)
  float mx = sv[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sv[j]);
  mx = quad_max(mx);
  const bool grow = mx > m_run + kLazyMax;
  if (__any(grow)) {
    const float m_new = grow ? mx : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // as in softmax_step
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) o_acc[ct] *= alpha;
    for (int cg = 0; cg < n_z; ++cg) z_acc[cg] *= alpha;
  }
  float p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = 8 * quad + j < own_len ? __builtin_amdgcn_exp2f(sv[j] - m_run) : 0.0f;
    l_run += p[j];
  }
#pragma unroll 1
  for (int t = 0; t < tail_len; ++t) {
    // row t's probability for head n lives in lane n + 16 * (t / 8), slot t % 8
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

// J > 1: J groups per step share the matrix columns (2-bit values, g <= 16 / J; see process_block).
// VP > 0: the A^2 value policy's VP corrected tokens per group (2-bit values and 2-bit keys).
template <int D, int R, bool VQ2, bool NB, int J, int VP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(J == 1 || VQ2, "packed columns are built for 2-bit values");
  static_assert(VP == 0 || (VQ2 && !NB), "the value policy is built for 2-bit values and 2-bit keys");
  constexpr int NKT = D / 32, NCT = D / 16, NG = D / 32;
  constexpr int RU = R > 0 ? R : 1;
  constexpr int SLOT = KSide<D, R, VQ2, NB>::BYTES;
  constexpr int PSLOT = VP * D * 2;            // corrections of one group
  __shared__ float qs[kMaxGqa][D];            // scaled queries
  __shared__ float qu_s[kMaxGqa][RU];         // U^T q (scaled)
  __shared__ float inv_scale_s[kMaxGqa];      // 2^e undoing the per-head query scale
  __shared__ u32x4 kslot[kWaves][J * SLOT / 16];  // per-wave staging of the groups of a step
  __shared__ u32x4 pslot_s[kWaves][VP > 0 ? J * PSLOT / 16 : 1];  // their corrections
  __shared__ float m_w[kWaves][kMaxGqa], l_w[kWaves][kMaxGqa];
  __shared__ float o_w[kWaves][kMaxGqa][D];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform per wave: keeps group offsets scalar
  const int n = lane % 16, quad = lane / 16;
  const int g = a.gqa;
  // column n of the matrix products: block jl (the step's group it follows) and head hd; columns
  // past J * g are padding (their results are never merged)
  const int jl = J > 1 ? n / g : 0, hd = J > 1 ? n % g : n;
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
  const int groups_cap = (int)(a.cap / kGroup);
  constexpr int KROW = KSide<D, R, VQ2, NB>::KC / kGroup;  // key-code bytes per token
  s.kcode = make_rsrc(a.kcode + bh * a.cap * KROW, a.cap * KROW);
  s.kmeta = make_rsrc(a.kmeta + bh * groups_cap * 2 * D, (int64_t)groups_cap * 4 * D);
  s.scode = make_rsrc(R > 0 ? a.scode + bh * a.cap * (R / 2) : a.kcode, R > 0 ? a.cap * (R / 2) : 0);
  s.ssc = make_rsrc(R > 0 ? a.ssc + bh * a.cap : a.kmeta, R > 0 ? a.cap * 2 : 0);
  if constexpr (VQ2) {
    s.v = make_rsrc(a.vcode + bh * a.cap * (D / 4), a.cap * (D / 4));
    s.vmeta = make_rsrc(a.vmeta + bh * groups_cap * 2 * D, (int64_t)groups_cap * 4 * D);
  } else {
    s.v = make_rsrc((const uint16_t*)a.vdense + bh * a.cap * D, a.cap * D * 2);
    s.vmeta = s.v;
  }
  if constexpr (VP > 0) {
    s.vprot = make_rsrc(a.vprot + bh * groups_cap * VP * D, (int64_t)groups_cap * PSLOT);
    s.vpidx = make_rsrc(a.vpidx + bh * groups_cap, (int64_t)groups_cap * 4);
  }
  // group indices are 32-bit and wave-uniform, so every offset below stays in scalar registers
  // this row's attended tokens: whole groups, then the unfinished one from the tails
  int64_t n_ctx = a.n_ctx;
  if (a.row_len) {
    const int64_t r = a.row_len[b];
    n_ctx = r < 0 ? 0 : (r > a.n_ctx ? a.n_ctx : r);
  }
  const int n_groups = (int)(n_ctx / kGroup);
  const int W = a.n_splits * kWaves;
  const int rot = n_groups > 0 ? (int)((bh * 40503) % n_groups) : 0;
  auto group_at = [&](int j) { const int x = j + rot; return x >= n_groups ? x - n_groups : x; };
  const int j_begin = split * kWaves + wave;
  // (contiguous caches: an empty resource over valid memory, so any load from it reads 0)
  const __amdgpu_buffer_rsrc_t table_row =
      make_rsrc(a.map.block_table ? (const void*)(a.map.block_table + (int64_t)b * a.map.max_pages)
                                  : (const void*)a.kcode,
                a.map.block_table ? a.map.max_pages * 4 : 0);
  auto page_at = [&](int j) { return j < n_groups ? request_page(a, table_row, group_at(j)) : 0; };
  // J > 1: the page of a step's group requested unconditionally (index clamped into the row;
  // n_groups >= 1 wherever it is called), so that the load into the page register never has to
  // wait for the previous one (a register write of 0 on the other path would)
  auto page_req = [&](int j) {
    const int x = group_at(j);
    const int off = __builtin_amdgcn_readfirstlane((x < n_groups ? x : n_groups - 1) * 4);
    return (int)__builtin_amdgcn_raw_buffer_load_b32(table_row, 0, off, 0);
  };
  int pa = 0, pb = 0;          // pages of the next groups loaded into ga / gb (paged caches)
  GroupRaw<D, R, VQ2, NB> ga, gb;  // ping-pong register sets: one group computed while the next loads
  GroupRaw<D, R, VQ2, NB> gj[J];   // J > 1: the next step's groups, loaded while a step computes
  int pj[J];                       // J > 1: their pages (paged caches), requested one step ahead
  ProtRaw<D, VP> qa, qb, qj[J];    // VP > 0: the policy's corrections of ga, gb, gj
  // one group's loads (and its corrections) into register set g / q
  auto load = [&](GroupRaw<D, R, VQ2, NB>& gr, ProtRaw<D, VP>& qr, int page, int gi) {
    load_group<D, R, VQ2, NB>(gr, s, a, h, page, lane, n, quad, gi);
    if constexpr (VP > 0) load_prot<D, R, NB, VP>(qr, s, a, h, page, lane, gi);
  };
  auto first_loads = [&]() {
    if constexpr (J == 1) {
      if (j_begin < n_groups) load(ga, qa, page_at(j_begin), group_at(j_begin));
      if (j_begin + W < n_groups) load(gb, qb, page_at(j_begin + W), group_at(j_begin + W));
      pa = page_at(j_begin + 2 * W);
      pb = page_at(j_begin + 3 * W);
    } else {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int sl = j_begin + W * j;
        if (sl < n_groups) load(gj[j], qj[j], page_at(sl), group_at(sl));
      }
#pragma unroll
      for (int j = 0; j < J; ++j) pj[j] = page_at(j_begin + W * (J + j));
    }
  };
  // the wave that takes the unfinished group requests its first groups after it (fewer live registers)
  const bool tail_wave = n_ctx % kGroup && split == 0 && wave == 0;
  if (!tail_wave) first_loads();
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
      qu_s[hh][r] = a.corr_scale * acc;  // the correction's scale rides on U^T q
    }
  }
  __syncthreads();

  // ---- per-lane fixed operands
  Fixed<D, R> f;
#pragma unroll
  for (int t = 0; t < NKT; ++t)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = qs[hd][(D / 4) * quad + 8 * t + j];
      f.bq_hi[t][j] = f16_hi(x);
      f.bq_lo[t][j] = f16_lo(x);
    }
  f.inv_scale = inv_scale_s[hd];
  if constexpr (R == 32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f.bu_hi8[j] = f16_hi(qu_s[hd][8 * quad + j]);
      f.bu_lo8[j] = f16_lo(qu_s[hd][8 * quad + j]);
    }
  } else if constexpr (R > 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * quad + j;
      const float x = r < R ? qu_s[hd][r] : 0.0f;
      f.bu_hi4[j] = f16_hi(x);
      f.bu_lo4[j] = f16_lo(x);
    }
  }

  floatx4 o_acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o_acc[ct] = (floatx4){0.f, 0.f, 0.f, 0.f};
  float z_acc[NG];  // 2-bit values: sum_j p_j z_j per channel group (this lane's tokens)
#pragma unroll
  for (int cg = 0; cg < NG; ++cg) z_acc[cg] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // ---- the unfinished last group (exact, from the tails), by one wave per stream
  if (tail_wave) {
    process_tail<D>(a, n_ctx, bh, b, hq0, g, n, hd, J == 1 || jl == 0, quad, qs, f.inv_scale, o_acc, z_acc,
                    VQ2 ? NG : 0, m_run, l_run);
    first_loads();
  }

  // ---- this wave's groups
  uint8_t* slot = reinterpret_cast<uint8_t*>(kslot[wave]);
  uint8_t* pslot = reinterpret_cast<uint8_t*>(pslot_s[wave]);
  if constexpr (J > 1) {
    // steps of J groups (the wave's group slots j_begin + W*k, k = k0 .. k0+J-1): stage the
    // step's groups, request the next step's, compute this one from LDS
    for (int k0 = 0; j_begin + W * k0 < n_groups; k0 += J) {
      int nv = 0, gis[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int sl = j_begin + W * (k0 + j);
        nv = sl < n_groups ? j + 1 : nv;
        gis[j] = group_at(sl < n_groups ? sl : j_begin + W * k0);
      }
      lds_wave_fence();
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (j < nv) {
          stage_group<D, R, VQ2, NB>(gj[j], slot + j * SLOT, lane);
          if constexpr (VP > 0)
            *reinterpret_cast<typename Bytes<VP * D / 32>::T*>(pslot + j * PSLOT + lane * (VP * D / 32)) = qj[j].vp;
        }
      lds_wave_fence();
      typename Bytes<D / 8>::T vcs[J];
      uint32_t pidx[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        vcs[j] = gj[j].vc;
        pidx[j] = qj[j].idx;
      }
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int sl = j_begin + W * (k0 + J + j);
        if (sl < n_groups) load(gj[j], qj[j], pj[j], group_at(sl));
      }
#pragma unroll
      for (int j = 0; j < J; ++j) pj[j] = page_req(j_begin + W * (k0 + 2 * J + j));
      process_block<D, R, NB, J, VP>(vcs, pidx, gis, nv, f, slot, pslot, a, b, hq0, g, jl, hd, n, quad, o_acc, z_acc,
                                     m_run, l_run);
    }
  } else
  for (int j = j_begin; j < n_groups; j += 2 * W) {
    process_group<D, R, VQ2, NB, VP>(ga, qa, f, slot, pslot, a, group_at(j), b, hq0, g, lane, n, quad, o_acc, z_acc,
                                     m_run, l_run);
    if (j + W >= n_groups) break;
    if (j + 2 * W < n_groups) {
      load(ga, qa, pa, group_at(j + 2 * W));
      pa = page_at(j + 4 * W);
    }
    process_group<D, R, VQ2, NB, VP>(gb, qb, f, slot, pslot, a, group_at(j + W), b, hq0, g, lane, n, quad, o_acc, z_acc,
                                     m_run,
                             l_run);
    if (j + 3 * W < n_groups) {
      load(gb, qb, pb, group_at(j + 3 * W));
      pb = page_at(j + 5 * W);
    }
  }
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

  // ---- merge the 4 waves of this workgroup, write the split partial
  l_run = quad_sum(l_run);
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
    // partials: every wave, and every block of columns of a packed layout (column jb*g + hh)
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
      for (int jb = 0; jb < J; ++jb) M = fmaxf(M, m_w[w][jb * g + hh]);
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
#pragma unroll
        for (int jb = 0; jb < J; ++jb) {
          const int col = jb * g + hh;
          if (m_w[w][col] == -INFINITY) continue;
          const float fct = exp2f(m_w[w][col] - M);
          L = fmaf(l_w[w][col], fct, L);
          O = fmaf(o_w[w][col][c], fct, O);
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
    m_w[0][tid] = L > 0.0f ? 1.0f / L : 0.0f;  // a row without tokens reads out zeros
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

template <int D, bool VQ2, bool NB, int J, int VP>
hipError_t launch_rjp(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.n_splits, (unsigned)a.hkv, (unsigned)a.batch);
  switch (a.r) {
    case 0: hipLaunchKernelGGL((decode_mfma_kernel<D, 0, VQ2, NB, J, VP>), grid, dim3(kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_mfma_kernel<D, 4, VQ2, NB, J, VP>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_mfma_kernel<D, 8, VQ2, NB, J, VP>), grid, dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((decode_mfma_kernel<D, 16, VQ2, NB, J, VP>), grid, dim3(kThreads), 0, s, a); break;
    case 32: hipLaunchKernelGGL((decode_mfma_kernel<D, 32, VQ2, NB, J, VP>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool VQ2, bool NB, int J>
hipError_t launch_rj(const DecodeArgs& a, hipStream_t s) {
  if constexpr (VQ2 && !NB && J <= 2) {
    if (a.value_protect == 1) return launch_rjp<D, true, false, J, 1>(a, s);
    if (a.value_protect == 2) return launch_rjp<D, true, false, J, 2>(a, s);
  }
  if (a.value_protect) return hipErrorInvalidValue;
  return launch_rjp<D, VQ2, NB, J, 0>(a, s);
}

// 2-bit values with few heads per KV head: J = 16 / g groups share the matrix columns, at most 3
// for d = 128 with 2-bit keys and no value policy, at most 2 otherwise (three groups in flight
// would spill registers there).
template <int D, bool VQ2, bool NB>
hipError_t launch_r(const DecodeArgs& a, hipStream_t s) {
  if constexpr (VQ2) {
    const int j = a.pack_columns ? (a.gqa <= 5 ? 3 : a.gqa <= 8 ? 2 : 1) : 1;
    if constexpr (D == 128 && !NB)
      if (j == 3 && a.value_protect == 0) return launch_rj<D, true, NB, 3>(a, s);
    if (j >= 2) return launch_rj<D, true, NB, 2>(a, s);
  }
  return launch_rj<D, VQ2, NB, 1>(a, s);
}

}  // namespace

hipError_t launch_decode_mfma_split(const DecodeArgs& a, hipStream_t s) {
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
