// append.hip — headq_cache_append on gfx950: the HeadQ cache write.
//
// HeadQ technical summary ("Technische Samenvatting"), §3 step 2 (Cache Schrijven): base-quantize
// each key (k_base = B_b(k)), form the residual e = k - k_base, project it on the calibration
// basis and side-quantize the projection, z = Q_q(U_h^T e); the cache keeps the base code and z.
//
// One launch writes keys and values. A workgroup (256 threads, 4 wave64) owns GPW 32-token
// groups of one (b, h) stream: two for long writes (the second one duplicated, with its stores
// masked, when the token range holds an odd number of groups), one for small launches such as
// the one-group append of a decode step, where the workgroup's latency is the whole cost:
//   1. the 32 x d key tiles are loaded with 128-bit loads into LDS as f32
//   2. per (group, channel): min/max over the 32 tokens -> binary16 step s and zero z (kmeta)
//   3. per (token, 16 channels): 2-bit codes (one 32-bit store) and residuals (back into LDS)
//   4. projection y = U^T e: a slot (a wave for two groups, a half-wave for one) owns a run of
//      components and its lane owns one token row, so U_h is uniform over the slot (scalar loads
//      for long writes, LDS broadcast for small ones) while the residual streams from LDS; every
//      component is one sequential f32 fma chain over channels 0..d-1 (the canonical order that
//      makes the side codes reproducible). The per-token maximum |y| is combined across the
//      slots in LDS; each slot then side-quantizes and packs its components.
//   5. values (when given): dense values are transposed into the channel-major group layout
//      (8 tokens of a channel per 16-byte store), 2-bit values quantized per (token, 32-channel
//      group) into the matrix-operand layout.
//   6. A^2 value policy (2-bit values, value_protect = P > 0; reading of the summary's §2.2 A^2
//      surrogate and §5 A^2-weighted value policy): per group, the P tokens of largest w_j * e_j
//      keep a bfloat16 correction v_j - v_hat_j. e_j = |v_j - v_hat_j|^2 (one f32 fma chain over
//      the channels), w_j = 2^n_j with n_j = clamp(rint(c2 * a_h.k_j), -64, 64) taken from the
//      keys in step 2 (a_h the mean calibration query, a_h.k_j one f32 fma chain); the products are
//      compared exactly in f64, ties to the lower token, slots in ascending token order.
//
// Numerics: no contraction anywhere in this file (every fma is explicit), IEEE division,
// rint = round half to even, binary16 conversion with round to nearest even.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>

#include "headq_internal.h"

namespace headq {
namespace {

constexpr int kThreads = 256;

typedef const __attribute__((address_space(4))) float* const_f32_ptr;  // read through scalar loads

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Min/max grid of one channel (or channel group): compare-select in index order, so that
// equal values of opposite zero sign resolve the same way as a plain sequential scan.
__device__ __forceinline__ void minmax_step_zero(float lo, float hi, float levels, float& s, float& z,
                                                 float& inv, uint16_t& s_bits, uint16_t& z_bits) {
  s_bits = f32_to_f16_bits((hi - lo) / levels);
  z_bits = f32_to_f16_bits(lo);
  s = f16_bits_to_f32(s_bits);
  z = f16_bits_to_f32(z_bits);
  inv = (s == 0.0f) ? 0.0f : 1.0f / s;
}

__device__ __forceinline__ uint32_t base_code(float k, float z, float inv, float levels) {
  float c = __builtin_rintf((k - z) * inv);
  c = c < 0.0f ? 0.0f : c;
  c = c > levels ? levels : c;
  return (uint32_t)c;
}

// The workgroup's GPW groups: row = 32 * gl + t. The appended range [start, end) touches groups
// floor(start/32) .. ceil(end/32)-1; group gl of this workgroup is touched group GPW*blockIdx.x + gl,
// clamped to the last one (a duplicate whose stores are masked) when the count is odd. A group is
// encoded only if it is whole once the range is in (32 * (g + 1) <= end); the rows of a group
// before `start` come from the dense tail, rows at or past `end` do not exist yet. (Plain scalars
// with selects: a small array indexed by a lane value would live in scratch memory.)
struct Tile {
  int64_t bh;
  int64_t g0, g1;  // cache groups of rows 0..31 and 32..63
  bool w0, w1;     // the group is whole and real: it is encoded and stored
  __device__ int64_t group(int gl) const { return gl ? g1 : g0; }
  __device__ bool whole(int gl) const { return gl ? w1 : w0; }
};

template <int GPW>
__device__ __forceinline__ Tile tile_of(const AppendArgs& a, int64_t start) {
  Tile tl;
  tl.bh = (int64_t)blockIdx.z * a.hkv + blockIdx.y;
  const int64_t end = start + a.n_new;
  const int64_t g_first = start / kGroup, n_touch = (end + kGroup - 1) / kGroup - g_first;
  tl.g0 = g_first + (int64_t)blockIdx.x * GPW;
  const bool real1 = GPW > 1 && (int64_t)blockIdx.x * GPW + 1 < n_touch;
  tl.g1 = real1 ? tl.g0 + 1 : tl.g0;
  tl.w0 = (tl.g0 + 1) * kGroup <= end;
  tl.w1 = real1 && (tl.g1 + 1) * kGroup <= end;
  return tl;
}

// Cache token of LDS row `row`.
__device__ __forceinline__ int64_t row_token(const Tile& tl, int row) {
  return tl.group(row / kGroup) * kGroup + row % kGroup;
}

// Address of 16 bytes at element `c` of cache token `tok`'s row for a given input: the dense
// tail (tokens before `start`), the caller's rows (tokens in [start, end)), or nullptr (tokens
// past `end`, which do not exist yet). `es` is the element size, `base` the caller's (b, h) row 0.
__device__ __forceinline__ const void* row_src(const AppendArgs& a, int64_t start, const void* base, int64_t ts,
                                               const void* tail, int64_t bh, int D, int es, int64_t tok, int c) {
  if (tok < start) return (const char*)tail + ((bh * kGroup + tok % kGroup) * D + c) * es;
  if (tok < start + a.n_new) return (const char*)base + ((tok - start) * ts + c) * es;
  return nullptr;
}

// Load the 32 * GPW rows of f32/bf16 input (element stride 1 along channels, token stride ts)
// into an f32 LDS tile with row pitch P, with 128-bit loads; rows that do not exist yet read as zero.
template <int D, int P, bool BF16, int GPW>
__device__ __forceinline__ void load_rows(float (*dst)[P], const AppendArgs& a, int64_t start, const void* base,
                                          int64_t ts, const void* tail, const Tile& tl) {
  constexpr int kRows = GPW * kGroup;
  constexpr int kElem = BF16 ? 8 : 4;  // elements per 16-byte load
  constexpr int kChunks = D / kElem;   // 16-byte chunks per row
  for (int i = threadIdx.x; i < kRows * kChunks; i += kThreads) {
    const int row = i / kChunks, ch = i % kChunks;
    const void* src = row_src(a, start, base, ts, tail, tl.bh, D, BF16 ? 2 : 4, row_token(tl, row), ch * kElem);
    const uint4 w = src ? *reinterpret_cast<const uint4*>(src) : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    if constexpr (BF16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[row][ch * 8 + 2 * j] = __uint_as_float(u[j] << 16);
        dst[row][ch * 8 + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[row][ch * 4 + j] = __uint_as_float(u[j]);
    }
  }
}

// Copy the caller's rows of the unfinished last group into the dense tails (rows t % 32).
// Done by workgroup 0 only, after every read of the tails in this launch: the only group that
// reads tail rows is the first touched one, which workgroup 0 owns.
__device__ __forceinline__ void write_tails(const AppendArgs& a, int64_t start, int64_t bh, int D, const void* kbase,
                                            int kes, const void* vbase, int ves) {
  const int64_t end = start + a.n_new;
  if (end % kGroup == 0) return;
  const int64_t t_lo = start > end / kGroup * kGroup ? start : end / kGroup * kGroup;
  const int n_rows = (int)(end - t_lo);
  for (int pass = 0; pass < 2; ++pass) {
    const int es = pass ? ves : kes;
    const char* src = (const char*)(pass ? vbase : kbase);
    char* tail = (char*)(pass ? a.vtail : a.ktail);
    const int64_t ts = pass ? a.vs_t : a.ks_t;
    if (!src) continue;
    const int chunks = D * es / 16;
    for (int i = threadIdx.x; i < n_rows * chunks; i += kThreads) {
      const int64_t tok = t_lo + i / chunks;
      const int ch = i % chunks;
      *reinterpret_cast<uint4*>(tail + (bh * kGroup + tok % kGroup) * D * es + ch * 16) =
          *reinterpret_cast<const uint4*>(src + (tok - start) * ts * es + ch * 16);
    }
  }
}

// UL: U_h staged in LDS and read with wave-uniform (broadcast) addresses, the shorter critical
// path for small launches (one group per stream, as in a decode step); otherwise U_h comes
// through scalar loads, which leaves more LDS for concurrent workgroups of a long prefill.
template <int D, int R, bool KBF16, bool UL, int GPW>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
  static_assert(GPW == 2 || (GPW == 1 && UL), "a half-wave projection slot reads U_h from LDS");
  constexpr int kRows = GPW * kGroup;      // token rows per workgroup (one per lane of a slot)
  constexpr int P = D + 1;  // LDS row pitch (floats): a column read by 64 rows spreads over the banks
  constexpr int SLOTS = GPW == 2 ? 4 : 8;  // projection slots: waves (64 rows) or half-waves (32 rows)
  // components per slot: r/SLOTS, at least 2 so that every slot packs whole bytes
  constexpr int CW = R / SLOTS >= 2 ? R / SLOTS : 2;
  constexpr int NWP = R > 0 ? R / CW : 0;  // slots that project
  constexpr int NG = D / 32;               // 32-channel groups (2-bit values)
  __shared__ float ke[kRows][P];           // keys, then residuals; values in step 5
  __shared__ float s_s[GPW * D], z_s[GPW * D], inv_s[GPW * D];
  __shared__ float amax_s[SLOTS][kRows];
  __shared__ float U_s[UL && R > 0 ? D * R : 1];
  __shared__ int pn_s[kRows];              // A^2 value policy: weight exponent per token row
  __shared__ double pr_s[kRows];           //   w_j * e_j
  __shared__ int sel_s[kRows];             //   chosen
  __shared__ int tok_s[GPW][2];            //   token of each slot

  const int h = blockIdx.y, b = blockIdx.z;
  const float klev = (float)a.key_levels;  // base-code levels of the keys (values are 2-bit: 3)
  // this row's append position; a row that would pass the capacity is left untouched
  const int64_t st = a.row_start ? (int64_t)a.row_start[b] : a.start;
  if (st < 0 || st + a.n_new > a.cap) return;
  const Tile tl = tile_of<GPW>(a, st);
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const char* kin = (const char*)a.k + ((int64_t)b * a.ks_b + (int64_t)h * a.ks_h) * (KBF16 ? 2 : 4);
  const int ves = a.value_bf16 ? 2 : 4;
  const char* vin = a.v ? (const char*)a.v + ((int64_t)b * a.vs_b + (int64_t)h * a.vs_h) * ves : nullptr;
  if (!tl.w0) {  // no whole group here (the second one cannot be whole either): tail rows only
    if (blockIdx.x == 0) write_tails(a, st, tl.bh, D, kin, KBF16 ? 2 : 4, vin, ves);
    return;
  }

  // value rows requested first, into registers: their latency overlaps the whole key pipeline
  constexpr int VMAX = D / 16;                  // 16-byte chunks per thread for f32 values
  const bool vbf = a.value_bf16;
  const int vper = vbf ? 8 : 4;                 // elements per chunk
  const int vchunks = D / vper;                 // chunks per row
  const int vpt = kRows * vchunks / kThreads;   // chunks per thread
  uint4 vr[VMAX];
  if (a.v) {
#pragma unroll
    for (int k = 0; k < VMAX; ++k) {
      if (k < vpt) {
        const int i = tid + k * kThreads, row = i / vchunks, c0 = (i % vchunks) * vper;
        const void* src = row_src(a, st, vin, a.vs_t, a.vtail, tl.bh, D, ves, row_token(tl, row), c0);
        vr[k] = src ? *reinterpret_cast<const uint4*>(src) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }

  load_rows<D, P, KBF16, GPW>(ke, a, st, kin, a.ks_t, a.ktail, tl);
  if constexpr (UL && R > 0) {
    const float4* Ug = reinterpret_cast<const float4*>(a.U + (int64_t)h * D * R);
    for (int i = tid; i < D * R / 4; i += kThreads) reinterpret_cast<float4*>(U_s)[i] = Ug[i];
  }
  __syncthreads();

  // 2. per (group, channel) step and zero (binary16) over the 32 tokens
  for (int i = tid; i < GPW * D; i += kThreads) {
    const int gl = i / D, c = i % D;
    float lo = ke[gl * kGroup][c], hi = lo;
#pragma unroll
    for (int t = 1; t < kGroup; ++t) {
      const float x = ke[gl * kGroup + t][c];
      lo = x < lo ? x : lo;
      hi = x > hi ? x : hi;
    }
    float s, z, inv;
    uint16_t sb, zb;
    minmax_step_zero(lo, hi, klev, s, z, inv, sb, zb);
    if (tl.whole(gl)) {
      uint16_t* meta = a.kmeta + a.map.block(b, h, tl.group(gl)) * 2 * D;
      meta[c] = sb;
      meta[D + c] = zb;
    }
    s_s[i] = s;
    z_s[i] = z;
    inv_s[i] = inv;
  }
  // the A^2 value policy's weight exponent of each row, from the keys (step 3 replaces them by
  // residuals); the last kRows threads, the ones step 2 leaves idle for one-group launches
  const bool prot = a.value_protect > 0 && a.v != nullptr;
  if (prot && tid >= kThreads - kRows) {
    const int row = tid - (kThreads - kRows);
    const const_f32_ptr ad = (const_f32_ptr)(a.vdir + (int64_t)h * D);
    float dot = 0.0f;
    for (int c = 0; c < D; ++c) dot = __builtin_fmaf(ad[c], ke[row][c], dot);
    float nf = __builtin_rintf(dot * a.prot_c2);
    nf = nf < -64.0f ? -64.0f : nf;
    nf = nf > 64.0f ? 64.0f : nf;
    pn_s[row] = (int)nf;
  }
  __syncthreads();

  // 3. codes (16 channels -> one 32-bit word at 2 bits, two nibble words at 3 or 4 bits) and
  // residuals e = k - fma(code, s, z)
  const bool nib = a.key_levels != 3;
  for (int i = tid; i < kRows * (D / 16); i += kThreads) {
    const int row = i / (D / 16), c0 = (i % (D / 16)) * 16, gl = row / kGroup;
    uint32_t word = 0, w4[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = c0 + j, m = gl * D + c;
      const float k = ke[row][c];
      const uint32_t code = base_code(k, z_s[m], inv_s[m], klev);
      word |= code << kcode_bit(j);
      w4[j / 8] |= code << kcode4_bit(j % 8);
      ke[row][c] = k - __builtin_fmaf((float)code, s_s[m], z_s[m]);
    }
    if (tl.whole(gl)) {
      const int64_t tok = row_token(tl, row);
      if (nib)
        *reinterpret_cast<uint2*>(a.kcode + a.map.row(b, h, tok) * (D / 2) + c0 / 2) = make_uint2(w4[0], w4[1]);
      else
        *reinterpret_cast<uint32_t*>(a.kcode + a.map.row(b, h, tok) * (D / 4) + c0 / 4) = word;
    }
  }

  if constexpr (R > 0) {
    __syncthreads();
    // 4. side code. Slot w < NWP projects components [w*CW, (w+1)*CW) of its lane's token row.
    const int row = lane % kRows, gl = row / kGroup;
    const int slot = GPW == 2 ? wave : 2 * wave + lane / kGroup;
    float y[CW];
#pragma unroll
    for (int j = 0; j < CW; ++j) y[j] = 0.0f;
    if (slot < NWP) {
      if constexpr (UL) {
        const float* Uw = U_s + slot * CW;
#pragma unroll 8
        for (int c = 0; c < D; ++c) {
          const float e = ke[row][c];
#pragma unroll
          for (int j = 0; j < CW; ++j) y[j] = __builtin_fmaf(Uw[c * R + j], e, y[j]);
        }
      } else {
        const const_f32_ptr Uw = (const_f32_ptr)(a.U + (int64_t)h * D * R) + wave * CW;
#pragma unroll 8
        for (int c = 0; c < D; ++c) {
          const float e = ke[row][c];
#pragma unroll
          for (int j = 0; j < CW; ++j) y[j] = __builtin_fmaf(Uw[c * R + j], e, y[j]);
        }
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const float m = __builtin_fabsf(y[j]);
      amax = m > amax ? m : amax;
    }
    amax_s[slot][row] = amax;
    __syncthreads();
    if (slot < NWP) {
#pragma unroll
      for (int w = 0; w < NWP; ++w) {
        const float m = amax_s[w][row];
        amax = m > amax ? m : amax;
      }
      const uint16_t sg_bits = f32_to_f16_bits(amax / 7.0f);
      const float sg = f16_bits_to_f32(sg_bits);
      const float inv = (sg == 0.0f) ? 0.0f : 1.0f / sg;
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < CW; ++j) {
        float zc = __builtin_rintf(y[j] * inv);
        zc = zc < -7.0f ? -7.0f : zc;
        zc = zc > 7.0f ? 7.0f : zc;
        packed |= (uint32_t)((int)zc + 8) << (4 * j);
      }
      if (tl.whole(gl)) {
        const int64_t tok = row_token(tl, row);
        const int64_t trow = a.map.row(b, h, tok);
        uint8_t* dst = a.scode + trow * (R / 2) + slot * (CW / 2);
        if constexpr (CW == 8)
          *reinterpret_cast<uint32_t*>(dst) = packed;
        else if constexpr (CW == 4)
          *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
        else
          *dst = (uint8_t)packed;
        if (slot == 0) a.ssc[trow] = sg_bits;
      }
    }
  }
  if (a.v) {
  // 5. values of the same rows (LDS reused once every wave is done with the residuals)
  __syncthreads();
  if (a.value_mode == HEADQ_V_DENSE) {
    // raw elements into LDS, then each group written channel-major ([d][32])
    uint32_t (*raw)[P] = reinterpret_cast<uint32_t (*)[P]>(ke);
#pragma unroll
    for (int k = 0; k < VMAX; ++k) {
      if (k < vpt) {
        const int i = tid + k * kThreads, row = i / vchunks, c0 = (i % vchunks) * vper;
        const uint32_t u[4] = {vr[k].x, vr[k].y, vr[k].z, vr[k].w};
        if (vbf) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            raw[row][c0 + 2 * j] = u[j] & 0xffffu;
            raw[row][c0 + 2 * j + 1] = u[j] >> 16;
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) raw[row][c0 + j] = u[j];
        }
      }
    }
    __syncthreads();
    // 8 tokens of one channel per thread: one 16-byte store (bf16) or two (f32)
    for (int i = tid; i < kRows * D / 8; i += kThreads) {
      const int t8 = i % 4, c = (i / 4) % D, gl = i / (4 * D);
      if (!tl.whole(gl)) continue;
      const int row0 = gl * kGroup + t8 * 8;
      const int64_t idx = (a.map.block(b, h, tl.group(gl)) * D + c) * kGroup + t8 * 8;
      uint32_t x[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = raw[row0 + k][c];
      if (vbf) {
        *reinterpret_cast<uint4*>((uint16_t*)a.vdense + idx) =
            make_uint4(x[0] | x[1] << 16, x[2] | x[3] << 16, x[4] | x[5] << 16, x[6] | x[7] << 16);
      } else {
        uint4* dst = reinterpret_cast<uint4*>((uint32_t*)a.vdense + idx);
        dst[0] = make_uint4(x[0], x[1], x[2], x[3]);
        dst[1] = make_uint4(x[4], x[5], x[6], x[7]);
      }
    }
  } else {
    // 2-bit values: per (token, 32-channel group) min/max grid, codes in matrix-operand order
#pragma unroll
    for (int k = 0; k < VMAX; ++k) {
      if (k < vpt) {
        const int i = tid + k * kThreads, row = i / vchunks, c0 = (i % vchunks) * vper;
        const uint32_t u[4] = {vr[k].x, vr[k].y, vr[k].z, vr[k].w};
        if (vbf) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ke[row][c0 + 2 * j] = __uint_as_float(u[j] << 16);
            ke[row][c0 + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) ke[row][c0 + j] = __uint_as_float(u[j]);
        }
      }
    }
    __syncthreads();
    // grid of (row, channel group) in the key step/zero arrays, now free: kRows * NG = GPW * D
    for (int i = tid; i < kRows * NG; i += kThreads) {
      const int row = i % kRows, gc = i / kRows, gl = row / kGroup, t = row % kGroup;
      float lo = ke[row][gc * 32], hi = lo;
#pragma unroll
      for (int c = 1; c < 32; ++c) {
        const float x = ke[row][gc * 32 + c];
        lo = x < lo ? x : lo;
        hi = x > hi ? x : hi;
      }
      float s, z, inv;
      uint16_t sb, zb;
      minmax_step_zero(lo, hi, 3.0f, s, z, inv, sb, zb);
      if (tl.whole(gl)) {
        const int64_t gabs = a.map.block(b, h, tl.group(gl));
        a.vmeta[(gabs * 2 + 0) * NG * kGroup + gc * kGroup + t] = sb;
        a.vmeta[(gabs * 2 + 1) * NG * kGroup + gc * kGroup + t] = zb;
      }
      s_s[row * NG + gc] = s;
      z_s[row * NG + gc] = z;
      inv_s[row * NG + gc] = inv;
    }
    __syncthreads();
    // group block of d*8 code bytes: lane l = 16*quad + n owns d/8 bytes, two per 16-channel
    // tile ct (channel 16*ct + n, tokens 8*quad .. 8*quad+7); token item i = 4q + 2b + e of the
    // eight sits in byte b of the pair at bit 4e + 2q
    for (int i = tid; i < GPW * D * 8; i += kThreads) {
      const int gl = i / (D * 8), byte = i % (D * 8);
      const int ln = byte / (D / 8), within = byte % (D / 8);
      const int c = 16 * (within / 2) + ln % 16, bb = within % 2, gc = c / 32;
      const int t0 = 8 * (ln / 16) + 2 * bb;
      uint32_t v = 0;
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int row = gl * kGroup + t0 + 4 * q + e;
          v |= base_code(ke[row][c], z_s[row * NG + gc], inv_s[row * NG + gc], 3.0f) << (4 * e + 2 * q);
        }
      if (tl.whole(gl)) a.vcode[a.map.block(b, h, tl.group(gl)) * D * 8 + byte] = (uint8_t)v;
    }
    if (prot) {
      // 6. the A^2 value policy: w_j * e_j per row (reads what the code loop reads)
      if (tid < kRows) {
        const int row = tid;
        float e = 0.0f;
        for (int c = 0; c < D; ++c) {
          const int m = row * NG + c / 32;
          const uint32_t code = base_code(ke[row][c], z_s[m], inv_s[m], 3.0f);
          const float diff = ke[row][c] - __builtin_fmaf((float)code, s_s[m], z_s[m]);
          e = __builtin_fmaf(diff, diff, e);
        }
        pr_s[row] = ldexp((double)e, pn_s[row]);
      }
      __syncthreads();
      const int NP = a.value_protect;
      if (tid < kRows) {
        const int gl = tid / kGroup, t = tid % kGroup;
        const double me = pr_s[tid];
        int rank = 0;
        for (int u = 0; u < kGroup; ++u) {
          const double o = pr_s[gl * kGroup + u];
          rank += (o > me || (o == me && u < t)) ? 1 : 0;
        }
        sel_s[tid] = rank < NP;
      }
      __syncthreads();
      if (tid < kRows && sel_s[tid]) {
        const int gl = tid / kGroup, t = tid % kGroup;
        int slot = 0;
        for (int u = 0; u < t; ++u) slot += sel_s[gl * kGroup + u];
        tok_s[gl][slot] = t;
      }
      __syncthreads();
      if (tid < GPW && tl.whole(tid)) {
        uint32_t word = 0;
        for (int k = 0; k < NP; ++k) word |= (uint32_t)tok_s[tid][k] << (8 * k);
        a.vpidx[a.map.block(b, h, tl.group(tid))] = word;
      }
      for (int i = tid; i < GPW * NP * D; i += kThreads) {
        const int gl = i / (NP * D), k = (i / D) % NP, c = i % D;
        if (!tl.whole(gl)) continue;
        const int row = gl * kGroup + tok_s[gl][k];
        const int m = row * NG + c / 32;
        const uint32_t code = base_code(ke[row][c], z_s[m], inv_s[m], 3.0f);
        const float dlt = ke[row][c] - __builtin_fmaf((float)code, s_s[m], z_s[m]);
        a.vprot[(a.map.block(b, h, tl.group(gl)) * NP + k) * D + c] = __builtin_bit_cast(uint16_t, (__bf16)dlt);
      }
    }
  }
  }  // values

  if (blockIdx.x == 0 && (st + a.n_new) % kGroup) {
    __syncthreads();  // every tail row this workgroup read has been consumed
    write_tails(a, st, tl.bh, D, kin, KBF16 ? 2 : 4, vin, ves);
  }
}

template <int D, int R>
hipError_t launch_dr(const AppendArgs& a, hipStream_t s) {
  const int64_t end = a.start + a.n_new;
  // groups the range touches; with per-row positions, the most any row can touch
  const int64_t n_touch = a.row_start ? (a.n_new + kGroup - 1) / kGroup + 1 : (end + kGroup - 1) / kGroup - a.start / kGroup;
  // small launches (at most ~8 groups per CU): one group per workgroup, U_h from LDS; long
  // writes: two groups per workgroup, U_h through scalar loads
  const bool small = n_touch * a.hkv * a.batch <= 2048;
  dim3 grid((unsigned)(small ? n_touch : (n_touch + 1) / 2), (unsigned)a.hkv, (unsigned)a.batch);
  if (a.key_bf16) {
    if (small)
      hipLaunchKernelGGL((append_kernel<D, R, true, true, 1>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((append_kernel<D, R, true, false, 2>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (small)
      hipLaunchKernelGGL((append_kernel<D, R, false, true, 1>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((append_kernel<D, R, false, false, 2>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AppendArgs& a, hipStream_t s) {
  switch (a.r) {
    case 0: return launch_dr<D, 0>(a, s);
    case 4: return launch_dr<D, 4>(a, s);
    case 8: return launch_dr<D, 8>(a, s);
    case 16: return launch_dr<D, 16>(a, s);
    case 32: return launch_dr<D, 32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.d == 64) return launch_d<64>(a, s);
  if (a.d == 128) return launch_d<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace headq
