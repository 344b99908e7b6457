// append.hip — headq_cache_append on gfx950: the HeadQ cache write.
//
// HeadQ technical summary ("Technische Samenvatting"), §3 step 2 (Cache Schrijven): base-quantize
// each key (k_base = B_b(k)), form the residual e = k - k_base, project it on the calibration
// basis and side-quantize the projection, z = Q_q(U_h^T e); the cache keeps the base code and z.
//
// One workgroup (256 threads, 4 wave64) owns one 32-token group of one (b, h) stream:
//   1. the 32 x d key tile is loaded with 128-bit loads into LDS as f32
//   2. per channel: min/max over the 32 tokens -> binary16 step s and zero z (kmeta)
//   3. per (token, 16 channels): 2-bit codes (one 32-bit store) and residuals (back into LDS)
//   4. per (token, component block): y = U^T e as one sequential f32 fma chain per component
//      (channel order 0..d-1, the canonical order that makes the side codes reproducible),
//      then the per-token symmetric 4-bit side quantizer and nibble packing.
// Values (when given) are written by separate kernels: dense values are transposed into the
// channel-major group layout, 2-bit values quantized per (token, 32-channel group).
//
// Numerics: no contraction anywhere in this file (every fma is explicit), IEEE division,
// rint = round half to even, binary16 conversion with round to nearest even.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>

#include "headq_internal.h"

namespace headq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  _Float16 h = (_Float16)x;  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Load a 32 x D tile of f32/bf16 rows (element stride 1 along channels, row stride ts) into an
// f32 LDS tile with row pitch P.
template <int D, int P, bool BF16>
__device__ __forceinline__ void load_tile(float (*dst)[P], const void* src, int64_t ts) {
  constexpr int kElem = BF16 ? 8 : 4;          // elements per 16-byte load
  constexpr int kChunks = D / kElem;           // 16-byte chunks per row
  for (int i = threadIdx.x; i < kGroup * kChunks; i += kThreads) {
    const int t = i / kChunks, ch = i % kChunks;
    if constexpr (BF16) {
      const uint4 w = *reinterpret_cast<const uint4*>((const uint16_t*)src + (int64_t)t * ts + ch * kElem);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dst[t][ch * 8 + 2 * j] = __uint_as_float(u[j] << 16);
        dst[t][ch * 8 + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
      }
    } else {
      const float4 w = *reinterpret_cast<const float4*>((const float*)src + (int64_t)t * ts + ch * kElem);
      dst[t][ch * 4 + 0] = w.x;
      dst[t][ch * 4 + 1] = w.y;
      dst[t][ch * 4 + 2] = w.z;
      dst[t][ch * 4 + 3] = w.w;
    }
  }
}

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

__device__ __forceinline__ uint32_t base_code(float k, float z, float inv) {
  float c = __builtin_rintf((k - z) * inv);
  c = c < 0.0f ? 0.0f : c;
  c = c > 3.0f ? 3.0f : c;
  return (uint32_t)c;
}

template <int D, int R, bool KBF16>
__global__ __launch_bounds__(kThreads) void append_keys_kernel(AppendArgs a) {
  constexpr int P = D + 4;  // LDS row pitch (floats): spreads token rows over the banks
  constexpr int RU = R > 0 ? R : 1;
  __shared__ float ke[kGroup][P];  // keys, then residuals
  __shared__ float Us[D][RU];
  __shared__ float s_s[D], z_s[D], inv_s[D];

  const int grp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t tok0 = a.start + (int64_t)grp * kGroup;  // first cache token of this group

  const char* kin = (const char*)a.k + ((int64_t)b * a.ks_b + (int64_t)h * a.ks_h + (int64_t)grp * kGroup * a.ks_t) *
                                           (KBF16 ? 2 : 4);
  load_tile<D, P, KBF16>(ke, kin, a.ks_t);
  if constexpr (R > 0) {
    const float* Uh = a.U + (int64_t)h * D * R;
    for (int i = tid; i < D * R; i += kThreads) Us[i / R][i % R] = Uh[i];
  }
  __syncthreads();

  // 2. per-channel step and zero (binary16) over the group
  if (tid < D) {
    float lo = ke[0][tid], hi = lo;
    for (int t = 1; t < kGroup; ++t) {
      const float x = ke[t][tid];
      lo = x < lo ? x : lo;
      hi = x > hi ? x : hi;
    }
    float s, z, inv;
    uint16_t sb, zb;
    minmax_step_zero(lo, hi, 3.0f, s, z, inv, sb, zb);
    uint16_t* meta = a.kmeta + (bh * (a.cap / kGroup) + tok0 / kGroup) * 2 * D;
    meta[tid] = sb;
    meta[D + tid] = zb;
    s_s[tid] = s;
    z_s[tid] = z;
    inv_s[tid] = inv;
  }
  __syncthreads();

  // 3. codes (16 channels -> one 32-bit word) and residuals e = k - fma(code, s, z)
  for (int i = tid; i < kGroup * (D / 16); i += kThreads) {
    const int t = i / (D / 16), c0 = (i % (D / 16)) * 16;
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = c0 + j;
      const float k = ke[t][c];
      const uint32_t code = base_code(k, z_s[c], inv_s[c]);
      word |= code << kcode_bit(j);
      ke[t][c] = k - __builtin_fmaf((float)code, s_s[c], z_s[c]);
    }
    *reinterpret_cast<uint32_t*>(a.kcode + (bh * a.cap + tok0 + t) * (D / 4) + c0 / 4) = word;
  }

  if constexpr (R > 0) {
    __syncthreads();
    // 4. side code: TPT threads per token, CPT consecutive components each
    constexpr int TPT = (R / 2) < 8 ? (R / 2) : 8;
    constexpr int CPT = R / TPT;  // 2 or 4
    const int t = tid / TPT, sub = tid % TPT;
    if (t < kGroup) {
      const int i0 = sub * CPT;
      float y[CPT];
#pragma unroll
      for (int j = 0; j < CPT; ++j) y[j] = 0.0f;
      for (int c = 0; c < D; c += 4) {
        const float4 e4 = *reinterpret_cast<const float4*>(&ke[t][c]);
        const float e[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int j = 0; j < CPT; ++j) y[j] = __builtin_fmaf(Us[c + cc][i0 + j], e[cc], y[j]);
      }
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const float m = __builtin_fabsf(y[j]);
        amax = m > amax ? m : amax;
      }
#pragma unroll
      for (int off = 1; off < TPT; off <<= 1) {
        const float o = __shfl_xor(amax, off, TPT);
        amax = o > amax ? o : amax;
      }
      const uint16_t sg_bits = f32_to_f16_bits(amax / 7.0f);
      const float sg = f16_bits_to_f32(sg_bits);
      const float inv = (sg == 0.0f) ? 0.0f : 1.0f / sg;
      uint32_t packed = 0;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        float zc = __builtin_rintf(y[j] * inv);
        zc = zc < -7.0f ? -7.0f : zc;
        zc = zc > 7.0f ? 7.0f : zc;
        packed |= (uint32_t)((int)zc + 8) << (4 * j);
      }
      uint8_t* row = a.scode + (bh * a.cap + tok0 + t) * (R / 2) + i0 / 2;
      if constexpr (CPT == 4)
        *reinterpret_cast<uint16_t*>(row) = (uint16_t)packed;
      else
        *row = (uint8_t)packed;
      if (sub == 0) a.ssc[bh * a.cap + tok0 + t] = sg_bits;
    }
  }
}

// Dense values: copy a 32-token group into the channel-major group layout [d][32].
template <int D, bool VBF16>
__global__ __launch_bounds__(kThreads) void append_values_dense_kernel(AppendArgs a) {
  using E = typename std::conditional<VBF16, uint16_t, uint32_t>::type;
  __shared__ E tile[kGroup][D + (VBF16 ? 2 : 1)];
  const int grp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t tok0 = a.start + (int64_t)grp * kGroup;
  const E* src = (const E*)a.v + (int64_t)b * a.vs_b + (int64_t)h * a.vs_h + (int64_t)grp * kGroup * a.vs_t;
  for (int i = threadIdx.x; i < kGroup * D; i += kThreads) {
    const int t = i / D, c = i % D;
    tile[t][c] = src[(int64_t)t * a.vs_t + c];
  }
  __syncthreads();
  E* dst = (E*)a.vdense + (bh * (a.cap / kGroup) + tok0 / kGroup) * (int64_t)D * kGroup;
  for (int i = threadIdx.x; i < kGroup * D; i += kThreads) {
    const int c = i / kGroup, t = i % kGroup;
    dst[i] = tile[t][c];
  }
}

// 2-bit values: per (token, 32-channel group) min/max quantizer, stored channel-major per group.
template <int D, bool VBF16>
__global__ __launch_bounds__(kThreads) void append_values_q2_kernel(AppendArgs a) {
  constexpr int P = D + 1;
  constexpr int NG = D / 32;
  __shared__ float tile[kGroup][P];
  __shared__ float s_s[kGroup][NG], z_s[kGroup][NG], inv_s[kGroup][NG];
  const int grp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int64_t tok0 = a.start + (int64_t)grp * kGroup;
  const int64_t g_abs = bh * (a.cap / kGroup) + tok0 / kGroup;
  const int64_t base = (int64_t)b * a.vs_b + (int64_t)h * a.vs_h + (int64_t)grp * kGroup * a.vs_t;
  for (int i = threadIdx.x; i < kGroup * D; i += kThreads) {
    const int t = i / D, c = i % D;
    tile[t][c] = VBF16 ? bf16_to_f32(((const uint16_t*)a.v)[base + (int64_t)t * a.vs_t + c])
                       : ((const float*)a.v)[base + (int64_t)t * a.vs_t + c];
  }
  __syncthreads();
  if (threadIdx.x < kGroup * NG) {
    const int t = threadIdx.x % kGroup, gc = threadIdx.x / kGroup;
    float lo = tile[t][gc * 32], hi = lo;
    for (int c = 1; c < 32; ++c) {
      const float x = tile[t][gc * 32 + c];
      lo = x < lo ? x : lo;
      hi = x > hi ? x : hi;
    }
    float s, z, inv;
    uint16_t sb, zb;
    minmax_step_zero(lo, hi, 3.0f, s, z, inv, sb, zb);
    a.vmeta[(g_abs * 2 + 0) * NG * kGroup + gc * kGroup + t] = sb;
    a.vmeta[(g_abs * 2 + 1) * NG * kGroup + gc * kGroup + t] = zb;
    s_s[t][gc] = s;
    z_s[t][gc] = z;
    inv_s[t][gc] = inv;
  }
  __syncthreads();
  // Group block of d*8 code bytes in matrix-operand order: lane l = 16*quad + n owns d/8 bytes,
  // two per 16-channel tile ct (channel 16*ct + n, tokens 8*quad .. 8*quad+7); token item
  // i = 4q + 2b + e of the eight sits in byte b of the pair at bit 4e + 2q.
  for (int i = threadIdx.x; i < D * 8; i += kThreads) {
    const int lane = i / (D / 8), within = i % (D / 8);
    const int c = 16 * (within / 2) + lane % 16, bb = within % 2, gc = c / 32;
    const int t0 = 8 * (lane / 16) + 2 * bb;
    uint32_t byte = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int t = t0 + 4 * q + e;
        byte |= base_code(tile[t][c], z_s[t][gc], inv_s[t][gc]) << (4 * e + 2 * q);
      }
    a.vcode[g_abs * D * 8 + i] = (uint8_t)byte;
  }
}

template <int D, int R>
hipError_t launch_keys(const AppendArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.n_new / kGroup), (unsigned)a.hkv, (unsigned)a.batch);
  if (a.key_bf16)
    hipLaunchKernelGGL((append_keys_kernel<D, R, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((append_keys_kernel<D, R, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AppendArgs& a, hipStream_t s) {
  hipError_t e;
  switch (a.r) {
    case 0: e = launch_keys<D, 0>(a, s); break;
    case 4: e = launch_keys<D, 4>(a, s); break;
    case 8: e = launch_keys<D, 8>(a, s); break;
    case 16: e = launch_keys<D, 16>(a, s); break;
    case 32: e = launch_keys<D, 32>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || !a.v) return e;
  dim3 grid((unsigned)(a.n_new / kGroup), (unsigned)a.hkv, (unsigned)a.batch);
  if (a.value_mode == HEADQ_V_DENSE) {
    if (a.value_bf16)
      hipLaunchKernelGGL((append_values_dense_kernel<D, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((append_values_dense_kernel<D, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (a.value_bf16)
      hipLaunchKernelGGL((append_values_q2_kernel<D, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((append_values_q2_kernel<D, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.d == 64) return launch_d<64>(a, s);
  if (a.d == 128) return launch_d<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace headq
