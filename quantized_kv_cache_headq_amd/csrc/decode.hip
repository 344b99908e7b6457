// decode.hip — headq_decode_attn on gfx950: HeadQ cache read with split-token softmax.
//
// HeadQ technical summary ("Technische Samenvatting"), §3 step 3 (Cache Uitlezen): the runtime
// query decodes the side code through U_h^T q and the logit is corrected additively,
//     s_j = q.k_base_j / sqrt(d) + (U_h^T q).z_hat_j / sqrt(d),
// followed by softmax over the cached tokens and the readout sum_j p_j v_j (§1, §2.2).
//
// Work decomposition: grid (splits, KV heads, batch). A workgroup owns one contiguous range of
// 32-token groups of one (b, h) stream and all g = Hq/Hkv query heads that read it, so every
// cache byte is read once per call. Logits are kept in log2 units (the query is pre-scaled by
// log2(e)/sqrt(d)) so the softmax uses exp2. Per group:
//   A  logits for 32 tokens x g heads: base term from the 2-bit codes and the binary16 grid,
//      correction sigma_j * (sum_i qu_i u_ji - 8 sum_i qu_i) from the offset-binary nibbles
//   B  online-softmax update of the running max / sum per head (16-lane shuffle reductions)
//   C  rescale the output accumulators and add p . V for the group
// Each workgroup writes (max, sum, unnormalised output) per head; a second kernel merges the
// splits by log-sum-exp and normalises.
#include <hip/hip_runtime.h>

#include "headq_internal.h"

namespace headq {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

template <int D, int R, int VMODE, bool VBF16>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int RU = R > 0 ? R : 1;
  constexpr int HS = kThreads / D;  // head sets in phase C (2 for d=128, 4 for d=64)
  constexpr int HPT = kMaxGqa / HS; // max heads per thread in phase C
  __shared__ float qbar[kMaxGqa][D];
  __shared__ float qu[kMaxGqa][RU];
  __shared__ float qusum[kMaxGqa];
  __shared__ float sz[2][D];            // step and zero of the current group
  __shared__ float sc[kMaxGqa][kGroup]; // logits, then probabilities
  __shared__ float m_s[kMaxGqa], l_s[kMaxGqa], alpha_s[kMaxGqa];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int g = a.gqa;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int hq0 = h * g;  // first query head of this KV head
  const float qscale = kLog2e / sqrtf((float)D);

  // prologue: scaled queries and their projection on U_h
  for (int i = tid; i < g * D; i += kThreads) {
    const int hh = i / D, c = i % D;
    const int64_t qi = ((int64_t)b * a.hq + hq0 + hh) * D + c;
    const float x = a.query_bf16 ? bf16_to_f32(((const uint16_t*)a.q)[qi]) : ((const float*)a.q)[qi];
    qbar[hh][c] = x * qscale;
  }
  if (tid < kMaxGqa) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.0f;
  }
  __syncthreads();
  if constexpr (R > 0) {
    const float* Uh = a.U + (int64_t)h * D * R;
    for (int i = tid; i < g * R; i += kThreads) {
      const int hh = i / R, r = i % R;
      float acc = 0.0f;
      for (int c = 0; c < D; ++c) acc = fmaf(Uh[c * R + r], qbar[hh][c], acc);
      qu[hh][r] = acc;
    }
    __syncthreads();
    if (tid < g) {
      float s = 0.0f;
      for (int r = 0; r < R; ++r) s += qu[tid][r];
      qusum[tid] = s;
    }
  }

  // phase C ownership: channel c, heads hs, hs + HS, ...
  const int c_own = tid % D, hs = tid / D;
  float o[HPT];
#pragma unroll
  for (int j = 0; j < HPT; ++j) o[j] = 0.0f;

  // whole groups, then (index n_groups) the unfinished group held exactly in the tails
  int64_t n_ctx = a.n_ctx;  // this row's attended tokens
  if (a.row_len) {
    const int64_t r = a.row_len[b];
    n_ctx = r < 0 ? 0 : (r > a.n_ctx ? a.n_ctx : r);
  }
  const int64_t n_groups = n_ctx / kGroup;
  const int tail_len = (int)(n_ctx % kGroup);
  const int64_t n_units = n_groups + (tail_len ? 1 : 0);
  const int64_t g_begin = (int64_t)split * a.groups_per_split;
  int64_t g_end = g_begin + a.groups_per_split;
  if (g_end > n_units) g_end = n_units;

  for (int64_t gi = g_begin; gi < g_end; ++gi) {
    const bool is_tail = gi == n_groups;
    __syncthreads();  // previous group fully consumed
    if (is_tail) {
      // A (tail): exact logits q.k over the tail rows; rows past n_ctx get -inf
      const int t = tid / 8, sub = tid % 8;
      for (int hh = sub; hh < g; hh += 8) {
        float acc = -INFINITY;
        if (t < tail_len) {
          acc = 0.0f;
          const int64_t row = (bh * kGroup + t) * D;
          for (int c = 0; c < D; ++c) {
            const float k = a.key_bf16 ? bf16_to_f32(((const uint16_t*)a.ktail)[row + c]) : ((const float*)a.ktail)[row + c];
            acc = fmaf(qbar[hh][c], k, acc);
          }
          if (a.logits_dbg) a.logits_dbg[((int64_t)b * a.hq + hq0 + hh) * a.n_ctx + gi * kGroup + t] = acc * kLn2;
        }
        sc[hh][t] = acc;
      }
    } else if (tid < D) {
      const uint16_t* meta = a.kmeta + a.map.block(b, h, gi) * 2 * D;
      sz[0][tid] = f16_bits_to_f32(meta[tid]);
      sz[1][tid] = f16_bits_to_f32(meta[D + tid]);
    }
    __syncthreads();

    // A: logits. thread (token t, heads sub, sub + 8)
    if (!is_tail) {
      const int t = tid / 8, sub = tid % 8;
      const int64_t tok = gi * kGroup + t;
      const int64_t trow = a.map.row(b, h, tok);
      const bool nib = a.key_nib;  // 3- or 4-bit codes, one per nibble (rows of d/2 bytes)
      const uint32_t* kc = (const uint32_t*)(a.kcode + trow * (nib ? D / 2 : D / 4));
      uint32_t words[D / 8];
#pragma unroll
      for (int w = 0; w < D / 8; ++w) words[w] = (nib || w < D / 16) ? kc[w] : 0u;
      float sg = 0.0f;
      uint32_t sw[RU / 8 > 0 ? RU / 8 : 1];
      if constexpr (R > 0) {
        sg = f16_bits_to_f32(a.ssc[trow]);
        const uint8_t* sp = a.scode + trow * (R / 2);
        if constexpr (R >= 8) {
#pragma unroll
          for (int w = 0; w < R / 8; ++w) sw[w] = ((const uint32_t*)sp)[w];
        } else {
          sw[0] = *(const uint16_t*)sp;
        }
      }
      for (int hh = sub; hh < g; hh += 8) {
        float acc = 0.0f;
        if (nib) {
#pragma unroll
          for (int c = 0; c < D; ++c) {
            const float code = (float)((words[c / 8] >> kcode4_bit(c % 8)) & 15u);
            acc = fmaf(qbar[hh][c], fmaf(code, sz[0][c], sz[1][c]), acc);
          }
        } else {
#pragma unroll
          for (int c = 0; c < D; ++c) {
            const float code = (float)((words[c / 16] >> kcode_bit(c % 16)) & 3u);
            acc = fmaf(qbar[hh][c], fmaf(code, sz[0][c], sz[1][c]), acc);
          }
        }
        if constexpr (R > 0) {
          float cs = 0.0f;
#pragma unroll
          for (int i = 0; i < R; ++i) cs = fmaf(qu[hh][i], (float)((sw[i / 8] >> (4 * (i % 8))) & 15u), cs);
          acc = fmaf(a.corr_scale * sg, cs - 8.0f * qusum[hh], acc);
        }
        sc[hh][t] = acc;
        if (a.logits_dbg) a.logits_dbg[((int64_t)b * a.hq + hq0 + hh) * a.n_ctx + tok] = acc * kLn2;
      }
    }
    __syncthreads();

    // B: online softmax per head: 16 lanes per head, 2 tokens per lane
    {
      const int hh = tid / 16, k = tid % 16;
      if (hh < g) {
        const float x0 = sc[hh][2 * k], x1 = sc[hh][2 * k + 1];
        float mx = fmaxf(x0, x1);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
        const float m_old = m_s[hh];
        const float m_new = fmaxf(m_old, mx);
        const float p0 = exp2f(x0 - m_new), p1 = exp2f(x1 - m_new);
        sc[hh][2 * k] = p0;
        sc[hh][2 * k + 1] = p1;
        float sum = p0 + p1;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off, 16);
        if (k == 0) {
          const float al = exp2f(m_old - m_new);  // 0 on the first group (m_old = -inf)
          alpha_s[hh] = al;
          l_s[hh] = l_s[hh] * al + sum;
          m_s[hh] = m_new;
        }
      }
    }
    __syncthreads();

    // C: o = o * alpha + p . V
    {
      float v[kGroup];
      const int64_t gabs = is_tail ? 0 : a.map.block(b, h, gi);
      if (is_tail) {
        // exact tail values, zero past n_ctx (their probabilities are 0)
#pragma unroll
        for (int t = 0; t < kGroup; ++t) {
          const int64_t idx = (bh * kGroup + t) * D + c_own;
          v[t] = t >= tail_len ? 0.0f
                 : a.value_bf16 ? bf16_to_f32(((const uint16_t*)a.vtail)[idx]) : ((const float*)a.vtail)[idx];
        }
      } else if constexpr (VMODE == HEADQ_V_DENSE) {
        if constexpr (VBF16) {
          const uint4* src = (const uint4*)((const uint16_t*)a.vdense + (gabs * D + c_own) * kGroup);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint4 x = src[w];
            const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              v[w * 8 + 2 * j] = __uint_as_float(u[j] << 16);
              v[w * 8 + 2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
            }
          }
        } else {
          const float4* src = (const float4*)((const float*)a.vdense + (gabs * D + c_own) * kGroup);
#pragma unroll
          for (int w = 0; w < 8; ++w) {
            const float4 x = src[w];
            v[4 * w] = x.x;
            v[4 * w + 1] = x.y;
            v[4 * w + 2] = x.z;
            v[4 * w + 3] = x.w;
          }
        }
      } else {
        constexpr int NG = D / 32;
        const int gc = c_own / 32;
        uint32_t cw[4];  // the channel's 16-bit code pairs of tokens 8*qd .. 8*qd+7
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          cw[qd] = *(const uint16_t*)(a.vcode + gabs * D * 8 + vcode_pair_offset(D, c_own, 8 * qd));
        const uint16_t* vs = a.vmeta + (gabs * 2 + 0) * NG * kGroup + gc * kGroup;
        const uint16_t* vz = a.vmeta + (gabs * 2 + 1) * NG * kGroup + gc * kGroup;
#pragma unroll
        for (int t = 0; t < kGroup; ++t) {
          const float code = (float)((cw[t / 8] >> vcode_pair_bit(t)) & 3u);
          v[t] = fmaf(code, f16_bits_to_f32(vs[t]), f16_bits_to_f32(vz[t]));
        }
      }
#pragma unroll
      for (int j = 0; j < HPT; ++j) {
        const int hh = hs + j * HS;
        if (hh < g) {
          float acc = o[j] * alpha_s[hh];
#pragma unroll
          for (int t = 0; t < kGroup; ++t) acc = fmaf(sc[hh][t], v[t], acc);
          o[j] = acc;
        }
      }
    }
  }

  // partials: unnormalised output, running max and sum per head
#pragma unroll
  for (int j = 0; j < HPT; ++j) {
    const int hh = hs + j * HS;
    if (hh < g) a.ws_o[(((int64_t)b * a.hq + hq0 + hh) * a.n_splits + split) * D + c_own] = o[j];
  }
  if (tid < g) {
    float* ml = a.ws_ml + (((int64_t)b * a.hq + hq0 + tid) * a.n_splits + split) * 2;
    ml[0] = m_s[tid];
    ml[1] = l_s[tid];
  }
}

// Merge the splits of one (b, query head) by log-sum-exp and normalise.
template <int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, b = blockIdx.y, c = threadIdx.x;
  const int64_t row = (int64_t)b * a.hq + hq;
  const float* ml = a.ws_ml + row * a.n_splits * 2;
  float m = -INFINITY;
  for (int s = 0; s < a.n_splits; ++s) m = fmaxf(m, ml[2 * s]);
  float l = 0.0f, acc = 0.0f;
  for (int s = 0; s < a.n_splits; ++s) {
    const float ms = ml[2 * s];
    if (ms == -INFINITY) continue;  // empty split
    const float w = exp2f(ms - m);
    l = fmaf(ml[2 * s + 1], w, l);
    acc = fmaf(a.ws_o[(row * a.n_splits + s) * D + c], w, acc);
  }
  const float o = l > 0.0f ? acc / l : 0.0f;  // a row without tokens reads out zeros
  if (a.out_bf16)
    ((__bf16*)a.out)[row * D + c] = (__bf16)o;
  else
    ((float*)a.out)[row * D + c] = o;
}

template <int D, int R>
hipError_t launch_split(const DecodeArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.n_splits, (unsigned)a.hkv, (unsigned)a.batch);
  if (a.value_mode == HEADQ_V_Q2)
    hipLaunchKernelGGL((decode_split_kernel<D, R, HEADQ_V_Q2, false>), grid, dim3(kThreads), 0, s, a);
  else if (a.value_bf16)
    hipLaunchKernelGGL((decode_split_kernel<D, R, HEADQ_V_DENSE, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<D, R, HEADQ_V_DENSE, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.use_mfma) return launch_decode_mfma_split(a, s);  // merges the splits itself
  switch (a.r) {
    case 0: e = launch_split<D, 0>(a, s); break;
    case 4: e = launch_split<D, 4>(a, s); break;
    case 8: e = launch_split<D, 8>(a, s); break;
    case 16: e = launch_split<D, 16>(a, s); break;
    case 32: e = launch_split<D, 32>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3((unsigned)a.hq, (unsigned)a.batch), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.d == 64) return launch_d<64>(a, s);
  if (a.d == 128) return launch_d<128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace headq
