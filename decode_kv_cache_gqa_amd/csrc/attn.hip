// Split-K GQA decode attention that exposes per-token logits, with the
// step's new token appended on the way.
//
// Per (layer l, group g = (sequence, KV head), split of tokens) and for the
// HG query heads that share the KV head:
//   s[h][t] = (q_h . k_t) / sqrt(d)          ("QEvict" review, section 4.1,
//                                              (Attention))
//   m[h] = max_t s, l[h] = sum_t exp(s - m), o[h][:] = sum_t exp(s - m) v_t
// The logits are stored (fp32) for the probability pass, which normalises
// them once every split's (m, l) is merged; the post kernel does the merge.
// The group's cache holds count[g] tokens in slots [0, count); the new
// token is slot count[g] and is read from k_new / v_new, then written to its
// page by the block that owns that slot.
#include "common.h"
#include "kvev_internal.h"

namespace kvev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& r) {
  bf16x8 v;
  __builtin_memcpy(&v, &r, sizeof(v));
  return v;
}

// ---------------------------------------------------------------------------
// bf16, head_dim 128, group of 4 query heads: q.K^T on MFMA, p.V on VALU.
//
// A wave owns NG groups of 16 consecutive slots (one cache page each).  For
// group j it loads, with all loads of all groups issued before any use:
//   K (MFMA B operand): lane (r16, q4) reads slot r16, channels
//     32*s + 8*q4 .. +8 for k-steps s = 0..3 (16-byte loads);
//   V (p.V layout):      lane (r16, q4) reads slot q4 + 4*u, channels
//     8*r16 .. +8 for u = 0..3.
// v_mfma_f32_16x16x32_bf16 with A = the 4 query rows (rows 4..15 zero) gives
// lane r16 (q4 == 0) the 4 heads' logits of slot r16.
// ---------------------------------------------------------------------------
template <int NG, int NW>
__global__ __launch_bounds__(NW * kWave) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
    const int* __restrict__ ptab, const int* __restrict__ count, float* __restrict__ logits,
    float* __restrict__ part_ml, float* __restrict__ part_o, int L, int G, int Hkv, int Hq,
    int64_t P, int maxpages, int64_t cap, int S, float scale, int write_logits) {
  constexpr int D = 128, HG = 4;
  constexpr int WT = NG * 16;   // slots per wave
  constexpr int CT = NW * WT;   // slots per block
  __shared__ __align__(16) float p_lds[NW][WT][HG];
  __shared__ __align__(16) float wstat[NW][HG][2];
  __shared__ __align__(16) float o_lds[NW][HG][D];

  const int split = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int t0 = split * CT;
  const int wt0 = t0 + wave * WT;
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
  // page indices do not depend on the count: load them alongside it
  int pages[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) pages[j] = pt[min((wt0 + 16 * j) / kPageTokens, maxpages - 1)];
  const int n = count[g] + 1;  // slots including the new token
  if (t0 >= n) return;
  const int B = G / Hkv, b = g / Hkv, kvh = g % Hkv;
  const int r16 = lane % 16, q4 = lane / 16;
  const int tnew = n - 1;
  const int64_t new_off = (static_cast<int64_t>(l * B + b) * Hkv + kvh) * D;

  bf16x8 qa[4];
  {
    uint4 z = make_uint4(0, 0, 0, 0);
    const uint16_t* qp = q + (static_cast<int64_t>(l * B + b) * Hq + kvh * HG + (r16 < HG ? r16 : 0)) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 r = r16 < HG ? *reinterpret_cast<const uint4*>(qp + 32 * s + 8 * q4) : z;
      qa[s] = as_bf16x8(r);
    }
  }

  uint4 kr[NG][4], vr[NG][4];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int gbase = wt0 + 16 * j;
    const int64_t prow = pool_row(l, pages[j], 0, 0, P, 1, kPageTokens);
    const int tk = gbase + r16;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 r = make_uint4(0, 0, 0, 0);
      if (tk < n) {
        const uint16_t* src = (tk == tnew) ? k_new + new_off : kpool + (prow + r16) * D;
        r = *reinterpret_cast<const uint4*>(src + 32 * s + 8 * q4);
      }
      kr[j][s] = r;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tv = gbase + q4 + 4 * u;
      uint4 r = make_uint4(0, 0, 0, 0);
      if (tv < n) {
        const uint16_t* src = (tv == tnew) ? v_new + new_off : vpool + (prow + q4 + 4 * u) * D;
        r = *reinterpret_cast<const uint4*>(src + 8 * r16);
      }
      vr[j][u] = r;
    }
  }

  // append: the lanes holding the new token write it into its page slot
  if (tnew >= wt0 && tnew < wt0 + WT) {
    const int j = (tnew - wt0) / 16;
    const int64_t row = pool_row(l, pt[tnew / kPageTokens], 0, tnew % kPageTokens, P, 1, kPageTokens) * D;
#pragma unroll
    for (int jj = 0; jj < NG; ++jj) {
      if (jj != j) continue;
      if (wt0 + 16 * jj + r16 == tnew) {
#pragma unroll
        for (int s = 0; s < 4; ++s) *reinterpret_cast<uint4*>(kpool + row + 32 * s + 8 * q4) = kr[jj][s];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (wt0 + 16 * jj + q4 + 4 * u == tnew) *reinterpret_cast<uint4*>(vpool + row + 8 * r16) = vr[jj][u];
    }
  }

  // logits on MFMA
  float sv[NG][HG];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], as_bf16x8(kr[j][s]), acc, 0, 0, 0);
    const int tk = wt0 + 16 * j + r16;
    const bool valid = q4 == 0 && tk < n;
#pragma unroll
    for (int h = 0; h < HG; ++h) sv[j][h] = valid ? acc[h] * scale : -INFINITY;
    if (valid && write_logits) {
      float4 o4 = make_float4(sv[j][0], sv[j][1], sv[j][2], sv[j][3]);
      *reinterpret_cast<float4*>(logits + ((static_cast<int64_t>(g) * L + l) * cap + tk) * HG) = o4;
    }
  }

  // wave max / exp / sum
  float mh[HG], lh[HG];
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    float m = sv[0][h];
#pragma unroll
    for (int j = 1; j < NG; ++j) m = fmaxf(m, sv[j][h]);
    mh[h] = wave_max(m);
  }
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float p = mh[h] == -INFINITY ? 0.f : __expf(sv[j][h] - mh[h]);
      sv[j][h] = p;
      sum += p;
    }
    lh[h] = wave_sum(sum);
  }
  if (q4 == 0) {
#pragma unroll
    for (int j = 0; j < NG; ++j)
      *reinterpret_cast<float4*>(&p_lds[wave][16 * j + r16][0]) =
          make_float4(sv[j][0], sv[j][1], sv[j][2], sv[j][3]);
  }
  __syncthreads();

  // p . V
  float acc[HG][8];
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float4 pp = *reinterpret_cast<const float4*>(&p_lds[wave][16 * j + q4 + 4 * u][0]);
      float vf[8];
      Vec16<bf16_t>::widen(vr[j][u], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[0][e] += pp.x * vf[e];
        acc[1][e] += pp.y * vf[e];
        acc[2][e] += pp.z * vf[e];
        acc[3][e] += pp.w * vf[e];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[h][e];
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      acc[h][e] = v;
    }
  if (q4 == 0) {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      *reinterpret_cast<float4*>(&o_lds[wave][h][8 * r16]) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *reinterpret_cast<float4*>(&o_lds[wave][h][8 * r16 + 4]) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      wstat[wave][h][0] = mh[h];
      wstat[wave][h][1] = lh[h];
    }
  }
  __syncthreads();

  // merge the block's waves into one partial
  const int64_t pbase = (static_cast<int64_t>(l) * G + g) * S + split;
  for (int idx = tid; idx < HG * D; idx += NW * kWave) {
    const int h = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wstat[w][h][0]);
    float o = 0.f, Z = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = wstat[w][h][0] == -INFINITY ? 0.f : __expf(wstat[w][h][0] - M);
      o += f * o_lds[w][h][c];
      Z += f * wstat[w][h][1];
    }
    part_o[pbase * HG * D + idx] = o;
    if (c == 0) {
      part_ml[(pbase * HG + h) * 2 + 0] = M;
      part_ml[(pbase * HG + h) * 2 + 1] = Z;
    }
  }
}

// ---------------------------------------------------------------------------
// Generic VALU version (fp32 or bf16, head_dim 64 or 128): lanes split each
// row into 16-byte pieces; dot products are reduced with cross-lane adds.
// Used for the fp32 cache and for head_dim 64.
// ---------------------------------------------------------------------------
template <typename T, int D, int HG, int NT, int CT>
__global__ __launch_bounds__(NT) void attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    T* __restrict__ kpool, T* __restrict__ vpool, const int* __restrict__ ptab,
    const int* __restrict__ count, float* __restrict__ logits, float* __restrict__ part_ml,
    float* __restrict__ part_o, int L, int G, int Hkv, int Hq, int64_t P, int maxpages, int64_t cap,
    int S, float scale, int write_logits) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPT = D / EPL;
  constexpr int TPW = kWave / LPT;
  constexpr int NW = NT / kWave;
  constexpr int U = 4;
  static_assert(LPT <= kWave && (kWave % LPT) == 0, "row must fit a wave");

  __shared__ float s_lds[CT][HG];
  __shared__ float red[NW][HG];
  __shared__ float o_lds[NW][HG][D];

  const int split = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int n = count[g] + 1;
  const int t0 = split * CT;
  if (t0 >= n) return;
  const int cnt = min(n - t0, CT);
  const int B = G / Hkv, b = g / Hkv, kvh = g % Hkv;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int sub = lane % LPT, tslot = lane / LPT;
  const int tnew = n - 1;
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
  const int64_t new_off = (static_cast<int64_t>(l * B + b) * Hkv + kvh) * D + sub * EPL;
  auto row_of = [&](int t) {
    return pool_row(l, pt[t / kPageTokens], 0, t % kPageTokens, P, 1, kPageTokens) * D + sub * EPL;
  };

  float qv[HG][EPL];
  {
    const T* qb = q + (static_cast<int64_t>(l * B + b) * Hq + kvh * HG) * D + sub * EPL;
#pragma unroll
    for (int h = 0; h < HG; ++h) Vec16<T>::widen(*reinterpret_cast<const uint4*>(qb + h * D), qv[h]);
  }

  for (int base = wave * TPW; base < cnt; base += NW * TPW * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NW * TPW + tslot;
      raw[u] = make_uint4(0, 0, 0, 0);
      if (i < cnt) {
        const int t = t0 + i;
        if (t == tnew) {
          raw[u] = *reinterpret_cast<const uint4*>(k_new + new_off);
          *reinterpret_cast<uint4*>(kpool + row_of(t)) = raw[u];
        } else {
          raw[u] = *reinterpret_cast<const uint4*>(kpool + row_of(t));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NW * TPW + tslot;
      float kf[EPL];
      Vec16<T>::widen(raw[u], kf);
      float acc[HG];
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a += qv[h][e] * kf[e];
        acc[h] = a;
      }
#pragma unroll
      for (int o = LPT / 2; o > 0; o >>= 1)
#pragma unroll
        for (int h = 0; h < HG; ++h) acc[h] += __shfl_xor(acc[h], o, kWave);
      if (i < cnt && sub == 0) {
        float* dst = logits + ((static_cast<int64_t>(g) * L + l) * cap + t0 + i) * HG;
#pragma unroll
        for (int h = 0; h < HG; ++h) {
          const float s = acc[h] * scale;
          s_lds[i][h] = s;
          if (write_logits) dst[h] = s;
        }
      }
    }
  }
  __syncthreads();

  float mx[HG], sm[HG];
#pragma unroll
  for (int h = 0; h < HG; ++h) mx[h] = -INFINITY;
  for (int i = tid; i < cnt; i += NT)
#pragma unroll
    for (int h = 0; h < HG; ++h) mx[h] = fmaxf(mx[h], s_lds[i][h]);
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    const float w = wave_max(mx[h]);
    if (lane == 0) red[wave][h] = w;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    float w = red[0][h];
#pragma unroll
    for (int k = 1; k < NW; ++k) w = fmaxf(w, red[k][h]);
    mx[h] = w;
    sm[h] = 0.f;
  }
  __syncthreads();
  for (int i = tid; i < cnt; i += NT)
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float p = __expf(s_lds[i][h] - mx[h]);
      s_lds[i][h] = p;
      sm[h] += p;
    }
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    const float w = wave_sum(sm[h]);
    if (lane == 0) red[wave][h] = w;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    float w = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) w += red[k][h];
    sm[h] = w;
  }

  float acc[HG][EPL];
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  for (int base = wave * TPW; base < cnt; base += NW * TPW * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NW * TPW + tslot;
      raw[u] = make_uint4(0, 0, 0, 0);
      if (i < cnt) {
        const int t = t0 + i;
        if (t == tnew) {
          raw[u] = *reinterpret_cast<const uint4*>(v_new + new_off);
          *reinterpret_cast<uint4*>(vpool + row_of(t)) = raw[u];
        } else {
          raw[u] = *reinterpret_cast<const uint4*>(vpool + row_of(t));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NW * TPW + tslot;
      if (i < cnt) {
        float vf[EPL];
        Vec16<T>::widen(raw[u], vf);
#pragma unroll
        for (int h = 0; h < HG; ++h) {
          const float p = s_lds[i][h];
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] += p * vf[e];
        }
      }
    }
  }
#pragma unroll
  for (int o = LPT; o < kWave; o <<= 1)
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], o, kWave);
  if (tslot == 0)
#pragma unroll
    for (int h = 0; h < HG; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o_lds[wave][h][sub * EPL + e] = acc[h][e];
  __syncthreads();
  const int64_t pbase = (static_cast<int64_t>(l) * G + g) * S + split;
  for (int idx = tid; idx < HG * D; idx += NT) {
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) v += o_lds[k][idx / D][idx % D];
    part_o[pbase * HG * D + idx] = v;
  }
  if (tid < HG) {
    part_ml[(pbase * HG + tid) * 2 + 0] = mx[tid];
    part_ml[(pbase * HG + tid) * 2 + 1] = sm[tid];
  }
}

// MFMA kernel shape: 4 waves x 4 groups of 16 slots = 256 slots per split.
constexpr int kMfmaNG = 4, kMfmaNW = 4;
static_assert(kMfmaNG * 16 * kMfmaNW == kAttnChunk, "split size");

template <typename T, int D>
static hipError_t attention_valu(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                                 int n_max, int write_logits) {
  constexpr int NT = 256;
  const auto& cf = c->cfg;
  dim3 grid((n_max + kAttnChunk - 1) / kAttnChunk, c->G, cf.n_layers);
  attn_valu_kernel<T, D, 4, NT, kAttnChunk><<<grid, NT, 0, c->stream>>>(
      static_cast<const T*>(q), static_cast<const T*>(k_new), static_cast<const T*>(v_new),
      static_cast<T*>(c->d.kpool), static_cast<T*>(c->d.vpool), c->d.ptab, c->d.count,
      c->d.logits, c->d.part_ml, c->d.part_o, cf.n_layers, c->G, cf.n_kv_heads, cf.n_q_heads, c->P,
      c->maxpages, c->cap, c->max_splits, 1.0f / sqrtf(static_cast<float>(D)), write_logits);
  return hipGetLastError();
}

hipError_t launch_attention(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                            int n_max, int write_logits) {
  const auto& cf = c->cfg;
  const int D = cf.head_dim;
  if (c->HG != 4) return hipErrorInvalidValue;
  if (cf.dtype == KVEV_BF16 && D == 128) {
    dim3 grid((n_max + kAttnChunk - 1) / kAttnChunk, c->G, cf.n_layers);
    attn_mfma_kernel<kMfmaNG, kMfmaNW><<<grid, kMfmaNW * kWave, 0, c->stream>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_new),
        static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(c->d.kpool),
        static_cast<uint16_t*>(c->d.vpool), c->d.ptab, c->d.count, c->d.logits, c->d.part_ml,
        c->d.part_o, cf.n_layers, c->G, cf.n_kv_heads, cf.n_q_heads, c->P, c->maxpages, c->cap,
        c->max_splits, 1.0f / sqrtf(128.0f), write_logits);
    return hipGetLastError();
  }
  if (cf.dtype == KVEV_BF16) return attention_valu<bf16_t, 64>(c, q, k_new, v_new, n_max, write_logits);
  if (D == 128) return attention_valu<float, 128>(c, q, k_new, v_new, n_max, write_logits);
  return attention_valu<float, 64>(c, q, k_new, v_new, n_max, write_logits);
}

}  // namespace kvev
