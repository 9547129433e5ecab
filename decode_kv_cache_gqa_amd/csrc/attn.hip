// Split-K GQA decode attention that exposes per-token logits.
//
// Computes, per (layer l, group g = (sequence, KV head), split of
// kAttnChunk tokens), for the HG query heads sharing the KV head:
//   s[h][t] = (q_h . k_t) / sqrt(d)          ("QEvict" review, section 4.1,
//                                              (Attention))
//   m[h] = max_t s, l[h] = sum_t exp(s - m), o[h][:] = sum_t exp(s - m) v_t
// and stores s (fp32) so the probability pass can normalise it once the
// global (max, sum) of every head is known.  The combine kernel merges the
// splits into the attention output and the global (max, sum).
#include "common.h"
#include "kvev_internal.h"

namespace kvev {

template <typename T, int D, int HG, int NT>
__global__ __launch_bounds__(NT) void attn_split_kernel(
    const T* __restrict__ q, const T* __restrict__ kpool, const T* __restrict__ vpool,
    const int* __restrict__ ptab, const int* __restrict__ count, float* __restrict__ logits,
    float* __restrict__ part_ml, float* __restrict__ part_o, int L, int G, int Hkv, int Hq,
    int64_t P, int maxpages, int64_t cap, int S, float scale, int write_logits) {
  constexpr int EPL = Vec16<T>::N;  // elements per 16-byte lane load
  constexpr int LPT = D / EPL;      // lanes per token row
  constexpr int TPW = kWave / LPT;  // token rows per wave per load
  constexpr int NW = NT / kWave;
  constexpr int CH = kAttnChunk;
  constexpr int U = 4;              // loads in flight per lane
  static_assert(LPT <= kWave && (kWave % LPT) == 0, "row must fit a wave");

  __shared__ float s_lds[CH][HG];
  __shared__ float red[NW][HG];
  __shared__ float o_lds[NW][HG][D];

  const int split = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int n = count[g];
  const int t0 = split * CH;
  if (t0 >= n) return;
  const int cnt = min(n - t0, CH);
  const int B = G / Hkv;
  const int b = g / Hkv, kvh = g % Hkv;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int sub = lane % LPT, tslot = lane / LPT;
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;

  // this lane's slice of the group's query rows
  float qv[HG][EPL];
  {
    const T* qb = q + (static_cast<int64_t>(l * B + b) * Hq + kvh * HG) * D + sub * EPL;
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const uint4 r = *reinterpret_cast<const uint4*>(qb + h * D);
      Vec16<T>::widen(r, qv[h]);
    }
  }

  // ---- logits --------------------------------------------------------------
  for (int base = wave * TPW; base < cnt; base += NW * TPW * U) {
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = base + u * NW * TPW + tslot;
      if (i < cnt) {
        const int t = t0 + i;
        const int64_t row = pool_row(l, pt[t / kPageTokens], 0, t % kPageTokens, P, 1, kPageTokens);
        raw[u] = *reinterpret_cast<const uint4*>(kpool + row * D + sub * EPL);
      } else {
        raw[u] = make_uint4(0, 0, 0, 0);
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

  // ---- chunk max and sum of exp --------------------------------------------
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
      const float p = expf(s_lds[i][h] - mx[h]);
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

  // ---- p . V ------------------------------------------------------------------
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
      if (i < cnt) {
        const int t = t0 + i;
        const int64_t row = pool_row(l, pt[t / kPageTokens], 0, t % kPageTokens, P, 1, kPageTokens);
        raw[u] = *reinterpret_cast<const uint4*>(vpool + row * D + sub * EPL);
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
    const int h = idx / D, c = idx % D;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) v += o_lds[k][h][c];
    part_o[pbase * HG * D + idx] = v;
  }
  if (tid < HG) {
    part_ml[(pbase * HG + tid) * 2 + 0] = mx[tid];
    part_ml[(pbase * HG + tid) * 2 + 1] = sm[tid];
  }
}

// Merge the splits of one (layer, group): out = sum_s e^{m_s-M} o_s / Z with
// M = max_s m_s and Z = sum_s e^{m_s-M} l_s; also store (M, Z) per head.
template <int D, int HG>
__global__ void combine_kernel(const int* __restrict__ count, const float* __restrict__ part_ml,
                               const float* __restrict__ part_o, float* __restrict__ out,
                               float* __restrict__ ml, int G, int Hkv, int Hq, int S) {
  const int g = blockIdx.x, l = blockIdx.y;
  const int n = count[g];
  const int ns = (n + kAttnChunk - 1) / kAttnChunk;
  const int B = G / Hkv, b = g / Hkv, kvh = g % Hkv;
  const int64_t pbase = (static_cast<int64_t>(l) * G + g) * S;
  for (int idx = threadIdx.x; idx < HG * D; idx += blockDim.x) {
    const int h = idx / D, c = idx % D;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, part_ml[((pbase + s) * HG + h) * 2]);
    float Z = 0.f, o = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float w = expf(part_ml[((pbase + s) * HG + h) * 2] - M);
      Z += w * part_ml[((pbase + s) * HG + h) * 2 + 1];
      o += w * part_o[(pbase + s) * HG * D + idx];
    }
    out[(static_cast<int64_t>(l * B + b) * Hq + kvh * HG + h) * D + c] = o / Z;
    if (c == 0) {
      ml[((static_cast<int64_t>(l) * G + g) * HG + h) * 2 + 0] = M;
      ml[((static_cast<int64_t>(l) * G + g) * HG + h) * 2 + 1] = Z;
    }
  }
}

template <typename T, int D, int HG>
static hipError_t attention_impl(kvev_ctx* c, const void* q, int n_max, int write_logits) {
  constexpr int NT = 256;
  const auto& cf = c->cfg;
  const int splits = (n_max + kAttnChunk - 1) / kAttnChunk;
  dim3 grid(splits, c->G, cf.n_layers);
  attn_split_kernel<T, D, HG, NT><<<grid, NT, 0, c->stream>>>(
      static_cast<const T*>(q), static_cast<const T*>(c->d.kpool),
      static_cast<const T*>(c->d.vpool), c->d.ptab, c->d.count, c->d.logits, c->d.part_ml,
      c->d.part_o, cf.n_layers, c->G, cf.n_kv_heads, cf.n_q_heads, c->P, c->maxpages, c->cap,
      c->max_splits, 1.0f / sqrtf(static_cast<float>(D)), write_logits);
  return hipGetLastError();
}

hipError_t launch_attention(kvev_ctx* c, const void* q, int n_max, int write_logits) {
  const int D = c->cfg.head_dim;
  if (c->HG != 4) return hipErrorInvalidValue;
  if (c->cfg.dtype == KVEV_BF16) {
    if (D == 128) return attention_impl<bf16_t, 128, 4>(c, q, n_max, write_logits);
    if (D == 64) return attention_impl<bf16_t, 64, 4>(c, q, n_max, write_logits);
  } else {
    if (D == 128) return attention_impl<float, 128, 4>(c, q, n_max, write_logits);
    if (D == 64) return attention_impl<float, 64, 4>(c, q, n_max, write_logits);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine(kvev_ctx* c, float* out) {
  const auto& cf = c->cfg;
  dim3 grid(c->G, cf.n_layers);
  const int threads = c->HG * cf.head_dim;
  if (c->HG != 4) return hipErrorInvalidValue;
  if (cf.head_dim == 128)
    combine_kernel<128, 4><<<grid, threads, 0, c->stream>>>(c->d.count, c->d.part_ml, c->d.part_o,
                                                            out, c->d.ml, c->G, cf.n_kv_heads,
                                                            cf.n_q_heads, c->max_splits);
  else
    combine_kernel<64, 4><<<grid, threads, 0, c->stream>>>(c->d.count, c->d.part_ml, c->d.part_o,
                                                           out, c->d.ml, c->G, cf.n_kv_heads,
                                                           cf.n_q_heads, c->max_splits);
  return hipGetLastError();
}

}  // namespace kvev
