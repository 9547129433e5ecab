// Split-K GQA decode attention that exposes per-token logits, with the
// step's new token appended on the way.
//
// Per (layer l, group g = (sequence, KV head), split of slots) and for the
// HG query heads that share the KV head:
//   s[h][t] = (q_h . k_t) / sqrt(d)          ("QEvict" review, section 4.1,
//                                              (Attention))
//   m[h] = max_t s, l[h] = sum_t exp(s - m), o[h][:] = sum_t exp(s - m) v_t
// The logits are stored (fp32) for the probability pass, which normalises
// them once every split's (m, l) is merged; the post kernel does the merge.
// The group's cache holds count[g] tokens in slots [0, count] minus one free
// slot, hole[g] (count[g] itself unless the last eviction removed a single
// token and left its slot free); the new token takes the free slot: it is
// read from k_new / v_new and written into its page by the lanes that hold
// it.  Without a hole array (block mode) the free slot is count[g].
#include "common.h"
#include "kvev_internal.h"
#include "host_util.h"

namespace kvev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& r) {
  bf16x8 v;
  __builtin_memcpy(&v, &r, sizeof(v));
  return v;
}

// replace 16-bit element e (0..7) of a 16-byte register
__device__ __forceinline__ void put16(uint4& r, int e, uint32_t x) {
  const int sh = (e & 1) * 16;
  const uint32_t m = ~(0xffffu << sh);
  const uint32_t v = (x & 0xffffu) << sh;
  switch (e >> 1) {
    case 0: r.x = (r.x & m) | v; break;
    case 1: r.y = (r.y & m) | v; break;
    case 2: r.z = (r.z & m) | v; break;
    default: r.w = (r.w & m) | v; break;
  }
}

// ---------------------------------------------------------------------------
// bf16, head_dim 128, group of HG <= 8 query heads: q.K^T and p.V on the
// matrix cores (v_mfma_f32_16x16x32_bf16), 64 slots (4 pages) per wave.
//   q.K^T: A = the HG query rows (rows HG..15 zero), B = K^T; lane (r16, q4)
//     loads slot r16 of a page, channels 32*s + 8*q4 .. +8 (k-step s); the
//     lanes of quarter q4 receive rows 4*q4 .. 4*q4+3, i.e. the logits of
//     heads 4*q4 + i for slot r16.
//   p.V:   A = P (HG rows), B = V; 32 slots (2 pages) per k-step.  Lane
//     (r16, q4) loads channel 16*ct + r16, slots 8*(q4 & 1) .. +8 of page
//     2k + (q4 >> 1): 16 contiguous bytes of the channel-major V page.  P is
//     split into bf16 hi + lo parts (two products), so the rounding of P is
//     at most 2^-18 relative.
// Every load of the wave is issued before the first use.
// Optional outputs for the scorer variants ("What Matters ...", section 5.1
// and appendix E):
//   part_u  [L][G][S][HG]: sum over the split's slots of e^{s - m}(m - s),
//           m the split maximum (the entropy of a head's distribution is
//           ln Z + (sum p (M - s)), assembled from these after the merge);
//   vnorm   [G][L][lstride]: the l2 norm of every slot's value row, and
//   part_vn [L][G][S]: its sum over the split's slots.
// ---------------------------------------------------------------------------
template <int NW, int HG, bool SC>
__global__ __launch_bounds__(NW * kWave) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
    const int* __restrict__ ptab, const int* __restrict__ count, const int* __restrict__ hole,
    float* __restrict__ logits, float* __restrict__ part_ml, float* __restrict__ part_o,
    float* __restrict__ part_u, float* __restrict__ vnorm, float* __restrict__ part_vn, int L, int G,
    int Hkv, int Hq, int64_t P, int maxpages, int64_t lstride, int S, float scale, int write_logits,
    float* __restrict__ bpart) {
  static_assert(HG >= 1 && HG <= 8, "group size");
  constexpr int D = 128, NG = 4, WT = NG * 16;
  // bpart (16-token block mode): instead of per-slot logits, the sum over
  // each 16-slot block of exp(s - M_split) per head, [L][G][maxpages][HG]
  __shared__ float bsum[NW][NG][HG];
  __shared__ __align__(16) float p_lds[NW][HG][WT];
  __shared__ __align__(16) float wstat[NW][HG][2];
  __shared__ float wstat_u[SC ? NW : 1][HG];
  __shared__ float wvn[NW];
  __shared__ __align__(16) float o_lds[NW][HG][D];

  const int split = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: keep it scalar
  const int r16 = lane & 15, q4 = lane >> 4;
  const int h0 = 4 * q4;  // first head of this lane's output rows
  const int t0 = split * NW * WT, wt0 = t0 + wave * WT;
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
  // page indices do not depend on the count: load them alongside it
  int pages[NG];
#pragma unroll
  for (int j = 0; j < NG; ++j) pages[j] = pt[min((wt0 + 16 * j) / kPageTokens, maxpages - 1)];
  const int n = count[g] + 1;  // slots including the new token
  const int tnew = hole ? hole[g] : n - 1;
  if (t0 >= n) return;
  const int B = G / Hkv, b = g / Hkv, kvh = g % Hkv;
  const int64_t new_off = (static_cast<int64_t>(l * B + b) * Hkv + kvh) * D;
  // SC: compiled with the scorer variants' outputs (present when non-null)
  const bool ent = SC && part_u != nullptr, vn = SC && vnorm != nullptr;

  bf16x8 qa[4];
  {
    const uint16_t* qp = q + (static_cast<int64_t>(l * B + b) * Hq + kvh * HG + min(r16, HG - 1)) * D + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 r = *reinterpret_cast<const uint4*>(qp + 32 * s);
      if (r16 >= HG) r = make_uint4(0, 0, 0, 0);
      qa[s] = as_bf16x8(r);
    }
  }

  // the new token's rows, loaded first by the wave whose slots hold it (the
  // free slot may lie in any split, where this latency would otherwise
  // extend the block)
  const bool app = tnew >= wt0 && tnew < wt0 + WT;  // wave-uniform
  uint4 knew[4];
  uint32_t vnew[8];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    knew[s] = app ? *reinterpret_cast<const uint4*>(k_new + new_off + 32 * s + 8 * q4) : make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vnew[ct] = app ? v_new[new_off + 16 * ct + r16] : 0u;

  uint4 kr[NG][4];
  uint4 vr[2][8];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const bool live = wt0 + 16 * j < n;  // wave-uniform
    const uint16_t* kb = kpool + kidx(l, pages[j], r16, 8 * q4, P, D);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kr[j][s] = live ? *reinterpret_cast<const uint4*>(kb + 32 * s) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const bool second = (q4 >> 1) != 0;
    const bool live = wt0 + 16 * (2 * k + (second ? 1 : 0)) < n;
    const uint16_t* vb = vpool + vidx(l, second ? pages[2 * k + 1] : pages[2 * k], 8 * (q4 & 1), r16, P, D);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      vr[k][ct] = live ? *reinterpret_cast<const uint4*>(vb + ct * 16 * kPageTokens) : make_uint4(0, 0, 0, 0);
  }

  // append: the new token replaces the stale slot contents in registers
  // and is written into its page
  if (app) {
    const int jn = (tnew - wt0) >> 4, rn = (tnew - wt0) & 15;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      if (j != jn || r16 != rn) continue;
      uint16_t* kd = kpool + kidx(l, pages[j], rn, 8 * q4, P, D);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        kr[j][s] = knew[s];
        *reinterpret_cast<uint4*>(kd + 32 * s) = knew[s];
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k != (jn >> 1) || (q4 >> 1) != (jn & 1) || (q4 & 1) != (rn >> 3)) continue;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const uint16_t x = static_cast<uint16_t>(vnew[ct]);
        put16(vr[k][ct], rn & 7, x);
        vpool[vidx(l, pages[jn], rn, 16 * ct + r16, P, D)] = x;
      }
    }
  }

  // l2 norms of the value rows (VNorm scorer): lane (r16, q4) holds 8 slots
  // of 8 channels per k-step; the row sums over r16 give each slot's norm
  float vnsum = 0.f;
  if (vn) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float ss[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ss[e] = 0.f;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const uint32_t w[4] = {vr[k][ct].x, vr[k][ct].y, vr[k][ct].z, vr[k][ct].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
          ss[e] += x * x;
        }
      }
      float mine = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = row16_sum(ss[e]);
        mine = r16 == e ? t : mine;
      }
      const int tk = wt0 + 16 * (2 * k + (q4 >> 1)) + 8 * (q4 & 1) + r16;
      if (r16 < 8 && tk < n) {
        const float nv = sqrtf(mine);
        vnorm[(static_cast<int64_t>(g) * L + l) * lstride + tk] = nv;
        vnsum += nv;
      }
    }
    vnsum = wave_sum(vnsum);
    if (lane == 0) wvn[wave] = vnsum;
  }

  // q.K^T: sv[j][i] is the logit of head h0 + i for slot 16 j + r16
  float sv[NG][4];
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], as_bf16x8(kr[j][s]), acc, 0, 0, 0);
    const int tk = wt0 + 16 * j + r16;
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[j][i] = (h0 + i < HG && tk < n) ? acc[i] * scale : -INFINITY;
    if (h0 < HG && tk < n && write_logits) {
      float* dst = logits + ((static_cast<int64_t>(g) * L + l) * lstride + tk) * HG + h0;
      if constexpr (HG % 4 == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(sv[j][0], sv[j][1], sv[j][2], sv[j][3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (h0 + i < HG) dst[i] = sv[j][i];
      }
    }
  }

  // per-head max and sum over the wave's slots (a head's logits sit in the
  // 16 lanes of one quarter)
  float mh[4], lh[4], uh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = sv[0][i];
#pragma unroll
    for (int j = 1; j < NG; ++j) m = fmaxf(m, sv[j][i]);
    mh[i] = row16_max(m);
    float sum = 0.f, u = 0.f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float p = mh[i] == -INFINITY ? 0.f : __expf(sv[j][i] - mh[i]);
      if (ent) u += p > 0.f ? p * (mh[i] - sv[j][i]) : 0.f;  // masked slots: p = 0
      sv[j][i] = p;
      sum += p;
    }
    lh[i] = row16_sum(sum);
    uh[i] = ent ? row16_sum(u) : 0.f;
  }
  if (bpart) {  // per-block sums relative to the wave's maximum (uniform branch)
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bs = row16_sum(sv[j][i]);
        if (r16 == 0 && h0 + i < HG) bsum[wave][j][h0 + i] = bs;
      }
  }
  if (h0 < HG) {
#pragma unroll
    for (int j = 0; j < NG; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (h0 + i < HG) p_lds[wave][h0 + i][16 * j + r16] = sv[j][i];
    if (r16 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (h0 + i >= HG) continue;
        wstat[wave][h0 + i][0] = mh[i];
        wstat[wave][h0 + i][1] = lh[i];
        if (ent) wstat_u[wave][h0 + i] = uh[i];
      }
    }
  }
  __syncthreads();

  // p.V
  f32x4 oacc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float* prow = &p_lds[wave][min(r16, HG - 1)][32 * k + 8 * q4];
    const float4 a = *reinterpret_cast<const float4*>(prow);
    const float4 c = *reinterpret_cast<const float4*>(prow + 4);
    const float pv[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    uint32_t h16[8], l16[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = r16 < HG ? pv[e] : 0.f;
      h16[e] = bf16_rne(x);
      l16[e] = bf16_rne(x - __uint_as_float(h16[e] << 16));
    }
    const bf16x8 phi = as_bf16x8(make_uint4(h16[0] | (h16[1] << 16), h16[2] | (h16[3] << 16),
                                            h16[4] | (h16[5] << 16), h16[6] | (h16[7] << 16)));
    const bf16x8 plo = as_bf16x8(make_uint4(l16[0] | (l16[1] << 16), l16[2] | (l16[3] << 16),
                                            l16[4] | (l16[5] << 16), l16[6] | (l16[7] << 16)));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const bf16x8 vb = as_bf16x8(vr[k][ct]);
      oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, vb, oacc[ct], 0, 0, 0);
      oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, vb, oacc[ct], 0, 0, 0);
    }
  }
  if (h0 < HG) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (h0 + i < HG) o_lds[wave][h0 + i][16 * ct + r16] = oacc[ct][i];
  }
  __syncthreads();

  // merge the block's waves into one partial
  const int64_t pbase = (static_cast<int64_t>(l) * G + g) * S + split;
  for (int idx = tid; idx < HG * D; idx += NW * kWave) {
    const int h = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wstat[w][h][0]);
    float o = 0.f, Z = 0.f, U = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = wstat[w][h][0];
      const float f = mw == -INFINITY ? 0.f : __expf(mw - M);
      o += f * o_lds[w][h][c];
      Z += f * wstat[w][h][1];
      // sum p (M - s) = sum_w f (u_w + (M - m_w) l_w)
      if (ent && mw != -INFINITY) U += f * (wstat_u[w][h] + (M - mw) * wstat[w][h][1]);
    }
    part_o[pbase * HG * D + idx] = o;
    if (c == 0) {
      part_ml[(pbase * HG + h) * 2 + 0] = M;
      part_ml[(pbase * HG + h) * 2 + 1] = Z;
      if (ent) part_u[pbase * HG + h] = U;
    }
  }
  if (vn && tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += wvn[w];
    part_vn[pbase] = t;
  }
  if (bpart) {  // rescale each block's sum to the split's maximum
    for (int idx = tid; idx < NW * NG * HG; idx += NW * kWave) {
      const int w = idx / (NG * HG), j = (idx / HG) % NG, h = idx % HG;
      float M = -INFINITY;
#pragma unroll
      for (int x = 0; x < NW; ++x) M = fmaxf(M, wstat[x][h][0]);
      const float mw = wstat[w][h][0];
      const int e = split * (NW * NG) + w * NG + j;  // the block's table entry
      if (16 * e < n)
        bpart[((static_cast<int64_t>(l) * G + g) * maxpages + e) * HG + h] =
            mw == -INFINITY ? 0.f : __expf(mw - M) * bsum[w][j][h];
    }
  }
}

// ---------------------------------------------------------------------------
// Generic VALU version (fp32 or bf16, head_dim 64 or 128): lanes split each
// K row into 16-byte pieces and reduce the dot products with cross-lane
// adds; p.V reads the channel-major V pages element-wise.  Used for the
// fp32 cache and for head_dim 64.
// ---------------------------------------------------------------------------
template <typename T, int D, int HG, int NT, int CT, bool SC>
__global__ __launch_bounds__(NT) void attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k_new, const T* __restrict__ v_new,
    T* __restrict__ kpool, T* __restrict__ vpool, const int* __restrict__ ptab,
    const int* __restrict__ count, const int* __restrict__ hole, float* __restrict__ logits,
    float* __restrict__ part_ml, float* __restrict__ part_o, float* __restrict__ part_u,
    float* __restrict__ vnorm,
    float* __restrict__ part_vn, int L, int G, int Hkv, int Hq, int64_t P, int maxpages,
    int64_t lstride, int S, float scale, int write_logits) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPT = D / EPL;
  constexpr int TPW = kWave / LPT;
  constexpr int NW = NT / kWave;
  constexpr int U = 4;
  static_assert(LPT <= kWave && (kWave % LPT) == 0, "row must fit a wave");

  __shared__ float s_lds[CT][HG];
  __shared__ float red[NW][HG];
  __shared__ float red_u[NW][HG];
  __shared__ float red_vn[NW];
  __shared__ float o_lds[NW][HG][D];
  const bool ent = SC && part_u != nullptr, vn = SC && vnorm != nullptr;

  const int split = blockIdx.x, g = blockIdx.y, l = blockIdx.z;
  const int n = count[g] + 1;
  const int t0 = split * CT;
  if (t0 >= n) return;
  const int cnt = min(n - t0, CT);
  const int B = G / Hkv, b = g / Hkv, kvh = g % Hkv;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int sub = lane % LPT, tslot = lane / LPT;
  const int tnew = hole ? hole[g] : n - 1;
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
  const int64_t new_off = (static_cast<int64_t>(l * B + b) * Hkv + kvh) * D + sub * EPL;

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
        T* row = kpool + kidx(l, pt[t / kPageTokens], t % kPageTokens, sub * EPL, P, D);
        if (t == tnew) {
          raw[u] = *reinterpret_cast<const uint4*>(k_new + new_off);
          *reinterpret_cast<uint4*>(row) = raw[u];
        } else {
          raw[u] = *reinterpret_cast<const uint4*>(row);
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
        float* dst = logits + ((static_cast<int64_t>(g) * L + l) * lstride + t0 + i) * HG;
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
  float uu[HG];
#pragma unroll
  for (int h = 0; h < HG; ++h) uu[h] = 0.f;
  for (int i = tid; i < cnt; i += NT)
#pragma unroll
    for (int h = 0; h < HG; ++h) {
      const float s = s_lds[i][h];
      const float p = __expf(s - mx[h]);
      s_lds[i][h] = p;
      sm[h] += p;
      if (ent) uu[h] += p * (mx[h] - s);
    }
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    const float w = wave_sum(sm[h]);
    if (lane == 0) red[wave][h] = w;
    if (ent) {
      const float u = wave_sum(uu[h]);
      if (lane == 0) red_u[wave][h] = u;
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < HG; ++h) {
    float w = 0.f, u = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      w += red[k][h];
      if (ent) u += red_u[k][h];
    }
    sm[h] = w;
    uu[h] = u;
  }

  float acc[HG][EPL];
#pragma unroll
  for (int h = 0; h < HG; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  float vnsum = 0.f;
  for (int base = wave * TPW; base < cnt; base += NW * TPW) {
    const int i = base + tslot;
    float ss = 0.f;
    if (i < cnt) {
      const int t = t0 + i;
      const int page = pt[t / kPageTokens], r = t % kPageTokens;
      uint4 raw;
      T* vv = reinterpret_cast<T*>(&raw);
      if (t == tnew) {
        raw = *reinterpret_cast<const uint4*>(v_new + new_off);
#pragma unroll
        for (int e = 0; e < EPL; ++e) vpool[vidx(l, page, r, sub * EPL + e, P, D)] = vv[e];
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vv[e] = vpool[vidx(l, page, r, sub * EPL + e, P, D)];
      }
      float vf[EPL];
      Vec16<T>::widen(raw, vf);
#pragma unroll
      for (int h = 0; h < HG; ++h) {
        const float p = s_lds[i][h];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] += p * vf[e];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) ss += vf[e] * vf[e];
    }
    if (vn) {  // the row's squared norm over its LPT lanes (wave-uniform loop)
#pragma unroll
      for (int o = LPT / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, kWave);
      if (i < cnt && sub == 0) {
        const float nv = sqrtf(ss);
        vnorm[(static_cast<int64_t>(g) * L + l) * lstride + t0 + i] = nv;
        vnsum += nv;
      }
    }
  }
  if (vn) {
    vnsum = wave_sum(vnsum);
    if (lane == 0) red_vn[wave] = vnsum;
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
    if (ent) part_u[pbase * HG + tid] = uu[tid];
  }
  if (vn && tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) t += red_vn[k];
    part_vn[pbase] = t;
  }
}

// MFMA kernel shape: 4 waves x 64 slots = 256 slots per split.
constexpr int kMfmaNW = 4;
static_assert(kMfmaNW * 64 == kAttnChunk, "split size");

template <typename T, int D, int HG>
static hipError_t attention_valu(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                                 int n_max, int write_logits) {
  constexpr int NT = 256;
  const auto& cf = c->cfg;
  const int splits = (n_max + kAttnChunk - 1) / kAttnChunk;
  dim3 grid(splits, c->G, cf.n_layers);
  // the scorer variants' outputs are needed only with the logits
  float* pu = write_logits ? c->d.part_u : nullptr;
  float* vn = write_logits ? c->d.vnorm : nullptr;
  float* pvn = write_logits ? c->d.part_vn : nullptr;
  auto launch = [&](auto kern) {
    kern<<<grid, NT, 0, c->stream>>>(
        static_cast<const T*>(q), static_cast<const T*>(k_new), static_cast<const T*>(v_new),
        static_cast<T*>(c->d.kpool), static_cast<T*>(c->d.vpool), c->d.ptab, c->d.count, c->d.hole,
        c->d.logits, c->d.part_ml, c->d.part_o, pu, vn, pvn, cf.n_layers, c->G, cf.n_kv_heads,
        cf.n_q_heads, c->P, c->maxpages, c->lstride, splits, 1.0f / sqrtf(static_cast<float>(D)),
        write_logits);
  };
  if (pu || vn)
    launch(attn_valu_kernel<T, D, HG, NT, kAttnChunk, true>);
  else
    launch(attn_valu_kernel<T, D, HG, NT, kAttnChunk, false>);
  return hipGetLastError();
}

hipError_t launch_attention(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                            int n_max, int write_logits, const char* prof) {
  const auto& cf = c->cfg;
  const int D = cf.head_dim;
  return with_group(c->HG, [&](auto hg) -> hipError_t {
    constexpr int HG = decltype(hg)::value;
    if (cf.dtype == KVEV_BF16 && D == 128) {
      const int splits = (n_max + kAttnChunk - 1) / kAttnChunk;
      dim3 grid(splits, c->G, cf.n_layers);
      float* pu = write_logits ? c->d.part_u : nullptr;
      float* vn = write_logits ? c->d.vnorm : nullptr;
      float* pvn = write_logits ? c->d.part_vn : nullptr;
      float* bp = write_logits ? c->d.bpart : nullptr;  // block mode: block sums instead of logits
      auto launch = [&](auto kern) {
        return timed_launch(
            c, prof, kern, grid, dim3(kMfmaNW * kWave), 0, static_cast<const uint16_t*>(q),
            static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
            static_cast<uint16_t*>(c->d.kpool), static_cast<uint16_t*>(c->d.vpool),
            static_cast<const int*>(c->d.ptab), static_cast<const int*>(c->d.count),
            static_cast<const int*>(c->d.hole), c->d.logits, c->d.part_ml, c->d.part_o, pu, vn, pvn,
            static_cast<int>(cf.n_layers), c->G, static_cast<int>(cf.n_kv_heads),
            static_cast<int>(cf.n_q_heads), c->P, c->maxpages, c->lstride, splits, 1.0f / sqrtf(128.0f),
            bp ? 0 : write_logits, bp);
      };
      if (pu || vn) return launch(attn_mfma_kernel<kMfmaNW, HG, true>);
      return launch(attn_mfma_kernel<kMfmaNW, HG, false>);
    }
    ProfScope p(c, prof);  // the vector path is timed by events around it
    if (cf.dtype == KVEV_BF16) return attention_valu<bf16_t, 64, HG>(c, q, k_new, v_new, n_max, write_logits);
    if (D == 128) return attention_valu<float, 128, HG>(c, q, k_new, v_new, n_max, write_logits);
    return attention_valu<float, 64, HG>(c, q, k_new, v_new, n_max, write_logits);
  });
}

}  // namespace kvev
