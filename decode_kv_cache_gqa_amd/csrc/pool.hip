// Post-attention kernel of the sequence-pooled mode (one utility and one
// retained set per sequence).
#include "post_common.h"

namespace kvev {

// ---------------------------------------------------------------------------
// Post-attention kernel of the sequence-pooled mode: one utility per
// (sequence, token), the mean over all Hq query heads of their probability
// on the token ("What Matters ...", section 3.1 Eq.1; appendix E: a KV
// head's attention serves its query group before the pooling).  Every KV
// head group of a sequence holds the same slots; the sequence's first group
// (g0 = b * Hkv) carries the positions and utilities.  Grid (blocks per
// sequence, sequences), kPoolNT threads.  Block c:
//  * when it folds (observation step, slots [16c, 16c + 16) exist), merges
//    the split statistics of every (layer, query head) of the sequence;
//  * output block nblk + o (o < L * Hkv) instead merges the statistics of
//    layer o % L, KV head o / L, writes that output and leaves: the
//    sequence's last block ends with its selection;
//  * folds its slots' pooled mass layer by layer:
//    mass_l[t] = (1/Hq) sum over KV heads of (sum over the group's heads of
//    p), with the scorer variants' factors (VNorm per KV head; entropy: the
//    mean over all Hq heads).  The 64 lanes of a slot each take (layer, KV
//    head) pairs, every logit row of a lane loaded at once; the per-pair
//    masses are summed over KV heads in a fixed order;
//  * publishes its minimum eviction key and utility sum.
// The sequence's last block selects once: one over budget, the minimum of
// the published keys and the new token's, whose slot becomes every KV
// head's free slot (nothing moves); otherwise the radix select plans the
// hole fill in its first group's move lists, and the move kernel copies
// every KV head's rows.  Same hand-off rules as post_kernel.
// ---------------------------------------------------------------------------
constexpr int kPoolNT = 512;
constexpr int kPoolTok = kPoolTokens;             // slots per block
constexpr int kPoolLanes = kPoolNT / kPoolTok;    // lanes per slot
constexpr int kPoolPairs = 8;                     // (layer, KV head) rows per lane and batch (<= 4 heads)
static_assert(kPoolTok <= kWave, "a block's slots fit one wave");

template <typename T, int D, int HG, bool SC>
__global__ __launch_bounds__(kPoolNT) void pool_post_kernel(PostArgs A) {
  constexpr int NT = kPoolNT;
  constexpr int EO = (HG * D + NT - 1) / NT;  // output elements per thread
  constexpr int PP = HG <= 4 ? kPoolPairs : kPoolPairs / 2;  // rows per lane and batch
  extern __shared__ float dyn[];
  const int L = A.L, Hkv = A.Hkv, Hq = A.Hq;
  const int LK = L * Hkv;
  float* s_ml = dyn;                      // [L][Hq][2]
  float* s_w = s_ml + L * Hq * 2;         // [HG][S] split weights of this block's output
  float* s_part = s_w + HG * A.S;         // [L * Hkv][kPoolTok] per (layer, KV head) masses
  float* s_mass = s_part + LK * kPoolTok; // [L][kPoolTok]
  float* s_ent = s_mass + L * kPoolTok;   // [L][Hq] normalised entropies (entropy scorer)
  float* s_lw = s_ent + L * Hq;           // [L] layer factor: 1/Hq, times the entropy mean
  float* s_vw = s_lw + L;                 // [L][Hkv] n / sum of the value norms (VNorm)
  __shared__ float red[NT / kWave];
  __shared__ unsigned long long s_key[NT / kWave];
  __shared__ int s_slot[NT / kWave];
  __shared__ int s_last;
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid % kWave;
  const int g0 = b * Hkv;
  const int n = A.count[g0] + 1;  // slots spanned, the new token's included
  const int hn = A.hole[g0];       // the new token's slot
  const int newest = A.nextpos[g0];
  const int ns = (n + A.CT - 1) / A.CT;
  const int Bsz = A.G / Hkv;
  const int tbase = c * kPoolTok;
  int* gp = A.pos + static_cast<int64_t>(g0) * A.cap;
  float* gs = A.score + static_cast<int64_t>(g0) * A.cap;
  auto is_cand = [&](int p) { return !(p < A.n_sink || p > newest - A.n_recent); };
  const bool ent = SC && A.part_u != nullptr, vn = SC && A.vnorm != nullptr;
  // blocks c >= nblk write outputs only (and take no part in the arrival)
  const bool outb = c >= A.nblk;
  const int oc = c - A.nblk;
  const bool fold = !outb && A.refresh && tbase < n;
  // mass phase: slot ts of the block, lane j of the slot's kPoolLanes
  const int ts = tid % kPoolTok, j = tid / kPoolTok;
  const int t = tbase + ts;

  float prior = 0.f;
  int mypos = 0;
  if (!outb && tid < kPoolTok && t < n && t != hn) {
    prior = gs[t];
    mypos = gp[t];
  }
  // the first batch of this lane's logit rows (pairs j, j + kPoolLanes, ...)
  float x[PP][HG], vx[PP];
  auto load_pairs = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PP; ++u) {
      const int pr = min(j + (k0 + u) * kPoolLanes, LK - 1);
      const int l = pr / Hkv, kv = pr % Hkv;
      const int64_t r = (static_cast<int64_t>(g0 + kv) * L + l) * A.lstride + min(t, n - 1);
      load_heads<HG>(A.logits + r * HG, x[u]);
      vx[u] = vn ? A.vnorm[r] : 1.f;
    }
  };
  if (fold) load_pairs(0);
  // an output block's output: layer oc % L, KV head oc / L
  const int ol = outb ? oc % L : 0, okv = outb ? oc / L : 0;
  float po[EO][kMergeBatch];
  const float* pob = A.part_o + (static_cast<int64_t>(ol) * A.G + g0 + (outb ? okv : 0)) * A.S * HG * D;
  if (outb) {
#pragma unroll
    for (int e = 0; e < EO; ++e) {
      const int idx = tid + e * NT;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) po[e][k] = (idx < HG * D && k < ns) ? pob[k * HG * D + idx] : 0.f;
    }
  }

  // ---- (M, Z) per (layer, query head): every one for a folding block, else
  // only those of the block's output -----------------------------------------------
  const int m0 = outb ? ol * Hq + okv * HG : 0;
  const int m1 = fold ? L * Hq : (outb ? m0 + HG : 0);
  for (int i = m0 + tid; i < m1; i += NT) {
    const int l = i / Hq, hq = i % Hq;
    const int64_t sb = (static_cast<int64_t>(l) * A.G + g0 + hq / HG) * A.S * HG + hq % HG;
    const float2* pb = reinterpret_cast<const float2*>(A.part_ml) + sb;
    float M = -INFINITY, Z = 0.f, U = 0.f;
    for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
      float2 v[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) v[k] = s0 + k < ns ? pb[(s0 + k) * HG] : make_float2(-INFINITY, 0.f);
      float Mb = M;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) Mb = fmaxf(Mb, v[k].x);
      const float f0 = M == -INFINITY ? 0.f : __expf(M - Mb);
      float z = Z * f0;
      if (ent) {
        float u = M == -INFINITY ? 0.f : f0 * (U + (Mb - M) * Z);
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
          if (v[k].x == -INFINITY) continue;
          u += __expf(v[k].x - Mb) * (A.part_u[sb + (s0 + k) * HG] + (Mb - v[k].x) * v[k].y);
        }
        U = u;
      }
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) z += v[k].x == -INFINITY ? 0.f : v[k].y * __expf(v[k].x - Mb);
      M = Mb;
      Z = z;
    }
    s_ml[i * 2 + 0] = M;
    s_ml[i * 2 + 1] = Z;
    if (ent) s_ent[i] = n > 1 ? (__logf(Z) + U / Z) / __logf(static_cast<float>(n)) : 1.f;
  }
  if (vn && fold) {
    for (int i = tid; i < LK; i += NT) {
      const float* pv = A.part_vn + (static_cast<int64_t>(i / Hkv) * A.G + g0 + i % Hkv) * A.S;
      float sum = 0.f;
      for (int s = 0; s < ns; ++s) sum += pv[s];
      s_vw[i] = sum > 0.f ? static_cast<float>(n) / sum : 0.f;
    }
  }
  __syncthreads();

  auto write_output = [&]() __attribute__((always_inline)) {
    if (!outb) return;
    const float2* pml = reinterpret_cast<const float2*>(A.part_ml) + (static_cast<int64_t>(ol) * A.G + g0 + okv) * A.S * HG;
    const float* ml = &s_ml[(ol * Hq + okv * HG) * 2];
    for (int i = tid; i < HG * ns; i += NT) {
      const int h = i / ns, s = i % ns;
      const float ms = pml[s * HG + h].x;
      s_w[h * A.S + s] = ms == -INFINITY ? 0.f : __expf(ms - ml[2 * h]);
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EO; ++e) {
      const int idx = tid + e * NT;
      if (idx >= HG * D) continue;
      const int h = idx / D, cc = idx % D;
      float o = 0.f;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) o += k < ns ? s_w[h * A.S + k] * po[e][k] : 0.f;
      for (int s = kMergeBatch; s < ns; ++s) o += s_w[h * A.S + s] * pob[s * HG * D + idx];
      A.out[(static_cast<int64_t>(ol * Bsz + b) * Hq + okv * HG + h) * D + cc] = o / ml[2 * h + 1];
    }
  };

  // ---- pooled mass per (layer, slot), then the layer-ordered fold ------------
  float myscore = prior;
  if (fold) {
    for (int l = tid; l < L; l += NT) {
      float e = 1.f;
      if (ent) {
        e = 0.f;
        for (int hq = 0; hq < Hq; ++hq) e += s_ent[l * Hq + hq];
        e /= static_cast<float>(Hq);
      }
      s_lw[l] = e / static_cast<float>(Hq);
    }
    for (int k0 = 0; j + k0 * kPoolLanes < LK; k0 += PP) {
      if (k0 > 0) load_pairs(k0);
#pragma unroll
      for (int u = 0; u < PP; ++u) {
        const int pr = j + (k0 + u) * kPoolLanes;
        if (pr >= LK) continue;
        const int l = pr / Hkv, kv = pr % Hkv;
        const float* ml = &s_ml[(l * Hq + kv * HG) * 2];
        float m = 0.f;
#pragma unroll
        for (int h = 0; h < HG; ++h) m += __expf(x[u][h] - ml[2 * h]) / ml[2 * h + 1];
        if (vn) {
          const float w = s_vw[pr];
          m *= w > 0.f ? vx[u] * w : 1.f;
        }
        s_part[pr * kPoolTok + ts] = m;
      }
    }
    __syncthreads();
    for (int i = tid; i < L * kPoolTok; i += NT) {
      const int l = i / kPoolTok, sl = i % kPoolTok;
      float acc = 0.f;
      for (int kv = 0; kv < Hkv; ++kv) acc += s_part[(l * Hkv + kv) * kPoolTok + sl];
      s_mass[i] = acc * s_lw[l];
    }
    __syncthreads();
    if (tid < kPoolTok && t < n) {
      float m = (t == hn) ? 0.f : prior;
      const float keep = 1.0f - A.a;
      for (int l = 0; l < L; ++l) {
        const float mass = s_mass[l * kPoolTok + tid];
        m = A.cumulative ? m + mass : A.a * mass + keep * m;
      }
      st_coherent(gs + t, m);
      myscore = m;
    }
  }

  if (outb) {
    write_output();
    return;
  }

  // ---- block summary over slots other than the new token's (wave 0) ---------------
  if (tid < kWave) {
    const bool mine = tid < kPoolTok && t < n && t != hn;
    unsigned long long key = ~0ull;
    int slot = -1;
    if (mine && is_cand(mypos)) {
      key = (static_cast<unsigned long long>(float_key(myscore)) << 32) | static_cast<uint32_t>(mypos);
      slot = t;
    }
    // (with mean_init on an observation step: the sum of the starting utilities)
    float sum = mine ? ((A.refresh && A.mean_init) ? prior : myscore) : 0.f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long y = __shfl_xor(key, o, kWave);
      const int ys = __shfl_xor(slot, o, kWave);
      if (y < key) {
        key = y;
        slot = ys;
      }
    }
    sum = wave_sum(sum);
    if (tid == 0) {
      const int64_t bi = static_cast<int64_t>(g0) * A.max_blk + c;
      st_coherent(A.blk_key + bi, key);
      st_coherent(A.blk_slot + bi, slot);
      st_coherent(A.blk_sum + bi, sum);
    }
  }

  // ---- arrival ----------------------------------------------------------------------
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(&A.grpctr[g0], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == static_cast<unsigned>(A.nblk - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the sequence's last block ------------------------------------------------
  const bool one_over = A.do_select && n == A.B + 1;
  const float newscore_obs = A.refresh ? ld_state<true>(gs + hn) : 0.f;
  float part = 0.f;
  unsigned long long bkey = ~0ull;
  int bslot = -1;
  for (int i = tid; i < A.nblk; i += NT) {
    const int64_t bi = static_cast<int64_t>(g0) * A.max_blk + i;
    part += ld_state<true>(A.blk_sum + bi);
    const unsigned long long k2 = ld_state<true>(A.blk_key + bi);
    const int s2 = ld_state<true>(A.blk_slot + bi);
    if (k2 < bkey) {
      bkey = k2;
      bslot = s2;
    }
  }
  part = wave_sum(part);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long y = __shfl_xor(bkey, o, kWave);
    const int ys = __shfl_xor(bslot, o, kWave);
    if (y < bkey) {
      bkey = y;
      bslot = ys;
    }
  }
  if (lane == 0) {
    red[tid / kWave] = part;
    s_key[tid / kWave] = bkey;
    s_slot[tid / kWave] = bslot;
  }
  __syncthreads();
  float total = 0.f;
  bkey = s_key[0];
  bslot = s_slot[0];
  for (int w = 0; w < NT / kWave; ++w) {
    total += red[w];
    if (s_key[w] < bkey) {
      bkey = s_key[w];
      bslot = s_slot[w];
    }
  }
  float newscore = newscore_obs;
  if (!A.refresh) {
    newscore = n > 1 ? total / static_cast<float>(n - 1) : 0.f;
    if (tid == 0) st_coherent(gs + hn, newscore);
  } else if (A.mean_init) {
    // the new token's fold from 0 plus its start (the others' mean) times
    // the start's fold weight
    newscore = newscore_obs + A.wprior * (n > 1 ? total / static_cast<float>(n - 1) : 0.f);
    if (tid == 0) st_coherent(gs + hn, newscore);
  }
  if (tid == 0) {
    st_coherent(gp + hn, newest);
    for (int h = 0; h < Hkv; ++h) A.nextpos[g0 + h] = newest + 1;
    A.grpctr[g0] = 0u;
  }
  if (!one_over) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // every slot of [0, n) now holds a token; new_hole is the slot the next
  // token takes in every KV head's pages
  int final_n = n, nm = 0, new_hole = n;
  if (one_over) {
    // one over budget: the evicted slot stays free for the next token
    if (is_cand(newest)) {
      const unsigned long long kn =
          (static_cast<unsigned long long>(float_key(newscore)) << 32) | static_cast<uint32_t>(newest);
      if (kn < bkey) {
        bkey = kn;
        bslot = hn;
      }
    }
    final_n = A.B;
    if (bslot < 0) {
      if (tid == 0) atomicOr(A.errflag, 2);  // no candidate: impossible when B >= |protected|
      new_hole = hn;
    } else {
      new_hole = bslot;
    }
  } else if (A.do_select && n > A.B) {
    int* src = A.mv_src + static_cast<int64_t>(g0) * A.cap;
    int* dst = A.mv_dst + static_cast<int64_t>(g0) * A.cap;
    nm = select_group<NT, true>(n, A.B, newest, A.n_sink, A.n_recent, gp, gs, src, dst, A.errflag,
                                new_hole);
    final_n = A.B;
  }
  if (tid == 0) {
    for (int h = 0; h < Hkv; ++h) {
      A.count[g0 + h] = final_n;
      A.hole[g0 + h] = new_hole;
      A.nmoves[g0 + h] = nm;
    }
  }
}

template <typename T, int D>
hipError_t launch_pool_post(kvev_ctx* c, const PostArgs& A) {
  const auto& cf = c->cfg;
  dim3 grid(A.nblk + cf.n_layers * cf.n_kv_heads, cf.batch);  // slot blocks, then output blocks
  const size_t shm = pool_post_shm(cf.n_layers, cf.n_q_heads, cf.n_kv_heads, A.S) * sizeof(float);
  return with_group(c->HG, [&](auto hg) -> hipError_t {
    constexpr int HG = decltype(hg)::value;
    if (A.part_u || A.vnorm)
      pool_post_kernel<T, D, HG, true><<<grid, kPoolNT, shm, c->stream>>>(A);
    else
      pool_post_kernel<T, D, HG, false><<<grid, kPoolNT, shm, c->stream>>>(A);
    return hipGetLastError();
  });
}

template hipError_t launch_pool_post<bf16_t, 128>(kvev_ctx*, const PostArgs&);
template hipError_t launch_pool_post<bf16_t, 64>(kvev_ctx*, const PostArgs&);
template hipError_t launch_pool_post<float, 128>(kvev_ctx*, const PostArgs&);
template hipError_t launch_pool_post<float, 64>(kvev_ctx*, const PostArgs&);

}  // namespace kvev
