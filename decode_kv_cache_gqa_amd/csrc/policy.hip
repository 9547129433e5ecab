// Probability pass + score fold, top-budget selection with compaction plan,
// K/V moves, and the cache copy kernels.
#include "post_common.h"
#include "host_util.h"

namespace kvev {
// ---------------------------------------------------------------------------
// Post-attention kernel, grid (slot blocks + L output blocks, groups).  Slot
// block c < nblk owns slots [64c, 64c + 64); output block nblk + l writes
// the attention output of layer l, out = sum_s e^{m_s - M} o_s / Z, from its
// own merge of that layer's split statistics, and leaves (it takes no part
// in the arrival, so the group's last block ends with the selection).
// Every slot block:
//  * merges the splits' (max, sum) of all layers of its group (on an
//    observation step);
//  * on an observation step, folds its slots' probability mass layer by
//    layer: mass_l[t] = sum_{h in group} exp(s_l[h][t] - M_l[h]) / Z_l[h],
//    m <- a*mass + (1-a)*m (EMA) or m <- m + mass (cumulative), l = 0..L-1
//    ("What Matters ...", section 3.1 Eq.1 pooled per KV head, Eq.3/Eq.4,
//    appendix E "Layer scoring"); the new token starts at 0.  The scorer
//    variants of section 5.1 scale mass_l[t] by the slot's value norm over
//    the layer's mean norm (VNorm) and by the mean over the group's heads of
//    H_h / ln n, H_h = ln Z + sum_t p (M - s) (entropy weighting);
//  * publishes, for its slots other than the new token's, the minimum
//    eviction key (order-preserving score key, position) over the
//    unprotected slots and the sum of the utilities.
// All loads a block needs are issued before the first use.  The group's
// last block to finish (arrival counter, no waiting) gives the new token the
// mean utility on a non-observation step (appendix E "New token insertion"),
// records its position, commits the count and, when asked, selects: with one
// token over budget the eviction is the minimum of the published keys and
// the new token's key, and the evicted slot becomes the group's free slot,
// which the next token takes (nothing moves); otherwise a full radix select
// plans the hole fill, and the move kernel copies the planned K/V rows.
// Data handed between blocks is written through to device scope and read
// with device-scope loads; no agent-scope fence is used (on this GPU it
// writes back the whole L2).
// ---------------------------------------------------------------------------
template <typename T, int D, int HG, int NT, bool SC>
__global__ __launch_bounds__(NT) void post_kernel(PostArgs A) {
  static_assert(NT % kPostTok == 0 && NT >= 256, "block shape");
  constexpr int LG = NT / kPostTok;  // layer lanes per slot
  constexpr int EO = (HG * D + NT - 1) / NT;  // output elements per thread
  extern __shared__ float dyn[];
  const int L = A.L;
  float* s_ml = dyn;                        // [L][HG][2]
  float* s_w = dyn + L * HG * 2;            // [HG][S] split weights of this block's layer
  float* s_mass = s_w + HG * A.S;           // [L][kPostTok]
  float* s_ent = s_mass + L * kPostTok;     // [L][HG] normalised entropies (entropy scorer)
  float* s_vw = s_ent + L * HG;             // [L] n / sum of the value norms (VNorm scorer)
  __shared__ float red[NT / kWave];
  __shared__ unsigned long long s_key[NT / kWave];
  __shared__ int s_slot[NT / kWave];
  __shared__ int s_last;
  const int c = blockIdx.x, g = blockIdx.y, tid = threadIdx.x, lane = tid % kWave;
  // seq: the whole-cache attention already wrote the outputs and, on an
  // observation step, each slot's group mass per layer (A.logits then holds
  // [G][L][lstride] masses): no statistics to merge and no output blocks
  const bool seq = A.seq != 0;
  const bool outb = !seq && c >= A.nblk;  // an output block, for layer ol
  const int ol = c - A.nblk;
  const int n = A.count[g] + 1;  // slots spanned, the new token's included
  const int hn = A.hole[g];       // the new token's slot
  const int newest = A.nextpos[g];
  const int ns = (n + A.CT - 1) / A.CT;
  const int Bsz = A.G / A.Hkv, b = g / A.Hkv, kvh = g % A.Hkv;
  // slots per slot block: kPostTok on an observation step (the fold stages
  // every layer's mass of its slots in LDS), one per thread otherwise
  const int spb = A.refresh ? kPostTok : NT;
  const int tbase = c * spb;
  int* gp = A.pos + static_cast<int64_t>(g) * A.cap;
  float* gs = A.score + static_cast<int64_t>(g) * A.cap;
  auto is_cand = [&](int p) { return !(p < A.n_sink || p > newest - A.n_recent); };
  // SC: compiled with the scorer variants (active when their inputs are non-null)
  const bool ent = SC && A.part_u != nullptr, vn = SC && A.vnorm != nullptr;

  // ---- issue every load of the block ---------------------------------------
  const int tl = tid % kPostTok, lg = tid / kPostTok;
  const int t = A.refresh ? tbase + tl : tbase + tid;
  const bool holder = A.refresh ? tid < kPostTok : true;  // the thread summarises slot t
  const bool fold = !outb && A.refresh && tbase < n;
  float sx[8][HG];
  float vx[8];
  if (fold) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int l = lg + k * LG;
      const bool in = t < n && l < L;
      const int64_t r = (static_cast<int64_t>(g) * L + (in ? l : 0)) * A.lstride + (in ? t : 0);
      if (seq)
        sx[k][0] = A.logits[r];
      else
        load_heads<HG>(A.logits + r * HG, sx[k]);
      vx[k] = vn ? A.vnorm[r] : 1.f;
    }
  }
  float prior = 0.f;
  int mypos = 0;
  if (!outb && holder && t < n && t != hn) {
    prior = gs[t];
    mypos = gp[t];
  }
  // statistics merged: every layer's for a folding block, its layer's for an
  // output block, none otherwise
  const int m0 = outb ? ol * HG : 0;  // (ol is negative for a slot block)
  const int m1 = (fold && !seq) ? L * HG : (outb ? m0 + HG : 0);
  float2 pm[kMergeBatch];
  const int ml_l = (m0 + tid) / HG, ml_h = (m0 + tid) % HG;
  const float2* pmb = reinterpret_cast<const float2*>(A.part_ml) +
                      (static_cast<int64_t>(ml_l) * A.G + g) * A.S * HG + ml_h;
  if (m0 + tid < m1) {
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) pm[k] = k < ns ? pmb[k * HG] : make_float2(-INFINITY, 0.f);
  }
  float po[EO][kMergeBatch];
  const float* pob = A.part_o + (static_cast<int64_t>(outb ? ol : 0) * A.G + g) * A.S * HG * D;
  if (outb) {
#pragma unroll
    for (int e = 0; e < EO; ++e) {
      const int idx = tid + e * NT;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k)
        po[e][k] = (idx < HG * D && k < ns) ? pob[k * HG * D + idx] : 0.f;
    }
  }

  // ---- merge the split statistics: (M, Z) per (layer, head) ----------------
  for (int i = m0 + tid; i < m1; i += NT) {
    float M = -INFINITY, Z = 0.f, U = 0.f;
    const int64_t sb = (static_cast<int64_t>(i / HG) * A.G + g) * A.S * HG + i % HG;
    for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
      float2 v[kMergeBatch];
      if (i == m0 + tid && s0 == 0) {
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) v[k] = pm[k];
      } else {
        const float2* pb = reinterpret_cast<const float2*>(A.part_ml) + sb;
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) v[k] = s0 + k < ns ? pb[(s0 + k) * HG] : make_float2(-INFINITY, 0.f);
      }
      float Mb = M;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) Mb = fmaxf(Mb, v[k].x);
      const float f0 = M == -INFINITY ? 0.f : __expf(M - Mb);
      float z = Z * f0;
      if (ent) {
        // sum p (Mb - s) over the merged splits: shift the running part to Mb
        float u = M == -INFINITY ? 0.f : f0 * (U + (Mb - M) * Z);
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
          if (v[k].x == -INFINITY) continue;
          const float f = __expf(v[k].x - Mb);
          u += f * (A.part_u[sb + (s0 + k) * HG] + (Mb - v[k].x) * v[k].y);
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
    for (int l = tid; l < L; l += NT) {
      const float* pv = A.part_vn + (static_cast<int64_t>(l) * A.G + g) * A.S;
      float sum = 0.f;
      for (int s = 0; s < ns; ++s) sum += pv[s];
      s_vw[l] = sum > 0.f ? static_cast<float>(n) / sum : 0.f;
    }
  }
  __syncthreads();

  // ---- attention output of layer c (after the block's arrival: the
  // selection does not wait on it) ------------------------------------------------
  auto write_output = [&]() __attribute__((always_inline)) {
    const int l = ol;
    const float2* pml = reinterpret_cast<const float2*>(A.part_ml) + (static_cast<int64_t>(l) * A.G + g) * A.S * HG;
    for (int i = tid; i < HG * ns; i += NT) {
      const int h = i / ns, s = i % ns;
      const float ms = pml[s * HG + h].x;
      s_w[h * A.S + s] = ms == -INFINITY ? 0.f : __expf(ms - s_ml[(l * HG + h) * 2]);
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
      A.out[(static_cast<int64_t>(l * Bsz + b) * A.Hq + kvh * HG + h) * D + cc] = o / s_ml[(l * HG + h) * 2 + 1];
    }
  };

  // ---- probability mass per (layer, slot), then the layer-ordered fold --------
  // mass of one layer's slot: the group's probabilities, times the scorer
  // variants' factors
  auto slot_mass = [&](int l, const float* x, float v) {
    const float* ml = &s_ml[l * HG * 2];
    float m = 0.f;
#pragma unroll
    for (int h = 0; h < HG; ++h) m += __expf(x[h] - ml[2 * h]) / ml[2 * h + 1];
    if (vn) m *= s_vw[l] > 0.f ? v * s_vw[l] : 1.f;
    if (ent) {
      float e = 0.f;
#pragma unroll
      for (int h = 0; h < HG; ++h) e += s_ent[l * HG + h];
      m *= e * (1.0f / HG);
    }
    return m;
  };
  float myscore = prior;
  if (fold) {
    if (t < n) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int l = lg + k * LG;
        if (l >= L) continue;
        s_mass[l * kPostTok + tl] = seq ? sx[k][0] : slot_mass(l, sx[k], vx[k]);
      }
      for (int l = lg + 8 * LG; l < L; l += LG) {  // more than 8 * LG layers
        const int64_t r = (static_cast<int64_t>(g) * L + l) * A.lstride + t;
        if (seq) {
          s_mass[l * kPostTok + tl] = A.logits[r];
          continue;
        }
        float x[HG];
        load_heads<HG>(A.logits + r * HG, x);
        s_mass[l * kPostTok + tl] = slot_mass(l, x, vn ? A.vnorm[r] : 1.f);
      }
    }
    __syncthreads();
    if (tid < kPostTok && t < n) {
      float m = (t == hn) ? 0.f : prior;
      float raw = 0.f;
      const float keep = 1.0f - A.a;
      for (int l = 0; l < L; ++l) {
        const float mass = s_mass[l * kPostTok + tl];
        raw += mass;
        m = A.cumulative ? m + mass : A.a * mass + keep * m;
      }
      st_coherent(gs + t, m);
      myscore = m;
      if (A.dg_raw) {  // rank-trace diagnostics: the step's inputs per slot
        const int64_t r = static_cast<int64_t>(g) * A.cap + t;
        A.dg_pos[r] = t == hn ? newest : mypos;
        A.dg_raw[r] = raw;
        A.dg_util[r] = m;
        if (t == 0) A.dg_n[g] = n;
      }
    }
  }

  if (outb) {
    write_output();
    return;
  }

  // ---- block summary over slots other than the new token's -------------------
  unsigned long long skey = ~0ull;
  int sslot = -1;
  float ssum = 0.f;
  if (holder) {
    const bool mine = t < n && t != hn;
    unsigned long long key = ~0ull;
    int slot = -1;
    if (mine && is_cand(mypos)) {
      key = (static_cast<unsigned long long>(float_key(myscore)) << 32) | static_cast<uint32_t>(mypos);
      slot = t;
    }
    // the sum of the utilities (with mean_init on an observation step: of
    // the starting utilities, whose mean the new token starts at)
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
    skey = key;
    sslot = slot;
    ssum = sum;
  }
  if (!A.refresh) {  // the block's slots span every wave: combine them
    if (lane == 0) {
      s_key[tid / kWave] = skey;
      s_slot[tid / kWave] = sslot;
      red[tid / kWave] = ssum;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 1; w < NT / kWave; ++w) {
        ssum += red[w];
        if (s_key[w] < skey) {
          skey = s_key[w];
          sslot = s_slot[w];
        }
      }
    }
  }
  if (tid == 0) {
    const int64_t bi = static_cast<int64_t>(g) * A.max_blk + c;
    st_coherent(A.blk_key + bi, skey);
    st_coherent(A.blk_slot + bi, sslot);
    st_coherent(A.blk_sum + bi, ssum);
  }

  // ---- arrival ----------------------------------------------------------------------
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(&A.grpctr[g], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == static_cast<unsigned>(A.nblk - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the group's last block ------------------------------------------------
  // It loads the block summaries and the new token's utility (observation
  // step) in one batch.
  const bool one_over = A.do_select && n == A.B + 1;
  const float newscore_obs = A.refresh ? ld_state<true>(gs + hn) : 0.f;
  float part = 0.f;
  unsigned long long bkey = ~0ull;
  int bslot = -1;
  for (int i = tid; i < A.nblk; i += NT) {
    const int64_t bi = static_cast<int64_t>(g) * A.max_blk + i;
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
    // the fold is linear in the start: the new token's fold from 0 plus
    // the start (the others' mean) times its fold weight
    newscore = newscore_obs + A.wprior * (n > 1 ? total / static_cast<float>(n - 1) : 0.f);
    if (tid == 0) {
      st_coherent(gs + hn, newscore);
      if (A.dg_util) A.dg_util[static_cast<int64_t>(g) * A.cap + hn] = newscore;
    }
  }
  if (tid == 0) {
    st_coherent(gp + hn, newest);
    A.nextpos[g] = newest + 1;
    A.grpctr[g] = 0u;
  }
  if (!one_over) {
    // the full selection below reads the new token's state back
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // every slot of [0, n) now holds a token; new_hole is the slot the next
  // token takes
  int final_n = n, nm = 0, new_hole = n;
  if (one_over) {
    // one over budget: evict the smallest key, the new token included; the
    // evicted slot stays free for the next token, so nothing moves
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
    int* src = A.mv_src + static_cast<int64_t>(g) * A.cap;
    int* dst = A.mv_dst + static_cast<int64_t>(g) * A.cap;
    nm = select_group<NT, true>(n, A.B, newest, A.n_sink, A.n_recent, gp, gs, src, dst, A.errflag,
                                new_hole);
    final_n = A.B;
  }
  if (tid == 0) {
    A.count[g] = final_n;
    A.hole[g] = new_hole;
    A.nmoves[g] = nm;
  }
}

// ---------------------------------------------------------------------------
// Fold + selection after the whole-cache attention (which wrote the
// outputs and, on an observation step, every slot's group mass per layer
// into gmass [G][L][lstride]).  Slot blocks of 256 per group in a 1-D grid,
// group fastest; one slot per thread.  Each thread's loads do not wait for
// the group's count (slots past it are masked afterwards): the slot's
// utility and position and, on
// an observation step, its masses of every layer, folded in ascending layer
// order ("What Matters ...", section 3.1 Eq.3/Eq.4, appendix E "Layer
// scoring"; the new token starts at 0).  Each block publishes the minimum
// eviction key (order-preserving utility key, position) of its unprotected
// slots, its slot and the utility sum (the new token excluded), and the
// block holding the new token its folded utility; the group's last block
// to arrive (no waiting) gives the new token its state (on a step without
// an observation the mean of the others, appendix E "New token insertion")
// and selects as post_kernel's last block does.  Data handed between blocks
// is written through to device scope and read with device-scope loads.
// ---------------------------------------------------------------------------
constexpr int kFoldNT = 256;
constexpr int kFoldLayers = 64;  // the library's layer bound

struct FoldArgs {
  int* count;
  int* hole;
  int* pos;
  float* score;
  int* nextpos;
  const float* gmass;
  unsigned* grpctr;
  unsigned long long* blk_key;
  int* blk_slot;
  float* blk_sum;
  float* gnew;  // [G] the new token's folded utility (observation steps)
  int* mv_src;
  int* mv_dst;
  int* nmoves;
  int* errflag;
  int* dg_n;  // rank-trace diagnostics, or null
  int* dg_pos;
  float* dg_raw;
  float* dg_util;
  int L, max_blk, nblk, G;
  int64_t cap, lstride;
  float a;
  int cumulative, refresh, do_select, B, n_sink, n_recent;
  int mean_init;  // as in PostArgs
  float wprior;
  // per-sequence granularity: G counts sequences, each of pool_hkv KV head
  // groups whose state lives in its first group; a slot's layer
  // observation is the sum of the groups' masses times inv_hq (the mean
  // over every query head)
  int pool_hkv;
  float inv_hq;
};

template <int NL, bool POOL>
__global__ __launch_bounds__(kFoldNT) void fold_kernel(FoldArgs A) {
  constexpr int NT = kFoldNT, NWV = NT / kWave;
  __shared__ float red[NWV], s_new[NWV];
  __shared__ unsigned long long s_key[NWV];
  __shared__ int s_slot[NWV];
  __shared__ int s_last;
  // a 1-D grid, group fastest: workgroups go to the eight XCDs round-robin,
  // so group g's blocks share an XCD (and its L2) with the attention
  // workgroups of group g, which wrote the masses (grid (groups, layers))
  const int gi = blockIdx.x % A.G, blk = blockIdx.x / A.G, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int nhg = POOL ? A.pool_hkv : 1;  // the KV head groups that share the state
  const int g = gi * nhg;                 // the group holding the state
  const int t = blk * NT + tid;
  const bool valid = t < A.cap;
  int* gp = A.pos + static_cast<int64_t>(g) * A.cap;
  float* gs = A.score + static_cast<int64_t>(g) * A.cap;
  // loads that do not depend on the count
  const float prior = valid ? gs[t] : 0.f;
  const int mypos = valid ? gp[t] : 0;
  float x[NL];
  if (A.refresh) {
    const float* gm = A.gmass + static_cast<int64_t>(g) * A.L * A.lstride + (t < A.lstride ? t : 0);
#pragma unroll
    for (int l = 0; l < NL; ++l) x[l] = l < A.L ? gm[static_cast<int64_t>(l) * A.lstride] : 0.f;
    if constexpr (POOL) {
      // the other groups' masses, added in group order, then the mean over
      // every query head
      for (int h = 1; h < nhg; ++h) {
        const float* gh = gm + static_cast<int64_t>(h) * A.L * A.lstride;
        float y[NL];
#pragma unroll
        for (int l = 0; l < NL; ++l) y[l] = l < A.L ? gh[static_cast<int64_t>(l) * A.lstride] : 0.f;
#pragma unroll
        for (int l = 0; l < NL; ++l) x[l] += y[l];
      }
#pragma unroll
      for (int l = 0; l < NL; ++l) x[l] *= A.inv_hq;
    }
  }
  const int n = A.count[g] + 1, hn = A.hole[g], newest = A.nextpos[g];
  auto is_cand = [&](int p) { return !(p < A.n_sink || p > newest - A.n_recent); };
  const bool in = t < n;
  float m = (in && t != hn) ? prior : 0.f;
  if (A.refresh && in) {
    float raw = 0.f;
    const float keep = 1.0f - A.a;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      if (l < A.L) {
        raw += x[l];
        m = A.cumulative ? m + x[l] : A.a * x[l] + keep * m;
      }
    }
    st_coherent(gs + t, m);  // the selection of a larger eviction reads it back
    if (A.dg_raw) {  // rank-trace diagnostics: the step's inputs per slot
      const int64_t r = static_cast<int64_t>(g) * A.cap + t;
      A.dg_pos[r] = t == hn ? newest : mypos;
      A.dg_raw[r] = raw;
      A.dg_util[r] = m;
      if (t == 0) A.dg_n[g] = n;
    }
  }
  // block summary over slots other than the new token's
  const bool mine = in && t != hn;
  unsigned long long key = ~0ull;
  int slot = -1;
  if (mine && is_cand(mypos)) {
    key = (static_cast<unsigned long long>(float_key(m)) << 32) | static_cast<uint32_t>(mypos);
    slot = t;
  }
  // (with mean_init on an observation step: the sum of the starting utilities)
  float sum = mine ? ((A.refresh && A.mean_init) ? prior : m) : 0.f;
  float mn = (A.refresh && in && t == hn) ? m : 0.f;
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
  mn = wave_sum(mn);
  if (lane == 0) {
    s_key[wave] = key;
    s_slot[wave] = slot;
    red[wave] = sum;
    s_new[wave] = mn;
  }
  // a selection of more than one token reads every slot's utility back in
  // the group's last block: then each thread's utility store completes
  // before the block arrives (with one token over budget only the summaries
  // cross blocks, and thread 0 waits for those)
  if (A.do_select && n > A.B + 1) __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < NWV; ++w) {
      sum += red[w];
      mn += s_new[w];
      if (s_key[w] < key) {
        key = s_key[w];
        slot = s_slot[w];
      }
    }
    const int64_t bi = static_cast<int64_t>(g) * A.max_blk + blk;
    st_coherent(A.blk_key + bi, key);
    st_coherent(A.blk_slot + bi, slot);
    st_coherent(A.blk_sum + bi, sum);
    if (A.refresh && hn / NT == blk) st_coherent(A.gnew + g, mn);
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned old = __hip_atomic_fetch_add(&A.grpctr[g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old == static_cast<unsigned>(A.nblk - 1) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the group's last block ------------------------------------------------
  float part = 0.f;
  unsigned long long bkey = ~0ull;
  int bslot = -1;
  for (int i = tid; i < A.nblk; i += NT) {
    const int64_t bi = static_cast<int64_t>(g) * A.max_blk + i;
    part += ld_state<true>(A.blk_sum + bi);
    const unsigned long long k2 = ld_state<true>(A.blk_key + bi);
    const int s2 = ld_state<true>(A.blk_slot + bi);
    if (k2 < bkey) {
      bkey = k2;
      bslot = s2;
    }
  }
  const float newscore_obs = A.refresh ? ld_state<true>(A.gnew + g) : 0.f;
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
  __syncthreads();
  if (lane == 0) {
    red[wave] = part;
    s_key[wave] = bkey;
    s_slot[wave] = bslot;
  }
  __syncthreads();
  float total = 0.f;
  bkey = s_key[0];
  bslot = s_slot[0];
  for (int w = 0; w < NWV; ++w) {
    total += red[w];
    if (s_key[w] < bkey) {
      bkey = s_key[w];
      bslot = s_slot[w];
    }
  }
  const float mean = n > 1 ? total / static_cast<float>(n - 1) : 0.f;
  // mean_init: the new token's fold from 0 plus its start times the start's fold weight
  const float newscore = A.refresh ? newscore_obs + (A.mean_init ? A.wprior * mean : 0.f) : mean;
  // the group's state is written through to memory (about 0.2 us shorter
  // launches than with plain stores on the 32k workload)
  if (tid == 0) {
    if (!A.refresh || A.mean_init) st_coherent(gs + hn, newscore);
    if (A.refresh && A.mean_init && A.dg_util) A.dg_util[static_cast<int64_t>(g) * A.cap + hn] = newscore;
    st_coherent(gp + hn, newest);
    for (int h = 0; h < nhg; ++h) st_coherent(A.nextpos + g + h, newest + 1);
    st_coherent(A.grpctr + g, 0u);
  }
  const bool one_over = A.do_select && n == A.B + 1;
  int final_n = n, nm = 0, new_hole = n;
  if (one_over) {
    // one over budget: evict the smallest key, the new token included; the
    // evicted slot stays free for the next token, so nothing moves
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
    // the selection reads every slot's state back, the new token's included
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int* src = A.mv_src + static_cast<int64_t>(g) * A.cap;
    int* dst = A.mv_dst + static_cast<int64_t>(g) * A.cap;
    nm = select_group<NT, true>(n, A.B, newest, A.n_sink, A.n_recent, gp, gs, src, dst, A.errflag, new_hole);
    final_n = A.B;
  }
  if (tid == 0) {
    for (int h = 0; h < nhg; ++h) {  // every KV head group follows the state's plan
      st_coherent(A.count + g + h, final_n);
      st_coherent(A.hole + g + h, new_hole);
      st_coherent(A.nmoves + g + h, nm);
    }
  }
}

hipError_t launch_fold(kvev_ctx* c, int n_max, int refresh, int do_select, int64_t budget) {
  const auto& cf = c->cfg;
  FoldArgs A;
  A.count = c->d.count;
  A.hole = c->d.hole;
  A.pos = c->d.pos;
  A.score = c->d.score;
  A.nextpos = c->d.nextpos;
  A.gmass = c->d.logits;
  A.grpctr = c->d.grpctr;
  A.blk_key = c->d.blk_key;
  A.blk_slot = c->d.blk_slot;
  A.blk_sum = c->d.blk_sum;
  A.gnew = c->d.gnew;
  A.mv_src = c->d.mv_src;
  A.mv_dst = c->d.mv_dst;
  A.nmoves = c->d.nmoves;
  A.errflag = c->d.errflag;
  const bool dg = refresh && c->d.dg_raw != nullptr;
  A.dg_n = dg ? c->d.dg_n : nullptr;
  A.dg_pos = dg ? c->d.dg_pos : nullptr;
  A.dg_raw = dg ? c->d.dg_raw : nullptr;
  A.dg_util = dg ? c->d.dg_util : nullptr;
  A.L = cf.n_layers;
  A.max_blk = c->max_post_blocks;
  A.nblk = (n_max + kFoldNT - 1) / kFoldNT;
  A.G = c->pooled ? cf.batch : c->G;
  A.pool_hkv = c->pooled ? cf.n_kv_heads : 1;
  A.inv_hq = 1.0f / static_cast<float>(cf.n_q_heads);
  A.cap = c->cap;
  A.lstride = c->lstride;
  A.a = cf.alpha_new;
  A.cumulative = cf.policy == KVEV_CUMULATIVE;
  A.refresh = refresh;
  A.do_select = do_select;
  A.B = static_cast<int>(budget);
  A.n_sink = cf.n_sink;
  A.n_recent = cf.n_recent;
  A.mean_init = cf.new_token_init == KVEV_NEW_TOKEN_MEAN;
  A.wprior = prior_fold_weight(cf.alpha_new, cf.n_layers, A.cumulative != 0);
  dim3 grid(A.nblk * A.G);
  if (c->pooled)
    return cf.n_layers <= 32 ? timed_launch(c, "post", fold_kernel<32, true>, grid, dim3(kFoldNT), 0, A)
                             : timed_launch(c, "post", fold_kernel<kFoldLayers, true>, grid, dim3(kFoldNT), 0, A);
  if (cf.n_layers <= 32) return timed_launch(c, "post", fold_kernel<32, false>, grid, dim3(kFoldNT), 0, A);
  return timed_launch(c, "post", fold_kernel<kFoldLayers, false>, grid, dim3(kFoldNT), 0, A);
}

// Standalone selection (kvev_evict): one block per group, or, in the
// sequence-pooled mode (pool = Hkv > 0), one block per sequence working on
// its first group's state, whose plan every KV head's moves then follow.
constexpr int kSelNT = 1024;
__global__ __launch_bounds__(kSelNT) void select_kernel(
    int* __restrict__ count, int* __restrict__ hole, int* __restrict__ pos, float* __restrict__ score,
    const int* __restrict__ nextpos, int* __restrict__ mv_src, int* __restrict__ mv_dst,
    int* __restrict__ nmoves, int* __restrict__ errflag, int64_t cap, int B, int n_sink,
    int n_recent, int pool) {
  const int g = pool ? blockIdx.x * pool : blockIdx.x;
  const int ng = pool ? pool : 1;
  const int n = count[g];
  if (n <= B) {
    if (threadIdx.x == 0)
      for (int h = 0; h < ng; ++h) nmoves[g + h] = 0;
    return;
  }
  int new_hole = B;
  const int nm = select_group<kSelNT, false>(n, B, nextpos[g] - 1, n_sink, n_recent,
                                      pos + static_cast<int64_t>(g) * cap,
                                      score + static_cast<int64_t>(g) * cap,
                                      mv_src + static_cast<int64_t>(g) * cap,
                                      mv_dst + static_cast<int64_t>(g) * cap, errflag, new_hole);
  if (threadIdx.x == 0) {
    for (int h = 0; h < ng; ++h) {
      nmoves[g + h] = nm;
      count[g + h] = B;
      hole[g + h] = new_hole;
    }
  }
}

// Before a standalone selection: a group whose free slot lies inside its
// cache (count tokens spread over slots [0, count] after a single-token
// eviction) gets its last token (slot count) planned into the free slot, so
// that the selection sees its tokens in slots [0, count).  One thread per
// group; in the sequence-pooled mode (pool = Hkv) the state and the plan are
// the sequence's first group's, and every group of the sequence follows it.
__global__ void close_hole_kernel(const int* __restrict__ count, int* __restrict__ hole,
                                  int* __restrict__ pos, float* __restrict__ score,
                                  int* __restrict__ mv_src, int* __restrict__ mv_dst,
                                  int* __restrict__ nmoves, int64_t cap, int G, int B, int pool) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= G) return;
  const int n = count[g], h = hole[g];
  int nm = 0;
  if (n > B && h < n) {
    const int gc = pool ? g / pool * pool : g;
    if (g == gc) {
      const int64_t o = static_cast<int64_t>(gc) * cap;
      pos[o + h] = pos[o + n];
      score[o + h] = score[o + n];
      mv_src[o] = n;
      mv_dst[o] = h;
    }
    hole[g] = n;
    nm = 1;
  }
  nmoves[g] = nm;
}

// K/V moves of the compaction plan: block (chunk of moves, group, layer).
template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void move_kernel(T* __restrict__ kpool, T* __restrict__ vpool,
                                                  const int* __restrict__ ptab,
                                                  const int* __restrict__ mv_src,
                                                  const int* __restrict__ mv_dst,
                                                  const int* __restrict__ nmoves, int64_t P,
                                                  int maxpages, int64_t cap, int per_block, int pool) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  const int g = blockIdx.y, l = blockIdx.z;
  const int gm = pool ? g / pool * pool : g;  // the group whose plan applies (pooled: the sequence's first)
  const int nm = nmoves[g];
  const int j0 = blockIdx.x * per_block;
  const int j1 = min(nm, j0 + per_block);
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
  const int* ms = mv_src + static_cast<int64_t>(gm) * cap;
  const int* md = mv_dst + static_cast<int64_t>(gm) * cap;
  for (int idx = threadIdx.x; idx < (j1 - j0) * LPR; idx += NT) {
    const int j = j0 + idx / LPR, sub = idx % LPR;
    const int s = ms[j], d = md[j];
    if (s < 0 || s >= cap || d < 0 || d >= cap) continue;
    *reinterpret_cast<uint4*>(kpool + kidx(l, pt[d / kPageTokens], d % kPageTokens, sub * EPL, P, D)) =
        *reinterpret_cast<const uint4*>(kpool + kidx(l, pt[s / kPageTokens], s % kPageTokens, sub * EPL, P, D));
  }
  for (int idx = threadIdx.x; idx < (j1 - j0) * D; idx += NT) {
    const int j = j0 + idx / D, c = idx % D;
    const int s = ms[j], d = md[j];
    if (s < 0 || s >= cap || d < 0 || d >= cap) continue;
    vpool[vidx(l, pt[d / kPageTokens], d % kPageTokens, c, P, D)] =
        vpool[vidx(l, pt[s / kPageTokens], s % kPageTokens, c, P, D)];
  }
}

// Prefill: copy k, v [L][Hkv][n][D] of one sequence into its groups' pages
// (table entries e0, e0 + 1, ...), one page (16 tokens) per block; V goes
// through LDS to be stored channel-major.  Rows of the last page beyond n
// are zero-filled.
template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void scatter_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                     T* __restrict__ kpool, T* __restrict__ vpool,
                                                     const int* __restrict__ ptab, int seq, int Hkv,
                                                     int64_t n, int64_t P, int maxpages, int e0) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  __shared__ T tile[kPageTokens][D + EPL];
  const int pg = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int g = seq * Hkv + h;
  const int page = ptab[static_cast<int64_t>(g) * maxpages + e0 + pg];
  const int64_t tb = static_cast<int64_t>(pg) * kPageTokens;
  for (int idx = threadIdx.x; idx < kPageTokens * LPR; idx += NT) {
    const int r = idx / LPR, sub = idx % LPR;
    const int64_t t = tb + r;
    uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
    if (t < n) {
      const int64_t src = ((static_cast<int64_t>(l) * Hkv + h) * n + t) * D + sub * EPL;
      kv = *reinterpret_cast<const uint4*>(k + src);
      vv = *reinterpret_cast<const uint4*>(v + src);
    }
    *reinterpret_cast<uint4*>(kpool + kidx(l, page, r, sub * EPL, P, D)) = kv;
    *reinterpret_cast<uint4*>(&tile[r][sub * EPL]) = vv;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < D * kPageTokens; idx += NT) {
    const int c = idx / kPageTokens, r = idx % kPageTokens;
    vpool[vidx(l, page, r, c, P, D)] = tile[r][c];
  }
}

// Gather (dir 0) or scatter (dir 1) one group's slots against dense [L][n][D].
template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void group_copy_kernel(T* __restrict__ kd, T* __restrict__ vd,
                                                        T* __restrict__ kpool, T* __restrict__ vpool,
                                                        const int* __restrict__ ptab, int g,
                                                        int64_t n, int64_t ld, int64_t P,
                                                        int maxpages, int dir, int64_t skip) {
  const int l = blockIdx.y;
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x; idx < n * D;
       idx += static_cast<int64_t>(gridDim.x) * NT) {
    const int64_t i = idx / D;             // dense row
    const int64_t t = i + (i >= skip);     // its slot (the free slot is skipped)
    const int c = static_cast<int>(idx % D);
    const int page = pt[t / kPageTokens], r = static_cast<int>(t % kPageTokens);
    const int64_t dense = (static_cast<int64_t>(l) * ld + i) * D + c;
    if (dir == 0) {
      kd[dense] = kpool[kidx(l, page, r, c, P, D)];
      vd[dense] = vpool[vidx(l, page, r, c, P, D)];
    } else {
      kpool[kidx(l, page, r, c, P, D)] = kd[dense];
      vpool[vidx(l, page, r, c, P, D)] = vd[dense];
    }
  }
}

// Page-table updates passed by value: (flat index into ptab, page) pairs.
constexpr int kMaxPageUpd = 128;
struct PageUpd {
  int n;
  int idx[kMaxPageUpd];
  int page[kMaxPageUpd];
};
__global__ void set_pages_kernel(int* __restrict__ ptab, PageUpd u) {
  const int i = threadIdx.x;
  if (i < u.n) ptab[u.idx[i]] = u.page[i];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_set_pages(kvev_ctx* c, const int* upd, int n_upd) {
  for (int off = 0; off < n_upd; off += kMaxPageUpd) {
    PageUpd u;
    u.n = n_upd - off < kMaxPageUpd ? n_upd - off : kMaxPageUpd;
    for (int i = 0; i < u.n; ++i) {
      u.idx[i] = upd[2 * (off + i)];
      u.page[i] = upd[2 * (off + i) + 1];
    }
    set_pages_kernel<<<1, kMaxPageUpd, 0, c->stream>>>(c->d.ptab, u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D>
static hipError_t post_impl(kvev_ctx* c, float* out, const void* k_new, const void* v_new, int n_max,
                            int refresh, int do_select, int64_t budget, int seq) {
  constexpr int NT = 256;
  const auto& cf = c->cfg;
  PostArgs A;
  A.count = c->d.count;
  A.hole = c->d.hole;
  A.pos = c->d.pos;
  A.score = c->d.score;
  A.nextpos = c->d.nextpos;
  A.logits = c->d.logits;
  A.part_ml = c->d.part_ml;
  A.part_o = c->d.part_o;
  A.part_u = refresh ? c->d.part_u : nullptr;
  A.vnorm = refresh ? c->d.vnorm : nullptr;
  A.part_vn = refresh ? c->d.part_vn : nullptr;
  A.out = out;
  A.grpctr = c->d.grpctr;
  A.blk_key = c->d.blk_key;
  A.blk_slot = c->d.blk_slot;
  A.blk_sum = c->d.blk_sum;
  A.max_blk = c->max_post_blocks;
  A.k_new = k_new;
  A.v_new = v_new;
  A.mv_src = c->d.mv_src;
  A.mv_dst = c->d.mv_dst;
  A.nmoves = c->d.nmoves;
  A.errflag = c->d.errflag;
  // the diagnostics' inputs (recorded on observation steps)
  const bool dg = refresh && c->d.dg_raw != nullptr;
  A.dg_n = dg ? c->d.dg_n : nullptr;
  A.dg_pos = dg ? c->d.dg_pos : nullptr;
  A.dg_raw = dg ? c->d.dg_raw : nullptr;
  A.dg_util = dg ? c->d.dg_util : nullptr;
  A.kpool = c->d.kpool;
  A.vpool = c->d.vpool;
  A.ptab = c->d.ptab;
  A.L = cf.n_layers;
  A.G = c->G;
  A.Hkv = cf.n_kv_heads;
  A.Hq = cf.n_q_heads;
  A.S = (n_max + kAttnChunk - 1) / kAttnChunk;
  A.lstride = c->lstride;
  A.CT = kAttnChunk;
  A.maxpages = c->maxpages;
  A.cap = c->cap;
  A.P = c->P;
  A.a = cf.alpha_new;
  A.cumulative = cf.policy == KVEV_CUMULATIVE;
  A.refresh = refresh;
  A.do_select = do_select;
  A.seq = 0;
  A.mean_init = cf.new_token_init == KVEV_NEW_TOKEN_MEAN;
  A.wprior = prior_fold_weight(cf.alpha_new, cf.n_layers, A.cumulative != 0);
  A.B = static_cast<int>(budget);
  A.n_sink = cf.n_sink;
  A.n_recent = cf.n_recent;
  const int spb = refresh ? kPostTok : NT;  // slots per slot block (see post_kernel)
  const int tok_blocks = (n_max + spb - 1) / spb;
  if (c->pooled) {
    // one grid row per sequence: the slot blocks, then one block per (layer, KV head) output
    A.nblk = (n_max + kPoolTokens - 1) / kPoolTokens;
    ProfScope p(c, "post");
    return launch_pool_post<T, D>(c, A);
  }
  A.nblk = tok_blocks;  // slot blocks; the L output blocks follow them (split attention)
  A.seq = seq;
  dim3 grid(A.nblk + (seq ? 0 : cf.n_layers), c->G);
  const size_t shm = (static_cast<size_t>(cf.n_layers) * c->HG * 3 + static_cast<size_t>(c->HG) * A.S +
                      static_cast<size_t>(cf.n_layers) * (kPostTok + 1)) * sizeof(float);
  return with_group(c->HG, [&](auto hg) -> hipError_t {
    constexpr int HG = decltype(hg)::value;
    if (A.part_u || A.vnorm) return timed_launch(c, "post", post_kernel<T, D, HG, NT, true>, grid, dim3(NT), shm, A);
    return timed_launch(c, "post", post_kernel<T, D, HG, NT, false>, grid, dim3(NT), shm, A);
  });
}

hipError_t launch_post(kvev_ctx* c, float* out, const void* k_new, const void* v_new, int n_max,
                       int refresh, int do_select, int64_t budget, int seq) {
  const int D = c->cfg.head_dim;
  if (c->cfg.dtype == KVEV_BF16)
    return D == 128 ? post_impl<bf16_t, 128>(c, out, k_new, v_new, n_max, refresh, do_select, budget, seq)
                    : post_impl<bf16_t, 64>(c, out, k_new, v_new, n_max, refresh, do_select, budget, seq);
  return D == 128 ? post_impl<float, 128>(c, out, k_new, v_new, n_max, refresh, do_select, budget, seq)
                  : post_impl<float, 64>(c, out, k_new, v_new, n_max, refresh, do_select, budget, seq);
}

hipError_t launch_close_holes(kvev_ctx* c, int64_t budget) {
  constexpr int NT = 256;
  close_hole_kernel<<<(c->G + NT - 1) / NT, NT, 0, c->stream>>>(
      c->d.count, c->d.hole, c->d.pos, c->d.score, c->d.mv_src, c->d.mv_dst, c->d.nmoves, c->cap, c->G,
      static_cast<int>(budget), c->pooled ? c->cfg.n_kv_heads : 0);
  return hipGetLastError();
}

hipError_t launch_select(kvev_ctx* c, int64_t budget) {
  const auto& cf = c->cfg;
  const int pool = c->pooled ? cf.n_kv_heads : 0;
  select_kernel<<<pool ? cf.batch : c->G, kSelNT, 0, c->stream>>>(
      c->d.count, c->d.hole, c->d.pos, c->d.score, c->d.nextpos, c->d.mv_src, c->d.mv_dst,
      c->d.nmoves, c->d.errflag, c->cap, static_cast<int>(budget), cf.n_sink, cf.n_recent, pool);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t moves_impl(kvev_ctx* c, int max_moves) {
  constexpr int NT = 256, PER = 16;
  dim3 grid((max_moves + PER - 1) / PER, c->G, c->cfg.n_layers);
  move_kernel<T, D, NT><<<grid, NT, 0, c->stream>>>(
      static_cast<T*>(c->d.kpool), static_cast<T*>(c->d.vpool), c->d.ptab, c->d.mv_src,
      c->d.mv_dst, c->d.nmoves, c->P, c->maxpages, c->cap, PER, c->pooled ? c->cfg.n_kv_heads : 0);
  return hipGetLastError();
}

hipError_t launch_moves(kvev_ctx* c, int max_moves) {
  const int D = c->cfg.head_dim;
  if (c->cfg.dtype == KVEV_BF16) return D == 128 ? moves_impl<bf16_t, 128>(c, max_moves)
                                                 : moves_impl<bf16_t, 64>(c, max_moves);
  return D == 128 ? moves_impl<float, 128>(c, max_moves) : moves_impl<float, 64>(c, max_moves);
}

template <typename T, int D>
static hipError_t scatter_impl(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n, int e0) {
  constexpr int NT = 256;
  const int64_t npages = (n + kPageTokens - 1) / kPageTokens;
  if (e0 < 0 || e0 + npages > c->maxpages) return hipErrorInvalidValue;
  dim3 grid(static_cast<unsigned>(npages), c->cfg.n_kv_heads, c->cfg.n_layers);
  scatter_kernel<T, D, NT><<<grid, NT, 0, c->stream>>>(
      static_cast<const T*>(k), static_cast<const T*>(v), static_cast<T*>(c->d.kpool),
      static_cast<T*>(c->d.vpool), c->d.ptab, seq, c->cfg.n_kv_heads, n, c->P, c->maxpages, e0);
  return hipGetLastError();
}

hipError_t launch_scatter_at(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n, int e0) {
  const int D = c->cfg.head_dim;
  if (c->cfg.dtype == KVEV_BF16) return D == 128 ? scatter_impl<bf16_t, 128>(c, seq, k, v, n, e0)
                                                 : scatter_impl<bf16_t, 64>(c, seq, k, v, n, e0);
  return D == 128 ? scatter_impl<float, 128>(c, seq, k, v, n, e0)
                  : scatter_impl<float, 64>(c, seq, k, v, n, e0);
}

hipError_t launch_prefill_scatter(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n) {
  return launch_scatter_at(c, seq, k, v, n, 0);
}

template <typename T, int D>
static hipError_t group_copy_impl(kvev_ctx* c, int g, void* k, void* v, int64_t n, int64_t ld,
                                  int dir, int64_t skip) {
  constexpr int NT = 256;
  int64_t bx = (n * D + NT - 1) / NT;
  if (bx < 1) return hipSuccess;
  if (bx > 4096) bx = 4096;
  dim3 grid(static_cast<unsigned>(bx), c->cfg.n_layers);
  group_copy_kernel<T, D, NT><<<grid, NT, 0, c->stream>>>(
      static_cast<T*>(k), static_cast<T*>(v), static_cast<T*>(c->d.kpool),
      static_cast<T*>(c->d.vpool), c->d.ptab, g, n, ld, c->P, c->maxpages, dir, skip);
  return hipGetLastError();
}

static hipError_t group_copy(kvev_ctx* c, int g, void* k, void* v, int64_t n, int64_t ld, int dir,
                             int64_t skip) {
  const int D = c->cfg.head_dim;
  if (c->cfg.dtype == KVEV_BF16)
    return D == 128 ? group_copy_impl<bf16_t, 128>(c, g, k, v, n, ld, dir, skip)
                    : group_copy_impl<bf16_t, 64>(c, g, k, v, n, ld, dir, skip);
  return D == 128 ? group_copy_impl<float, 128>(c, g, k, v, n, ld, dir, skip)
                  : group_copy_impl<float, 64>(c, g, k, v, n, ld, dir, skip);
}

hipError_t launch_export(kvev_ctx* c, int g, void* k_out, void* v_out, int64_t n, int64_t cap,
                         int64_t skip) {
  return group_copy(c, g, k_out, v_out, n, cap, 0, skip);
}

hipError_t launch_import(kvev_ctx* c, int g, const void* k, const void* v, int64_t n) {
  return group_copy(c, g, const_cast<void*>(k), const_cast<void*>(v), n, n, 1, n);
}

}  // namespace kvev
