// Probability pass + score fold, top-budget selection with compaction plan,
// K/V moves, and the cache copy kernels.
#include "common.h"
#include "kvev_internal.h"

namespace kvev {

// ---------------------------------------------------------------------------
// Selection + compaction plan for one group, executed by one block of NT
// threads.  Keep the protected tokens (positions < n_sink, or among the
// n_recent newest) and evict the k = n - B lowest (score, position) keys of
// the rest, i.e. keep the top (B - |protected|) ("What Matters ...", section
// 3.1: evict the lowest utility when over budget; "MemDecay", section III-A
// (1): forcing F then taking the best B is optimal).  The k-th smallest key
// comes from an LDS radix select on order-preserving 32-bit score keys (four
// 8-bit digits), plus a radix select on positions only when equal scores
// straddle the cut; k == 1 is an argmin.  Plan: holes = unkept slots < B
// ascending, movers = kept slots >= B ascending, mover j fills hole j.
// Positions and utilities are moved here; returns the number of moves.
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ void scan_256(const int* hist, int* excl_out, int* wsum, int tid) {
  const int v = tid < 256 ? hist[tid] : 0;
  int x = v;
  const int lane = tid % kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (tid < 256 && lane == kWave - 1) wsum[tid / kWave] = x;
  __syncthreads();
  if (tid < 256) {
    int off = 0;
    for (int w = 0; w < tid / kWave; ++w) off += wsum[w];
    excl_out[tid] = off + x - v;
  }
  __syncthreads();
}

// Loads of slot state.  COH: the values may have been written by other
// blocks of the same kernel with write-through (device-scope) stores, so
// read them with device-scope loads that bypass the CU and L2 copies.
template <bool COH, typename T>
__device__ __forceinline__ T ld_state(const T* p) {
  if constexpr (COH)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}
template <typename T>
__device__ __forceinline__ void st_coherent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NT, bool COH>
__device__ int select_group(int n, int B, int newest, int n_sink, int n_recent,
                            int* __restrict__ gp, float* __restrict__ gs, int* __restrict__ src,
                            int* __restrict__ dst, int* __restrict__ errflag) {
  static_assert(NT >= 256, "selection needs >= 256 threads");
  __shared__ int hist[256];
  __shared__ int excl[256];
  __shared__ int wsum[4];
  __shared__ int sel[3];
  __shared__ unsigned long long wmin[NT / kWave];
  __shared__ int wcnt[2][NT / kWave];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int k = n - B;
  auto is_cand = [&](int p) { return !(p < n_sink || p > newest - n_recent); };

  uint32_t thr = 0;
  int pos_cut = 0x7fffffff;
  if (k == 1) {
    // argmin of (score key, position) over candidates, carrying the slot
    unsigned long long best = ~0ull;
    int slot = -1;
    for (int base = 0; base < n; base += NT * 8) {
      int pv[8];
      float sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NT + tid;
        pv[u] = i < n ? ld_state<COH>(gp + i) : -1;
        sv[u] = i < n ? ld_state<COH>(gs + i) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NT + tid;
        if (i >= n || !is_cand(pv[u])) continue;
        const unsigned long long kk =
            (static_cast<unsigned long long>(float_key(sv[u])) << 32) | static_cast<uint32_t>(pv[u]);
        if (kk < best) {
          best = kk;
          slot = i;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long y = __shfl_xor(best, o, kWave);
      const int ys = __shfl_xor(slot, o, kWave);
      if (y < best) {
        best = y;
        slot = ys;
      }
    }
    if (lane == 0) {
      wmin[wave] = best;
      wcnt[0][wave] = slot;
    }
    __syncthreads();
    best = wmin[0];
    int ev = wcnt[0][0];
    for (int w = 1; w < NT / kWave; ++w)
      if (wmin[w] < best) {
        best = wmin[w];
        ev = wcnt[0][w];
      }
    __syncthreads();
    if (best == ~0ull || ev < 0) {  // no candidate: impossible when B >= |protected|
      if (tid == 0) atomicOr(errflag, 2);
      return 0;
    }
    if (ev >= B) return 0;  // the evicted token sits at slot B: nothing moves
    if (tid == 0) {
      src[0] = B;
      dst[0] = ev;
      gp[ev] = ld_state<COH>(gp + B);
      gs[ev] = ld_state<COH>(gs + B);
    }
    __syncthreads();
    return 1;
  }

  {
    uint32_t prefix = 0, mask = 0;
    int kk = k, eq = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += NT) {
        if (!is_cand(ld_state<COH>(gp + i))) continue;
        const uint32_t key = float_key(ld_state<COH>(gs + i));
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      scan_256<NT>(hist, excl, wsum, tid);
      if (tid < 256 && excl[tid] < kk && kk <= excl[tid] + hist[tid]) {
        sel[0] = tid;
        sel[1] = excl[tid];
        sel[2] = hist[tid];
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(sel[0]) << shift;
      mask |= 255u << shift;
      kk -= sel[1];
      eq = sel[2];
      __syncthreads();
    }
    thr = prefix;
    if (kk < eq) {
      uint32_t pprefix = 0, pmask = 0;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += NT) {
          const int p = ld_state<COH>(gp + i);
          if (!is_cand(p) || float_key(ld_state<COH>(gs + i)) != thr) continue;
          const uint32_t key = static_cast<uint32_t>(p);
          if ((key & pmask) == pprefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        scan_256<NT>(hist, excl, wsum, tid);
        if (tid < 256 && excl[tid] < kk && kk <= excl[tid] + hist[tid]) {
          sel[0] = tid;
          sel[1] = excl[tid];
        }
        __syncthreads();
        pprefix |= static_cast<uint32_t>(sel[0]) << shift;
        pmask |= 255u << shift;
        kk -= sel[1];
        __syncthreads();
      }
      pos_cut = static_cast<int>(pprefix);
    }
  }

  auto keep = [&](int i) {
    const int p = ld_state<COH>(gp + i);
    if (!is_cand(p)) return true;
    const uint32_t key = float_key(ld_state<COH>(gs + i));
    return key > thr || (key == thr && p > pos_cut);
  };
  int hole_base = 0, mover_base = 0;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int tile = 0; tile < n; tile += NT) {
    const int i = tile + tid;
    const bool in = i < n;
    const bool kp = in && keep(i);
    const bool hole = in && i < B && !kp;
    const bool mover = in && i >= B && kp;
    const unsigned long long bh = __ballot(hole), bm = __ballot(mover);
    if (lane == 0) {
      wcnt[0][wave] = __popcll(bh);
      wcnt[1][wave] = __popcll(bm);
    }
    __syncthreads();
    int oh = hole_base, om = mover_base, th = 0, tm = 0;
    for (int w = 0; w < NT / kWave; ++w) {
      if (w < wave) {
        oh += wcnt[0][w];
        om += wcnt[1][w];
      }
      th += wcnt[0][w];
      tm += wcnt[1][w];
    }
    if (hole) dst[oh + __popcll(bh & lt)] = i;
    if (mover) src[om + __popcll(bm & lt)] = i;
    hole_base += th;
    mover_base += tm;
    __syncthreads();
  }
  // the two counts agree by construction; a disagreement is reported, never used
  const int nm = hole_base < mover_base ? hole_base : mover_base;
  if (tid == 0 && hole_base != mover_base) atomicOr(errflag, 1);
  __syncthreads();
  for (int j = tid; j < nm; j += NT) {
    const int s = src[j], d = dst[j];
    gp[d] = ld_state<COH>(gp + s);
    gs[d] = ld_state<COH>(gs + s);
  }
  __syncthreads();
  return nm;
}

// Copy `nm` planned moves of one group for every layer (K and V rows).
template <typename T, int D, int NT>
__device__ void copy_moves(T* __restrict__ kpool, T* __restrict__ vpool, const int* __restrict__ pt,
                           const int* __restrict__ src, const int* __restrict__ dst, int nm, int L,
                           int64_t P, int64_t cap) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  const int total = nm * L * LPR;
  for (int idx = threadIdx.x; idx < total; idx += NT) {
    const int sub = idx % LPR, rest = idx / LPR;
    const int l = rest % L, j = rest / L;
    const int s = src[j], d = dst[j];
    if (s < 0 || s >= cap || d < 0 || d >= cap) continue;
    const int64_t rs = pool_row(l, pt[s / kPageTokens], 0, s % kPageTokens, P, 1, kPageTokens) * D + sub * EPL;
    const int64_t rd = pool_row(l, pt[d / kPageTokens], 0, d % kPageTokens, P, 1, kPageTokens) * D + sub * EPL;
    *reinterpret_cast<uint4*>(kpool + rd) = *reinterpret_cast<const uint4*>(kpool + rs);
    *reinterpret_cast<uint4*>(vpool + rd) = *reinterpret_cast<const uint4*>(vpool + rs);
  }
}

// ---------------------------------------------------------------------------
// Post-attention kernel, grid (blocks per group, groups).  Every block:
//  * merges the splits' (max, sum) of all layers of its group;
//  * block c < L writes the attention output of layer c
//    (out = sum_s e^{m_s - M} o_s / Z);
//  * on an observation step, folds its slots' probability mass layer by
//    layer: mass_l[t] = sum_{h in group} exp(s_l[h][t] - M_l[h]) / Z_l[h],
//    m <- a*mass + (1-a)*m (EMA) or m <- m + mass (cumulative), l = 0..L-1
//    ("What Matters ...", section 3.1 Eq.1 pooled per KV head, Eq.3/Eq.4,
//    appendix E "Layer scoring"); the new token starts at 0.
// The group's last block to finish (fence + arrival counter, no waiting)
// records the new token's position, gives it the mean utility on a
// non-observation step (appendix E "New token insertion"), commits the
// count and, when asked, selects and compacts the group.
// ---------------------------------------------------------------------------
struct PostArgs {
  int* count;
  int* pos;
  float* score;
  int* nextpos;
  const float* logits;
  const float* part_ml;
  const float* part_o;
  float* out;
  unsigned* grpctr;
  int* mv_src;
  int* mv_dst;
  int* nmoves;
  int* errflag;
  void* kpool;
  void* vpool;
  const int* ptab;
  int L, G, Hkv, Hq, S, CT, maxpages;
  int64_t cap, P;
  float a;
  int cumulative, refresh, do_select, B, n_sink, n_recent, inline_moves, nblk;
};

constexpr int kPostTok = 64;  // slots folded per post block

template <typename T, int D, int HG, int NT>
__global__ __launch_bounds__(NT) void post_kernel(PostArgs A) {
  static_assert(NT % kPostTok == 0, "block shape");
  constexpr int LG = NT / kPostTok;  // layer lanes per slot
  extern __shared__ float dyn[];
  const int L = A.L;
  float* s_ml = dyn;                        // [L][HG][2]
  float* s_w = dyn + L * HG * 2;            // [HG][S] split weights of this block's layer
  float* s_mass = s_w + HG * A.S;           // [L][kPostTok]
  __shared__ float red[NT / kWave];
  __shared__ int s_last;
  const int c = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int n = A.count[g] + 1;
  const int ns = (n + A.CT - 1) / A.CT;
  const int Bsz = A.G / A.Hkv, b = g / A.Hkv, kvh = g % A.Hkv;

  // merge every layer's split statistics: (M, Z) per (layer, head)
  for (int i = tid; i < L * HG; i += NT) {
    const int l = i / HG, h = i % HG;
    const float2* pm = reinterpret_cast<const float2*>(A.part_ml) +
                       (static_cast<int64_t>(l) * A.G + g) * A.S * HG + h;
    float M = -INFINITY, Z = 0.f;
    for (int s0 = 0; s0 < ns; s0 += 8) {
      float2 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = s0 + k < ns ? pm[(s0 + k) * HG] : make_float2(-INFINITY, 0.f);
      float Mb = M;
#pragma unroll
      for (int k = 0; k < 8; ++k) Mb = fmaxf(Mb, v[k].x);
      float z = M == -INFINITY ? 0.f : Z * __expf(M - Mb);
#pragma unroll
      for (int k = 0; k < 8; ++k) z += v[k].x == -INFINITY ? 0.f : v[k].y * __expf(v[k].x - Mb);
      M = Mb;
      Z = z;
    }
    s_ml[i * 2 + 0] = M;
    s_ml[i * 2 + 1] = Z;
  }
  __syncthreads();

  // attention output of layer c
  if (c < L) {
    const int l = c;
    const float2* pm = reinterpret_cast<const float2*>(A.part_ml) + (static_cast<int64_t>(l) * A.G + g) * A.S * HG;
    for (int i = tid; i < HG * ns; i += NT) {
      const int h = i / ns, s = i % ns;
      const float ms = pm[s * HG + h].x;
      s_w[h * A.S + s] = ms == -INFINITY ? 0.f : __expf(ms - s_ml[(l * HG + h) * 2]);
    }
    __syncthreads();
    const float* po = A.part_o + (static_cast<int64_t>(l) * A.G + g) * A.S * HG * D;
    for (int idx = tid; idx < HG * D; idx += NT) {
      const int h = idx / D, cc = idx % D;
      float o = 0.f;
      for (int s0 = 0; s0 < ns; s0 += 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = s0 + k < ns ? po[(s0 + k) * HG * D + idx] : 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) o += s0 + k < ns ? s_w[h * A.S + s0 + k] * v[k] : 0.f;
      }
      A.out[(static_cast<int64_t>(l * Bsz + b) * A.Hq + kvh * HG + h) * D + cc] = o / s_ml[(l * HG + h) * 2 + 1];
    }
  }

  // probability mass per (layer, slot), then the layer-ordered fold
  const int tbase = c * kPostTok;
  if (A.refresh && tbase < n) {
    const int tl = tid % kPostTok, lg = tid / kPostTok;
    const int t = tbase + tl;
    if (t < n) {
      for (int l0 = lg; l0 < L; l0 += LG * 8) {
        float4 s4[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int l = l0 + k * LG;
          s4[k] = l < L ? *reinterpret_cast<const float4*>(
                              A.logits + ((static_cast<int64_t>(g) * L + l) * A.cap + t) * HG)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int l = l0 + k * LG;
          if (l >= L) continue;
          const float* ml = &s_ml[l * HG * 2];
          s_mass[l * kPostTok + tl] = __expf(s4[k].x - ml[0]) / ml[1] + __expf(s4[k].y - ml[2]) / ml[3] +
                                      __expf(s4[k].z - ml[4]) / ml[5] + __expf(s4[k].w - ml[6]) / ml[7];
        }
      }
    }
    __syncthreads();
    if (tid < kPostTok && t < n) {
      float m = (t == n - 1) ? 0.f : A.score[static_cast<int64_t>(g) * A.cap + t];
      const float keep = 1.0f - A.a;
      for (int l = 0; l < L; ++l) {
        const float mass = s_mass[l * kPostTok + tl];
        m = A.cumulative ? m + mass : A.a * mass + keep * m;
      }
      st_coherent(A.score + static_cast<int64_t>(g) * A.cap + t, m);
    }
  }

  // Arrival: the group's last block finishes the step.  The only data other
  // blocks hand over are the utilities, written through to device scope
  // above; waiting for those stores before the arrival counter is bumped
  // orders them before it, and the last block reads them with device-scope
  // loads.  (No agent-scope fence: on this GPU it writes back the whole L2.)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(&A.grpctr[g], 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == static_cast<unsigned>(A.nblk - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  int* gp = A.pos + static_cast<int64_t>(g) * A.cap;
  float* gs = A.score + static_cast<int64_t>(g) * A.cap;
  const int newest = A.nextpos[g];
  if (!A.refresh) {
    float sum = 0.f;
    for (int base = 0; base < n - 1; base += NT * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = base + u * NT + tid;
        v[u] = i < n - 1 ? ld_state<true>(gs + i) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    sum = wave_sum(sum);
    if ((tid % kWave) == 0) red[tid / kWave] = sum;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int w = 0; w < NT / kWave; ++w) tot += red[w];
      st_coherent(gs + (n - 1), n > 1 ? tot / static_cast<float>(n - 1) : 0.f);
    }
  }
  if (tid == 0) {
    st_coherent(gp + (n - 1), newest);
    A.nextpos[g] = newest + 1;
    A.grpctr[g] = 0u;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int final_n = n, nm = 0;
  if (A.do_select && n > A.B) {
    int* src = A.mv_src + static_cast<int64_t>(g) * A.cap;
    int* dst = A.mv_dst + static_cast<int64_t>(g) * A.cap;
    nm = select_group<NT, true>(n, A.B, newest, A.n_sink, A.n_recent, gp, gs, src, dst, A.errflag);
    final_n = A.B;
    if (A.inline_moves)
      copy_moves<T, D, NT>(static_cast<T*>(A.kpool), static_cast<T*>(A.vpool),
                           A.ptab + static_cast<int64_t>(g) * A.maxpages, src, dst, nm, L, A.P, A.cap);
  }
  if (tid == 0) {
    A.count[g] = final_n;
    A.nmoves[g] = A.inline_moves ? 0 : nm;
  }
}

// Standalone selection (kvev_evict): one block per group.
constexpr int kSelNT = 1024;
__global__ __launch_bounds__(kSelNT) void select_kernel(
    int* __restrict__ count, int* __restrict__ pos, float* __restrict__ score,
    const int* __restrict__ nextpos, int* __restrict__ mv_src, int* __restrict__ mv_dst,
    int* __restrict__ nmoves, int* __restrict__ errflag, int64_t cap, int B, int n_sink,
    int n_recent) {
  const int g = blockIdx.x;
  const int n = count[g];
  if (n <= B) {
    if (threadIdx.x == 0) nmoves[g] = 0;
    return;
  }
  const int nm = select_group<kSelNT, false>(n, B, nextpos[g] - 1, n_sink, n_recent,
                                      pos + static_cast<int64_t>(g) * cap,
                                      score + static_cast<int64_t>(g) * cap,
                                      mv_src + static_cast<int64_t>(g) * cap,
                                      mv_dst + static_cast<int64_t>(g) * cap, errflag);
  if (threadIdx.x == 0) {
    nmoves[g] = nm;
    count[g] = B;
  }
}

// K/V moves of the compaction plan: block (chunk of moves, group, layer).
template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void move_kernel(T* __restrict__ kpool, T* __restrict__ vpool,
                                                  const int* __restrict__ ptab,
                                                  const int* __restrict__ mv_src,
                                                  const int* __restrict__ mv_dst,
                                                  const int* __restrict__ nmoves, int64_t P,
                                                  int maxpages, int64_t cap, int per_block) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  constexpr int RPB = NT / LPR;
  const int g = blockIdx.y, l = blockIdx.z;
  const int nm = nmoves[g];
  const int j0 = blockIdx.x * per_block;
  const int j1 = min(nm, j0 + per_block);
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
  const int sub = threadIdx.x % LPR;
  for (int j = j0 + threadIdx.x / LPR; j < j1; j += RPB) {
    const int s = mv_src[static_cast<int64_t>(g) * cap + j];
    const int d = mv_dst[static_cast<int64_t>(g) * cap + j];
    if (s < 0 || s >= cap || d < 0 || d >= cap) continue;
    const int64_t rs = pool_row(l, pt[s / kPageTokens], 0, s % kPageTokens, P, 1, kPageTokens) * D;
    const int64_t rd = pool_row(l, pt[d / kPageTokens], 0, d % kPageTokens, P, 1, kPageTokens) * D;
    *reinterpret_cast<uint4*>(kpool + rd + sub * EPL) =
        *reinterpret_cast<const uint4*>(kpool + rs + sub * EPL);
    *reinterpret_cast<uint4*>(vpool + rd + sub * EPL) =
        *reinterpret_cast<const uint4*>(vpool + rs + sub * EPL);
  }
}

// Prefill: copy k, v [L][Hkv][n][D] of one sequence into its groups' pages.
template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void scatter_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                     T* __restrict__ kpool, T* __restrict__ vpool,
                                                     const int* __restrict__ ptab, int seq, int Hkv,
                                                     int64_t n, int64_t P, int maxpages) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  constexpr int RPB = NT / LPR;
  const int h = blockIdx.y, l = blockIdx.z;
  const int g = seq * Hkv + h;
  const int sub = threadIdx.x % LPR;
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR; t < n;
       t += static_cast<int64_t>(gridDim.x) * RPB) {
    const int64_t src = ((static_cast<int64_t>(l) * Hkv + h) * n + t) * D + sub * EPL;
    const int64_t dst = pool_row(l, pt[t / kPageTokens], 0, static_cast<int>(t % kPageTokens), P, 1,
                                 kPageTokens) * D + sub * EPL;
    *reinterpret_cast<uint4*>(kpool + dst) = *reinterpret_cast<const uint4*>(k + src);
    *reinterpret_cast<uint4*>(vpool + dst) = *reinterpret_cast<const uint4*>(v + src);
  }
}

// Gather (dir 0) or scatter (dir 1) one group's slots against dense [L][n][D].
template <typename T, int D, int NT>
__global__ __launch_bounds__(NT) void group_copy_kernel(T* __restrict__ kd, T* __restrict__ vd,
                                                        T* __restrict__ kpool, T* __restrict__ vpool,
                                                        const int* __restrict__ ptab, int g,
                                                        int64_t n, int64_t ld, int64_t P,
                                                        int maxpages, int dir) {
  constexpr int EPL = Vec16<T>::N;
  constexpr int LPR = D / EPL;
  constexpr int RPB = NT / LPR;
  const int l = blockIdx.y;
  const int sub = threadIdx.x % LPR;
  const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR; t < n;
       t += static_cast<int64_t>(gridDim.x) * RPB) {
    const int64_t dense = (static_cast<int64_t>(l) * ld + t) * D + sub * EPL;
    const int64_t paged = pool_row(l, pt[t / kPageTokens], 0, static_cast<int>(t % kPageTokens), P,
                                   1, kPageTokens) * D + sub * EPL;
    if (dir == 0) {
      *reinterpret_cast<uint4*>(kd + dense) = *reinterpret_cast<const uint4*>(kpool + paged);
      *reinterpret_cast<uint4*>(vd + dense) = *reinterpret_cast<const uint4*>(vpool + paged);
    } else {
      *reinterpret_cast<uint4*>(kpool + paged) = *reinterpret_cast<const uint4*>(kd + dense);
      *reinterpret_cast<uint4*>(vpool + paged) = *reinterpret_cast<const uint4*>(vd + dense);
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
static hipError_t post_impl(kvev_ctx* c, float* out, int n_max, int refresh, int do_select,
                            int64_t budget, int inline_moves) {
  constexpr int NT = 256;
  const auto& cf = c->cfg;
  PostArgs A;
  A.count = c->d.count;
  A.pos = c->d.pos;
  A.score = c->d.score;
  A.nextpos = c->d.nextpos;
  A.logits = c->d.logits;
  A.part_ml = c->d.part_ml;
  A.part_o = c->d.part_o;
  A.out = out;
  A.grpctr = c->d.grpctr;
  A.mv_src = c->d.mv_src;
  A.mv_dst = c->d.mv_dst;
  A.nmoves = c->d.nmoves;
  A.errflag = c->d.errflag;
  A.kpool = c->d.kpool;
  A.vpool = c->d.vpool;
  A.ptab = c->d.ptab;
  A.L = cf.n_layers;
  A.G = c->G;
  A.Hkv = cf.n_kv_heads;
  A.Hq = cf.n_q_heads;
  A.S = c->max_splits;
  A.CT = kAttnChunk;
  A.maxpages = c->maxpages;
  A.cap = c->cap;
  A.P = c->P;
  A.a = cf.alpha_new;
  A.cumulative = cf.policy == KVEV_CUMULATIVE;
  A.refresh = refresh;
  A.do_select = do_select;
  A.B = static_cast<int>(budget);
  A.n_sink = cf.n_sink;
  A.n_recent = cf.n_recent;
  A.inline_moves = inline_moves;
  const int tok_blocks = (n_max + kPostTok - 1) / kPostTok;
  A.nblk = tok_blocks > cf.n_layers ? tok_blocks : cf.n_layers;
  dim3 grid(A.nblk, c->G);
  const size_t shm = (static_cast<size_t>(cf.n_layers) * c->HG * 2 + static_cast<size_t>(c->HG) * A.S +
                      static_cast<size_t>(cf.n_layers) * kPostTok) * sizeof(float);
  post_kernel<T, D, 4, NT><<<grid, NT, shm, c->stream>>>(A);
  return hipGetLastError();
}

hipError_t launch_post(kvev_ctx* c, float* out, int n_max, int refresh, int do_select,
                       int64_t budget, int inline_moves) {
  if (c->HG != 4) return hipErrorInvalidValue;
  const int D = c->cfg.head_dim;
  if (c->cfg.dtype == KVEV_BF16)
    return D == 128 ? post_impl<bf16_t, 128>(c, out, n_max, refresh, do_select, budget, inline_moves)
                    : post_impl<bf16_t, 64>(c, out, n_max, refresh, do_select, budget, inline_moves);
  return D == 128 ? post_impl<float, 128>(c, out, n_max, refresh, do_select, budget, inline_moves)
                  : post_impl<float, 64>(c, out, n_max, refresh, do_select, budget, inline_moves);
}

hipError_t launch_select(kvev_ctx* c, int64_t budget) {
  const auto& cf = c->cfg;
  select_kernel<<<c->G, kSelNT, 0, c->stream>>>(c->d.count, c->d.pos, c->d.score, c->d.nextpos,
                                                c->d.mv_src, c->d.mv_dst, c->d.nmoves,
                                                c->d.errflag, c->cap, static_cast<int>(budget),
                                                cf.n_sink, cf.n_recent);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t moves_impl(kvev_ctx* c, int max_moves) {
  constexpr int NT = 256, PER = 64;
  dim3 grid((max_moves + PER - 1) / PER, c->G, c->cfg.n_layers);
  move_kernel<T, D, NT><<<grid, NT, 0, c->stream>>>(
      static_cast<T*>(c->d.kpool), static_cast<T*>(c->d.vpool), c->d.ptab, c->d.mv_src,
      c->d.mv_dst, c->d.nmoves, c->P, c->maxpages, c->cap, PER);
  return hipGetLastError();
}

hipError_t launch_moves(kvev_ctx* c, int max_moves) {
  const int D = c->cfg.head_dim;
  if (c->cfg.dtype == KVEV_BF16) return D == 128 ? moves_impl<bf16_t, 128>(c, max_moves)
                                                 : moves_impl<bf16_t, 64>(c, max_moves);
  return D == 128 ? moves_impl<float, 128>(c, max_moves) : moves_impl<float, 64>(c, max_moves);
}

template <typename T, int D>
static hipError_t scatter_impl(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n) {
  constexpr int NT = 256;
  constexpr int RPB = NT / (D / Vec16<T>::N);
  int64_t bx = (n + RPB - 1) / RPB;
  if (bx > 4096) bx = 4096;
  dim3 grid(static_cast<unsigned>(bx), c->cfg.n_kv_heads, c->cfg.n_layers);
  scatter_kernel<T, D, NT><<<grid, NT, 0, c->stream>>>(
      static_cast<const T*>(k), static_cast<const T*>(v), static_cast<T*>(c->d.kpool),
      static_cast<T*>(c->d.vpool), c->d.ptab, seq, c->cfg.n_kv_heads, n, c->P, c->maxpages);
  return hipGetLastError();
}

hipError_t launch_prefill_scatter(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n) {
  const int D = c->cfg.head_dim;
  if (c->cfg.dtype == KVEV_BF16) return D == 128 ? scatter_impl<bf16_t, 128>(c, seq, k, v, n)
                                                 : scatter_impl<bf16_t, 64>(c, seq, k, v, n);
  return D == 128 ? scatter_impl<float, 128>(c, seq, k, v, n) : scatter_impl<float, 64>(c, seq, k, v, n);
}

template <typename T, int D>
static hipError_t group_copy_impl(kvev_ctx* c, int g, void* k, void* v, int64_t n, int64_t ld,
                                  int dir) {
  constexpr int NT = 256;
  constexpr int RPB = NT / (D / Vec16<T>::N);
  int64_t bx = (n + RPB - 1) / RPB;
  if (bx < 1) return hipSuccess;
  if (bx > 4096) bx = 4096;
  dim3 grid(static_cast<unsigned>(bx), c->cfg.n_layers);
  group_copy_kernel<T, D, NT><<<grid, NT, 0, c->stream>>>(
      static_cast<T*>(k), static_cast<T*>(v), static_cast<T*>(c->d.kpool),
      static_cast<T*>(c->d.vpool), c->d.ptab, g, n, ld, c->P, c->maxpages, dir);
  return hipGetLastError();
}

static hipError_t group_copy(kvev_ctx* c, int g, void* k, void* v, int64_t n, int64_t ld, int dir) {
  const int D = c->cfg.head_dim;
  if (c->cfg.dtype == KVEV_BF16) return D == 128 ? group_copy_impl<bf16_t, 128>(c, g, k, v, n, ld, dir)
                                                 : group_copy_impl<bf16_t, 64>(c, g, k, v, n, ld, dir);
  return D == 128 ? group_copy_impl<float, 128>(c, g, k, v, n, ld, dir)
                  : group_copy_impl<float, 64>(c, g, k, v, n, ld, dir);
}

hipError_t launch_export(kvev_ctx* c, int g, void* k_out, void* v_out, int64_t n, int64_t cap) {
  return group_copy(c, g, k_out, v_out, n, cap, 0);
}

hipError_t launch_import(kvev_ctx* c, int g, const void* k, const void* v, int64_t n) {
  return group_copy(c, g, const_cast<void*>(k), const_cast<void*>(v), n, n, 1);
}

}  // namespace kvev
