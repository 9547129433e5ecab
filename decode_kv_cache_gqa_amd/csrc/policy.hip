// Append, score fold, top-budget selection with compaction plan, K/V moves.
#include "common.h"
#include "kvev_internal.h"

namespace kvev {

// ---------------------------------------------------------------------------
// Append: one block per group writes the new token's K/V of every layer into
// slot n (page table lookup), sets its position and its starting utility:
// 0 on an observation step (then folded with its own mass), else the mean of
// the group's utilities ("What Matters ...", appendix E "New token insertion
// during non-refresh steps").  Then count = n + 1.
// ---------------------------------------------------------------------------
template <typename T, int NT>
__global__ __launch_bounds__(NT) void append_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new, T* __restrict__ kpool,
    T* __restrict__ vpool, const int* __restrict__ ptab, int* __restrict__ count,
    int* __restrict__ pos, int* __restrict__ nextpos, float* __restrict__ score, int L, int G,
    int Hkv, int D, int64_t P, int maxpages, int64_t cap, int refresh) {
  __shared__ float red[NT / kWave];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int B = G / Hkv, b = g / Hkv, kvh = g % Hkv;
  const int n = count[g];
  const int page = ptab[static_cast<int64_t>(g) * maxpages + n / kPageTokens];
  const int r = n % kPageTokens;
  for (int idx = tid; idx < L * D; idx += NT) {
    const int l = idx / D, c = idx % D;
    const int64_t src = (static_cast<int64_t>(l * B + b) * Hkv + kvh) * D + c;
    const int64_t dst = pool_row(l, page, 0, r, P, 1, kPageTokens) * D + c;
    kpool[dst] = k_new[src];
    vpool[dst] = v_new[src];
  }
  float init = 0.f;
  if (!refresh) {
    // fixed-order tree sum of score[0..n)
    float s = 0.f;
    const float* sc = score + static_cast<int64_t>(g) * cap;
    for (int i = tid; i < n; i += NT) s += sc[i];
    s = wave_sum(s);
    if ((tid % kWave) == 0) red[tid / kWave] = s;
    __syncthreads();
    float tot = 0.f;
    for (int k = 0; k < NT / kWave; ++k) tot += red[k];
    init = n > 0 ? tot / static_cast<float>(n) : 0.f;
  }
  __syncthreads();  // every thread has read count[g] before it changes
  if (tid == 0) {
    score[static_cast<int64_t>(g) * cap + n] = init;
    pos[static_cast<int64_t>(g) * cap + n] = nextpos[g];
    nextpos[g] = nextpos[g] + 1;
    count[g] = n + 1;
  }
}

// ---------------------------------------------------------------------------
// Probability pass + layer-sequential fold.  One thread per token:
//   G_l[t] = sum_{h in group} exp(s_l[h][t] - M_l[h]) / Z_l[h]
//   m <- a*G_l + (1-a)*m  (EMA) or m <- m + G_l (cumulative), l = 0..L-1
// ("What Matters ...", section 3.1 Eq.1 pooled per KV head, Eq.3 / Eq.4,
// appendix E "Layer scoring").
// ---------------------------------------------------------------------------
template <int HG, int NT>
__global__ __launch_bounds__(NT) void fold_kernel(const int* __restrict__ count,
                                                  const float* __restrict__ logits,
                                                  const float* __restrict__ ml,
                                                  float* __restrict__ score, int L, int G,
                                                  int64_t cap, float a, int cumulative) {
  extern __shared__ float s_ml[];  // [L][HG][2]
  const int g = blockIdx.y, tid = threadIdx.x;
  for (int i = tid; i < L * HG * 2; i += NT) {
    const int l = i / (HG * 2), rem = i % (HG * 2);
    s_ml[i] = ml[(static_cast<int64_t>(l) * G + g) * HG * 2 + rem];
  }
  __syncthreads();
  const int n = count[g];
  const int t = blockIdx.x * NT + tid;
  if (t >= n) return;
  float m = score[static_cast<int64_t>(g) * cap + t];
  const float keep = 1.0f - a;
  for (int l = 0; l < L; ++l) {
    const float* s = logits + ((static_cast<int64_t>(g) * L + l) * cap + t) * HG;
    float mass = 0.f;
#pragma unroll
    for (int h = 0; h < HG; ++h) mass += expf(s[h] - s_ml[(l * HG + h) * 2]) / s_ml[(l * HG + h) * 2 + 1];
    m = cumulative ? m + mass : a * mass + keep * m;
  }
  score[static_cast<int64_t>(g) * cap + t] = m;
}

// ---------------------------------------------------------------------------
// Selection + compaction plan, one block per group.
// Keep the protected tokens (positions < n_sink, or among the n_recent
// newest) and evict the k = n - B lowest (score, position) keys of the rest;
// equivalently keep the top (B - |protected|).  The k-th smallest key is
// found by an LDS radix select on order-preserving 32-bit score keys (four
// 8-bit digits), with a second radix select on positions only when equal
// scores straddle the cut.  k == 1 uses an argmin.
// Plan: holes = unkept slots < B ascending, movers = kept slots >= B
// ascending, mover j -> hole j; positions and utilities are moved here, K/V
// by move_kernel.
// ---------------------------------------------------------------------------
constexpr int kSelNT = 1024;

__device__ __forceinline__ void block_scan_256(const int* hist, int* excl_out, int tid) {
  // exclusive scan of hist[0..256) into excl_out, executed by threads 0..255
  __shared__ int wsum[4];
  int v = tid < 256 ? hist[tid] : 0;
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

__global__ __launch_bounds__(kSelNT) void select_kernel(
    int* __restrict__ count, int* __restrict__ pos, float* __restrict__ score,
    const int* __restrict__ nextpos, int* __restrict__ mv_src, int* __restrict__ mv_dst,
    int* __restrict__ nmoves, int* __restrict__ errflag, int64_t cap, int B, int n_sink,
    int n_recent) {
  __shared__ int hist[256];
  __shared__ int excl[256];
  __shared__ int sel[3];
  __shared__ unsigned long long wmin[kSelNT / kWave];
  __shared__ int wcnt[2][kSelNT / kWave];
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int n = count[g];
  if (n <= B) {
    if (tid == 0) nmoves[g] = 0;
    return;
  }
  int* gp = pos + static_cast<int64_t>(g) * cap;
  float* gs = score + static_cast<int64_t>(g) * cap;
  const int newest = nextpos[g] - 1;
  const int k = n - B;  // candidates to evict
  auto is_cand = [&](int p) { return !(p < n_sink || p > newest - n_recent); };

  uint32_t thr = 0;          // score key of the cut
  int pos_cut = 0x7fffffff;  // among keys == thr, evict positions <= pos_cut
  if (k == 1) {
    unsigned long long best = ~0ull;
    for (int i = tid; i < n; i += kSelNT) {
      const int p = gp[i];
      if (!is_cand(p)) continue;
      const unsigned long long kk = (static_cast<unsigned long long>(float_key(gs[i])) << 32) |
                                    static_cast<uint32_t>(p);
      best = kk < best ? kk : best;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long y = __shfl_xor(best, o, kWave);
      best = y < best ? y : best;
    }
    if (lane == 0) wmin[wave] = best;
    __syncthreads();
    best = wmin[0];
    for (int w = 1; w < kSelNT / kWave; ++w) best = wmin[w] < best ? wmin[w] : best;
    thr = static_cast<uint32_t>(best >> 32);
    pos_cut = static_cast<int>(best & 0xffffffffu);
  } else {
    uint32_t prefix = 0, mask = 0;
    int kk = k, eq = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelNT) {
        if (!is_cand(gp[i])) continue;
        const uint32_t key = float_key(gs[i]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      block_scan_256(hist, excl, tid);
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
      // ties on the cut score: evict the kk lowest positions among them
      uint32_t pprefix = 0, pmask = 0;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kSelNT) {
          const int p = gp[i];
          if (!is_cand(p) || float_key(gs[i]) != thr) continue;
          const uint32_t key = static_cast<uint32_t>(p);
          if ((key & pmask) == pprefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        block_scan_256(hist, excl, tid);
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
  __syncthreads();

  auto keep = [&](int i) {
    const int p = gp[i];
    if (!is_cand(p)) return true;
    const uint32_t key = float_key(gs[i]);
    return key > thr || (key == thr && p > pos_cut);
  };

  // holes / movers ranks by block-wide prefix sums over slot order
  int hole_base = 0, mover_base = 0;
  int* src = mv_src + static_cast<int64_t>(g) * cap;
  int* dst = mv_dst + static_cast<int64_t>(g) * cap;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int tile = 0; tile < n; tile += kSelNT) {
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
    for (int w = 0; w < kSelNT / kWave; ++w) {
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
  for (int j = tid; j < nm; j += kSelNT) {
    const int s = src[j], d = dst[j];
    gp[d] = gp[s];
    gs[d] = gs[s];
  }
  if (tid == 0) {
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
  constexpr int LPR = D / EPL;  // lanes per row
  constexpr int RPB = NT / LPR; // rows per pass
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

template <typename T>
static hipError_t append_impl(kvev_ctx* c, const void* k_new, const void* v_new, int refresh) {
  const auto& cf = c->cfg;
  append_kernel<T, 256><<<c->G, 256, 0, c->stream>>>(
      static_cast<const T*>(k_new), static_cast<const T*>(v_new), static_cast<T*>(c->d.kpool),
      static_cast<T*>(c->d.vpool), c->d.ptab, c->d.count, c->d.pos, c->d.nextpos, c->d.score,
      cf.n_layers, c->G, cf.n_kv_heads, cf.head_dim, c->P, c->maxpages, c->cap, refresh);
  return hipGetLastError();
}

hipError_t launch_append(kvev_ctx* c, const void* k_new, const void* v_new, int refresh) {
  if (c->cfg.dtype == KVEV_BF16) return append_impl<bf16_t>(c, k_new, v_new, refresh);
  return append_impl<float>(c, k_new, v_new, refresh);
}

hipError_t launch_fold(kvev_ctx* c, int n_max) {
  constexpr int NT = 256;
  const auto& cf = c->cfg;
  if (c->HG != 4) return hipErrorInvalidValue;
  dim3 grid((n_max + NT - 1) / NT, c->G);
  const size_t shm = static_cast<size_t>(cf.n_layers) * c->HG * 2 * sizeof(float);
  fold_kernel<4, NT><<<grid, NT, shm, c->stream>>>(c->d.count, c->d.logits, c->d.ml, c->d.score,
                                                   cf.n_layers, c->G, c->cap, cf.alpha_new,
                                                   cf.policy == KVEV_CUMULATIVE);
  return hipGetLastError();
}

hipError_t launch_select(kvev_ctx* c, int64_t budget, int /*n_max*/) {
  const auto& cf = c->cfg;
  select_kernel<<<c->G, kSelNT, 0, c->stream>>>(c->d.count, c->d.pos, c->d.score, c->d.nextpos,
                                                c->d.mv_src, c->d.mv_dst, c->d.nmoves,
                                                c->d.errflag, c->cap,
                                                static_cast<int>(budget), cf.n_sink, cf.n_recent);
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
