// Device helpers shared by the post-attention kernels: the top-budget
// selection with its compaction plan, slot-state access across blocks, and
// the kernels' argument block.
#pragma once
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
// straddle the cut; k == 1 is an argmin.  With k == 1 nothing moves: the
// evicted slot becomes the group's free slot, which the next token takes
// (*new_hole = that slot; the cache then spans B + 1 slots).  Otherwise the
// plan is the hole fill: holes = unkept slots < B ascending, movers = kept
// slots >= B ascending, mover j fills hole j (*new_hole = B).  All n slots
// hold tokens on entry.  Positions and utilities are moved here; returns the
// number of moves.
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
                            int* __restrict__ dst, int* __restrict__ errflag, int& new_hole) {
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
      new_hole = B;
      return 0;
    }
    new_hole = ev;  // the evicted slot is the next token's
    return 0;
  }
  new_hole = B;

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

constexpr int kPostTok = kPostTokens;  // slots per post block (one wave's worth)
constexpr int kMergeBatch = 16;

struct PostArgs {
  int* count;
  int* hole;
  int* pos;
  float* score;
  int* nextpos;
  const float* logits;
  const float* part_ml;
  const float* part_o;
  const float* part_u;   // entropy partials, or null
  const float* vnorm;    // value-row norms, or null
  const float* part_vn;  // per-split norm sums (with vnorm)
  float* out;
  unsigned* grpctr;
  unsigned long long* blk_key;
  int* blk_slot;
  float* blk_sum;
  int* mv_src;
  int* mv_dst;
  int* nmoves;
  int* errflag;
  int* dg_n;       // rank-trace diagnostics, or null: per slot of the step
  int* dg_pos;     // its position,
  float* dg_raw;   // the observation summed over layers,
  float* dg_util;  // the utility after the fold
  void* kpool;
  void* vpool;
  const int* ptab;
  const void* k_new;
  const void* v_new;
  int L, G, Hkv, Hq, S, CT, maxpages, max_blk;
  int64_t cap, P, lstride;
  float a;
  int cumulative, refresh, do_select, B, n_sink, n_recent, nblk;
  int seq;  // the whole-cache attention wrote the outputs and the per-slot group masses
  // mean_init: on an observation step the new token starts at the mean of
  // the others' utilities (else 0); wprior: the start's weight after the
  // fold over the L layers ((1 - a)^L, or 1 for the running sum)
  int mean_init;
  float wprior;
};

// The fold weight of a utility's starting value after L layers, formed in
// the fold's own fp32 order.
inline float prior_fold_weight(float a, int L, bool cumulative) {
  float w = 1.0f;
  if (!cumulative)
    for (int l = 0; l < L; ++l) w *= 1.0f - a;
  return w;
}

// HG consecutive fp32 logits (one slot of one layer)
template <int HG>
__device__ __forceinline__ void load_heads(const float* p, float* x) {
  if constexpr (HG % 4 == 0) {
#pragma unroll
    for (int h = 0; h < HG; h += 4) {
      const float4 v = *reinterpret_cast<const float4*>(p + h);
      x[h] = v.x; x[h + 1] = v.y; x[h + 2] = v.z; x[h + 3] = v.w;
    }
  } else if constexpr (HG % 2 == 0) {
#pragma unroll
    for (int h = 0; h < HG; h += 2) {
      const float2 v = *reinterpret_cast<const float2*>(p + h);
      x[h] = v.x; x[h + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int h = 0; h < HG; ++h) x[h] = p[h];
  }
}

// Post-attention launch of the sequence-pooled mode (A.nblk set by the caller).
template <typename T, int D>
hipError_t launch_pool_post(kvev_ctx* c, const PostArgs& A);

}  // namespace kvev
