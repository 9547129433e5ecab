// Block-granular LRFU mode: eviction per (sequence, 16-token block) over every
// layer and KV head.
//
// Sources: the "Attention-Aware Block Eviction" figure page (KV-cache docs,
// chapter 7: block unit, EMA score, priority (1 - score)(1 - e^{-beta idle}),
// score persistence across eviction and re-admission) and "MemDecay"
// section III (region labels, pinned system region, decay clock of Eq.3 with
// the threshold scaled to the uniform level, per-page eviction, Eq.7 rates).
//
// Layout.  Every KV head of a sequence shares one block table: entry e of
// sequence b holds logical block btab[b][e] (block id = position / 16), and
// group g = b*Hkv + h stores that block's tokens in physical page
// ptab[g][e].  Entries are kept in table order across evictions (stable
// compaction) and the block holding the newest token is always the last
// entry, so slot s of a group is token 16*btab[s/16] + s%16 and the groups'
// slot counts stay 16*(entries-1) + tail fill.  Each group owns the pages
// [g*maxpages, (g+1)*maxpages) and keeps the unused ones on a device-side
// stack, so eviction and block opening never wait for the host.
#include "kvev_internal.h"

namespace kvev {

struct BlockArgs {
  int* count;
  int* pos;
  int* nextpos;
  int* ptab;
  int* btab;
  int* nres;
  float* bscore;
  int* btref;
  int* bres;
  uint8_t* bcnt;
  int* fstack;
  int* ftop;
  float* bmass;
  const int* bbudget;
  int* errflag;
  const float* logits;
  float* ml;
  const float* part_ml;
  const float* part_o;
  float* out;
  // host-offload tier (null when off)
  int* ev_n;      // [batch] blocks the last selection evicted
  int* ev_blk;    // [batch][maxpages] their block ids, in table order
  int* ev_page;   // [G][maxpages] their pages, per KV head
  int* hslot;     // [batch][maxblk] host-pool slot holding an evicted block, or -1
  int* sowner;    // [offload_blocks] b * maxblk + block of each slot's block, or -1
  int* oring;     // [2] next ring slot, and its value after this selection
  float omin;     // evicted blocks scoring below omin are dropped, not offloaded
  int L, G, Hkv, Hq, HG, D, maxpages, maxblk, S, batch;
  int64_t cap, lstride;
  float alpha, beta, tau;
  float lam[kRegions];
  unsigned pinned_mask;
  int decode_region;
  int t;
};

// ---------------------------------------------------------------------------
// Open: before attention, give the new token its slot.  When the token's
// position starts a block, pop one page per KV head, append the block as the
// new last table entry with score 0 and clock t, and count the token in its
// block's region composition.  One block of threads per sequence.
// ---------------------------------------------------------------------------
__global__ void blk_open_kernel(BlockArgs A, int n_max) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int g0 = b * A.Hkv;
  const int newest = A.nextpos[g0];
  const int cnt = A.count[g0];
  if (cnt + 1 > n_max || newest / kPageTokens >= A.maxblk) {
    // the host's launch shape does not cover this sequence: refuse to let
    // the attention run past it (the context fails at the next sync)
    if (tid < A.Hkv) A.count[g0 + tid] = n_max - 1;
    if (tid == 0) atomicOr(A.errflag, 16);
    return;
  }
  const bool opens = newest % kPageTokens == 0;
  const int e = A.nres[b];
  const int j = newest / kPageTokens;
  if (opens && e >= A.maxpages) {
    if (tid == 0) atomicOr(A.errflag, 8);
    return;
  }
  if (tid < A.Hkv) {
    const int g = g0 + tid;
    if (opens) {
      const int top = A.ftop[g];
      if (top <= 0) {
        atomicOr(A.errflag, 8);
      } else {
        A.ptab[static_cast<int64_t>(g) * A.maxpages + e] = A.fstack[static_cast<int64_t>(g) * A.maxpages + top - 1];
        A.ftop[g] = top - 1;
      }
    }
    A.pos[static_cast<int64_t>(g) * A.cap + cnt] = newest;
    A.nextpos[g] = newest + 1;
  }
  if (tid == 0) {
    const int64_t bj = static_cast<int64_t>(b) * A.maxblk + j;
    if (opens) {
      A.btab[static_cast<int64_t>(b) * A.maxpages + e] = j;
      A.nres[b] = e + 1;
      A.bscore[bj] = 0.f;
      A.btref[bj] = A.t;
      A.bres[bj] = 1;
      for (int r = 0; r < kRegions; ++r) A.bcnt[bj * kRegions + r] = 0;
    }
    A.bcnt[bj * kRegions + A.decode_region] += 1;
  }
}

// ---------------------------------------------------------------------------
// Merge the attention splits of one (layer, group): per-head global (max,
// sum) into ml and the normalised output into out.
// ---------------------------------------------------------------------------
constexpr int kBlkMergeLoads = 16;
template <int NT>
__global__ __launch_bounds__(NT) void blk_merge_kernel(BlockArgs A) {
  const int l = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int b = g / A.Hkv, kvh = g % A.Hkv;
  const int HG = A.HG, D = A.D, S = A.S;
  extern __shared__ float sh[];
  float* s_w = sh;             // [HG][S] split weights
  float* s_mz = sh + HG * S;   // [HG][2]
  float2* s_pm = reinterpret_cast<float2*>(s_mz + HG * 2);  // [S][HG] split (max, sum)
  const float2* pm = reinterpret_cast<const float2*>(A.part_ml) + (static_cast<int64_t>(l) * A.G + g) * S * HG;
  // splits past the group's own token count were not written this step
  const int ns = (A.count[g] + 1 + kAttnChunk - 1) / kAttnChunk;
  // the splits' statistics in one batch of loads
  for (int i = tid; i < ns * HG; i += NT) s_pm[i] = pm[i];
  __syncthreads();
  if (tid < HG) {
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, s_pm[s * HG + tid].x);
    float Z = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float2 v = s_pm[s * HG + tid];
      const float w = v.x == -INFINITY ? 0.f : __expf(v.x - M);
      s_w[tid * S + s] = w;
      Z += v.y * w;
    }
    s_mz[tid * 2] = M;
    s_mz[tid * 2 + 1] = Z;
    reinterpret_cast<float2*>(A.ml)[(static_cast<int64_t>(l) * A.G + g) * HG + tid] =
        make_float2(M, Z);
  }
  __syncthreads();
  const float* po = A.part_o + (static_cast<int64_t>(l) * A.G + g) * S * HG * D;
  for (int idx = tid; idx < HG * D; idx += NT) {
    const int h = idx / D;
    float o = 0.f;
    // kBlkMergeLoads independent loads per batch, summed in split order
    for (int s0 = 0; s0 < ns; s0 += kBlkMergeLoads) {
      float v[kBlkMergeLoads];
#pragma unroll
      for (int k = 0; k < kBlkMergeLoads; ++k)
        v[k] = s0 + k < ns ? po[static_cast<int64_t>(s0 + k) * HG * D + idx] : 0.f;
#pragma unroll
      for (int k = 0; k < kBlkMergeLoads; ++k)
        if (s0 + k < ns) o += s_w[h * S + s0 + k] * v[k];
    }
    A.out[(static_cast<int64_t>(l * A.batch + b) * A.Hq + kvh * HG) * D + idx] = o / s_mz[h * 2 + 1];
  }
}

// ---------------------------------------------------------------------------
// Mass: per table entry, the probability landing on the block's tokens,
// summed over every layer, KV head and query head.  Block (4 entries,
// sequence); thread (slot of 64, quarter of the (layer, KV head) pairs).
// ---------------------------------------------------------------------------
constexpr int kMassNT = 256;
constexpr int kMassLoads = 16;
__global__ __launch_bounds__(kMassNT) void blk_mass_kernel(BlockArgs A) {
  const int b = blockIdx.y, tid = threadIdx.x;
  const int g0 = b * A.Hkv;
  const int nres = A.nres[b];
  const int e0 = blockIdx.x * 4;
  if (e0 >= nres) return;
  const int n = A.count[g0] + 1;  // slots including the new token
  extern __shared__ float sh[];
  float* s_ml = sh;                            // [L][Hkv][4][2]
  float* s_red = sh + A.L * A.Hkv * 8;         // [4][64]
  const int nml = A.L * A.Hkv * 8;
  for (int i = tid; i < nml; i += kMassNT) {
    const int l = i / (A.Hkv * 8), rest = i % (A.Hkv * 8);
    s_ml[i] = A.ml[((static_cast<int64_t>(l) * A.G + g0) * 4) * 2 + rest];
  }
  __syncthreads();
  const int sl = tid % 64, part = tid / 64;
  const int slot = e0 * kPageTokens + sl;
  float acc = 0.f;
  if (slot < n) {
    // the thread's (layer, KV head) pairs part, part + 4, ... in batches of
    // kMassLoads independent loads (indices clamped into the pairs; the
    // clamped ones are not summed), summed in pair order
    const int np = A.L * A.Hkv;
    for (int i0 = part; i0 < np; i0 += 4 * kMassLoads) {
      float4 x[kMassLoads];
#pragma unroll
      for (int k = 0; k < kMassLoads; ++k) {
        const int i = min(i0 + 4 * k, np - 1);
        const int l = i / A.Hkv, h = i % A.Hkv;
        x[k] = *reinterpret_cast<const float4*>(
            A.logits + ((static_cast<int64_t>(g0 + h) * A.L + l) * A.lstride + slot) * 4);
      }
#pragma unroll
      for (int k = 0; k < kMassLoads; ++k) {
        const int i = i0 + 4 * k;
        if (i >= np) continue;
        const float* m = &s_ml[i * 8];
        acc += __expf(x[k].x - m[0]) / m[1] + __expf(x[k].y - m[2]) / m[3] + __expf(x[k].z - m[4]) / m[5] +
               __expf(x[k].w - m[6]) / m[7];
      }
    }
  }
  s_red[part * 64 + sl] = acc;
  __syncthreads();
  if (tid < 64) {
    float v = s_red[tid] + s_red[64 + tid] + s_red[128 + tid] + s_red[192 + tid];
    v = row16_sum(v);
    const int e = e0 + tid / kPageTokens;
    if ((tid % kPageTokens) == 0 && e < nres) A.bmass[static_cast<int64_t>(b) * A.maxpages + e] = v;
  }
}

// Mass of each table entry from the attention's per-block sums (matrix-core
// path): sum over (layer, KV head, head) of bpart * exp(m_split - M) / Z,
// m_split the maximum of the entry's split (256 slots = 16 entries), M and
// Z the merged statistics.  One wave per entry, four entries per block.
__global__ __launch_bounds__(256) void blk_mass_part_kernel(BlockArgs A, const float* __restrict__ bpart) {
  extern __shared__ float fac[];  // [L * Hkv][4] exp(m_split - M) / Z of the block's split
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid % kWave;
  const int g0 = b * A.Hkv;
  const int e0 = blockIdx.x * 4, e = e0 + tid / kWave;
  const int nres = A.nres[b];
  if (e0 >= nres) return;
  const int split = e0 / (kAttnChunk / kPageTokens);  // the block's 4 entries share it
  const int np = A.L * A.Hkv;
  for (int i = tid; i < np; i += 256) {
    const int l = i / A.Hkv, h = i % A.Hkv;
    const int64_t lg = static_cast<int64_t>(l) * A.G + g0 + h;
    const float* ml = A.ml + lg * 8;                        // [4 heads][M, Z]
    const float* pm = A.part_ml + (lg * A.S + split) * 8;   // the split's [4][m, l]
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float ms = pm[2 * hh];
      fac[i * 4 + hh] = ms == -INFINITY ? 0.f : __expf(ms - ml[2 * hh]) / ml[2 * hh + 1];
    }
  }
  __syncthreads();
  float acc = 0.f;
  if (e < nres) {
    for (int i = lane; i < np; i += kWave) {
      const int l = i / A.Hkv, h = i % A.Hkv;
      const int64_t lg = static_cast<int64_t>(l) * A.G + g0 + h;
      const float4 x = *reinterpret_cast<const float4*>(bpart + (lg * A.maxpages + e) * 4);
      const float4 f = *reinterpret_cast<const float4*>(&fac[i * 4]);
      acc += x.x * f.x + x.y * f.y + x.z * f.z + x.w * f.w;
    }
  }
  acc = wave_sum(acc);
  if (lane == 0 && e < nres) A.bmass[static_cast<int64_t>(b) * A.maxpages + e] = acc;
}

// Mass after the whole-cache attention, which wrote the group mass of every
// table entry per (layer, KV head) into gm [batch][L][Hkv][maxpages]: per
// entry, their sum over every layer and KV head (each quarter of the
// threads sums a quarter of the pairs in order, the quarters are added in
// order).  Block (64 entries, sequence).
__global__ __launch_bounds__(256) void blk_entry_mass_kernel(BlockArgs A, const float* __restrict__ gm) {
  __shared__ float s_red[4][64];
  const int b = blockIdx.y, tid = threadIdx.x;
  const int e = blockIdx.x * 64 + tid % 64, part = tid / 64;
  const int nres = A.nres[b];
  if (blockIdx.x * 64 >= nres) return;
  const int np = A.L * A.Hkv;
  const float* src = gm + static_cast<int64_t>(b) * np * A.maxpages + (e < nres ? e : 0);
  float acc = 0.f;
  for (int i0 = part; i0 < np; i0 += 4 * kMassLoads) {
    float x[kMassLoads];
#pragma unroll
    for (int k = 0; k < kMassLoads; ++k) x[k] = src[static_cast<int64_t>(min(i0 + 4 * k, np - 1)) * A.maxpages];
#pragma unroll
    for (int k = 0; k < kMassLoads; ++k)
      if (i0 + 4 * k < np) acc += x[k];
  }
  s_red[part][tid % 64] = acc;
  __syncthreads();
  if (tid < 64 && e < nres)
    A.bmass[static_cast<int64_t>(b) * A.maxpages + e] =
        ((s_red[0][tid] + s_red[1][tid]) + s_red[2][tid]) + s_red[3][tid];
}

// Exclusive prefix sum of one int per thread over the block (NT threads).
template <int NT>
__device__ int block_exclusive_scan(int v, int* s_tmp, int* total) {
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) s_tmp[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < NT / kWave; ++i) {
    if (i < w) base += s_tmp[i];
    tot += s_tmp[i];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// ---------------------------------------------------------------------------
// Policy: per sequence, the score / clock update of every resident block
// (update), then (do_select) the priority of every block, the selection of
// the budget's lowest priorities with the pinned blocks forced, and the
// stable compaction of the block table, page tables and positions; evicted
// pages return to their group's stack.  appended: the step's new token is
// resident but not yet counted in count[].
// ---------------------------------------------------------------------------
constexpr int kPolNT = 256;
__global__ __launch_bounds__(kPolNT) void blk_policy_kernel(BlockArgs A, int update, int do_select,
                                                            int appended, int budget_override) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int g0 = b * A.Hkv;
  const int nres = A.nres[b];
  const int cnt = A.count[g0] + (appended ? 1 : 0);
  const int fill = cnt - kPageTokens * (nres - 1);
  const int B = budget_override > 0 ? budget_override : A.bbudget[b];
  const bool sel = do_select && nres > B;
  // LDS: the keys (later the new block table in their first half and the
  // staged table rows in their second half), then the new index per entry
  extern __shared__ unsigned char shb[];
  unsigned long long* s_key = reinterpret_cast<unsigned long long*>(shb);   // [maxpages]
  int* s_btab = reinterpret_cast<int*>(s_key);                             // [maxpages], after ranking
  int* s_row = s_btab + A.maxpages;                                        // [maxpages], after ranking
  int* s_new = reinterpret_cast<int*>(s_key + A.maxpages);                 // [maxpages]
  __shared__ int s_tmp[kPolNT / kWave];
  const int64_t brow = static_cast<int64_t>(b) * A.maxpages;
  const int64_t bblk = static_cast<int64_t>(b) * A.maxblk;
  const float inv = 1.0f / static_cast<float>(A.Hq * A.L);
  const float thr = A.tau / static_cast<float>(cnt);

  for (int e = tid; e < nres; e += kPolNT) {
    const int j = A.btab[brow + e];
    const int nb = (e == nres - 1) ? fill : kPageTokens;
    float sc = A.bscore[bblk + j];
    int tr = A.btref[bblk + j];
    if (update) {
      const float mass = A.bmass[brow + e] * inv;
      sc = A.alpha * mass + (1.0f - A.alpha) * sc;
      A.bscore[bblk + j] = sc;
      if (mass / static_cast<float>(nb) >= thr) {
        tr = A.t;
        A.btref[bblk + j] = tr;
      }
    }
    if (sel) {
      const float idle = static_cast<float>(A.t - tr);
      bool pin = e == nres - 1;
      float surv = 0.f;
      const uint8_t* cnt8 = A.bcnt + (bblk + j) * kRegions;
#pragma unroll
      for (int r = 0; r < kRegions; ++r) {
        const int c8 = cnt8[r];
        if (c8 == 0) continue;
        surv += static_cast<float>(c8) * __expf(-(A.beta + A.lam[r]) * idle);
        if ((A.pinned_mask >> r) & 1u) pin = true;
      }
      surv /= static_cast<float>(nb);
      const float prio = (1.0f - sc) * (1.0f - surv);
      // larger key is kept: lower priority first, then the higher block id
      s_key[e] = pin ? ~0ull
                     : (static_cast<unsigned long long>(~float_key(prio)) << 32) | static_cast<uint32_t>(j);
    }
  }
  if (!sel) {
    if (appended && tid < A.Hkv) A.count[g0 + tid] = cnt;
    if (A.ev_n && tid == 0) A.ev_n[b] = 0;
    return;
  }
  __syncthreads();

  // keep iff fewer than B keys are larger (pinned keys are all ~0: rank 0)
  const int per = (nres + kPolNT - 1) / kPolNT;
  const int e_lo = min(nres, tid * per), e_hi = min(nres, e_lo + per);
  int mine = 0;
  for (int e = e_lo; e < e_hi; ++e) {
    const unsigned long long k = s_key[e];
    int r = 0;
    if (k != ~0ull)
      for (int e2 = 0; e2 < nres; ++e2) r += s_key[e2] > k;
    const int keep = r < B;
    s_new[e] = keep;
    mine += keep;
  }
  int kept = 0;
  int base = block_exclusive_scan<kPolNT>(mine, s_tmp, &kept);
  // s_new[e] becomes the new index of a kept entry, or -1 - (evicted rank)
  for (int e = e_lo; e < e_hi; ++e) {
    const int keep = s_new[e];
    s_new[e] = keep ? base : -1 - (e - base);
    base += keep;
  }
  if (kept != B && tid == 0) atomicOr(A.errflag, 32);
  __syncthreads();

  // block table (built in LDS over the keys, which are no longer read),
  // evicted flags, then one page table per KV head
  for (int e = tid; e < nres; e += kPolNT) {
    const int ni = s_new[e];
    const int j = A.btab[brow + e];
    if (ni >= 0) {
      s_btab[ni] = j;
    } else {
      A.bres[bblk + j] = 0;
      if (A.ev_blk) A.ev_blk[brow + (-1 - ni)] = j;
    }
  }
  __syncthreads();
  for (int e = tid; e < kept; e += kPolNT) A.btab[brow + e] = s_btab[e];
  for (int h = 0; h < A.Hkv; ++h) {
    const int g = g0 + h;
    const int64_t grow = static_cast<int64_t>(g) * A.maxpages;
    const int top = A.ftop[g];
    for (int e = tid; e < nres; e += kPolNT) s_row[e] = A.ptab[grow + e];
    __syncthreads();
    for (int e = tid; e < nres; e += kPolNT) {
      const int ni = s_new[e];
      if (ni >= 0) {
        A.ptab[grow + ni] = s_row[e];
      } else {
        A.fstack[grow + top + (-1 - ni)] = s_row[e];
        if (A.ev_page) A.ev_page[grow + (-1 - ni)] = s_row[e];
      }
    }
    __syncthreads();
    if (tid == 0) A.ftop[g] = top + (nres - kept);
  }
  // positions of every kept slot (slot 16*i + r holds token 16*btab[i] + r)
  const int new_cnt = kPageTokens * (kept - 1) + fill;
  for (int i = tid; i < new_cnt * A.Hkv; i += kPolNT) {
    const int h = i / new_cnt, s = i % new_cnt;
    A.pos[static_cast<int64_t>(g0 + h) * A.cap + s] = s_btab[s / kPageTokens] * kPageTokens + s % kPageTokens;
  }
  if (tid < A.Hkv) A.count[g0 + tid] = new_cnt;
  if (tid == 0) A.nres[b] = kept;
  if (A.ev_n && tid == 0) A.ev_n[b] = nres - kept;
}

// ---------------------------------------------------------------------------
// Re-admission of n evicted blocks of sequence b: they take table entries
// [tail, tail + n) with their persisted score and clock t, the tail entry
// moves behind them, pages come from the groups' stacks.  One block.
// ---------------------------------------------------------------------------
__global__ void blk_readmit_kernel(BlockArgs A, int b, int n, const int* __restrict__ ids) {
  const int tid = threadIdx.x;
  const int g0 = b * A.Hkv;
  const int e_tail = A.nres[b] - 1;
  const int64_t brow = static_cast<int64_t>(b) * A.maxpages;
  const int64_t bblk = static_cast<int64_t>(b) * A.maxblk;
  if (tid < A.Hkv) {
    const int g = g0 + tid;
    const int64_t grow = static_cast<int64_t>(g) * A.maxpages;
    const int tail_page = A.ptab[grow + e_tail];
    int top = A.ftop[g];
    if (top < n) {
      atomicOr(A.errflag, 8);
      return;
    }
    for (int i = 0; i < n; ++i) A.ptab[grow + e_tail + i] = A.fstack[grow + --top];
    A.ptab[grow + e_tail + n] = tail_page;
    A.ftop[g] = top;
    const int fill = A.count[g] - kPageTokens * e_tail;
    A.count[g] += kPageTokens * n;
    // positions of the new entries and of the moved tail
    const int tail_j = A.btab[brow + e_tail];
    int* pg = A.pos + static_cast<int64_t>(g) * A.cap;
    for (int i = 0; i < n; ++i)
      for (int r = 0; r < kPageTokens; ++r) pg[kPageTokens * (e_tail + i) + r] = ids[i] * kPageTokens + r;
    for (int r = 0; r < fill; ++r) pg[kPageTokens * (e_tail + n) + r] = tail_j * kPageTokens + r;
  }
  __syncthreads();
  if (tid == 0) {
    const int tail_j = A.btab[brow + e_tail];
    for (int i = 0; i < n; ++i) {
      A.btab[brow + e_tail + i] = ids[i];
      A.bres[bblk + ids[i]] = 1;
      A.btref[bblk + ids[i]] = A.t;
    }
    A.btab[brow + e_tail + n] = tail_j;
    A.nres[b] = e_tail + 1 + n;
    // a resident block holds no host-pool slot
    if (A.hslot)
      for (int i = 0; i < n; ++i) {
        const int sl = A.hslot[bblk + ids[i]];
        if (sl >= 0) {
          A.sowner[sl] = -1;
          A.hslot[bblk + ids[i]] = -1;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Host-offload tier ("MemDecay" section III-E: pages offloaded to host memory
// before they are dropped, recovered when they become relevant again; the
// "Attention-Aware Block Eviction" page: a block's policy state survives its
// eviction).  After a selection, every evicted block's pages (each layer and
// KV head, K and V as stored) are copied into a slot of a pinned host pool
// of C slots, written by the kernel through its device mapping.  Order: the
// step's evictions whose persisted score is at least omin are offloaded,
// the others dropped; the offloaded ones are ranked by (sequence, block id)
// and, with E of them, the last min(C, E) take consecutive ring slots from
// oring[0] (the rest are dropped).  A slot's previous block loses its copy.
// offload_slot_kernel: one block per sequence ranks its evictions, assigns
// the slots and updates the slot tables; offload_copy_kernel: one block per
// (evicted block, layer) copies that layer's pages.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void offload_slot_kernel(BlockArgs A, int* __restrict__ ev_slot, int C,
                                                           int e_host) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int kb = A.ev_n[b];
  const int64_t brow = static_cast<int64_t>(b) * A.maxpages;
  auto eligible = [&](int i, int j) {  // j-th eviction of sequence i is offloaded
    const int64_t r = static_cast<int64_t>(i) * A.maxpages + j;
    return A.bscore[static_cast<int64_t>(i) * A.maxblk + A.ev_blk[r]] >= A.omin;
  };
  // the step's evictions (a consistency check), and the offloaded ones
  // before this sequence's and in all: each thread counts whole sequences
  int all = 0, off = 0, E = 0;
  for (int i = tid; i < A.batch; i += 256) {
    const int k = A.ev_n[i];
    int e = 0;
    for (int j = 0; j < k; ++j) e += eligible(i, j) ? 1 : 0;
    all += k;
    off += i < b ? e : 0;
    E += e;
  }
  {
    int v[3] = {all, off, E};
#pragma unroll
    for (int x = 0; x < 3; ++x) v[x] = wave_sum_int(v[x]);
    __shared__ int red3[3][256 / kWave];
    if (tid % kWave == 0)
#pragma unroll
      for (int x = 0; x < 3; ++x) red3[x][tid / kWave] = v[x];
    __syncthreads();
    all = red3[0][0] + red3[0][1] + red3[0][2] + red3[0][3];
    off = red3[1][0] + red3[1][1] + red3[1][2] + red3[1][3];
    E = red3[2][0] + red3[2][1] + red3[2][2] + red3[2][3];
  }
  const int kept = E < C ? E : C;
  const int ring = A.oring[0];
  if (b == 0 && tid == 0) A.oring[1] = (ring + kept) % C;  // committed by the copy kernel
  for (int j = tid; j < kb; j += 256) {
    if (all != e_host) {  // the host's count sizes the launch: never disagree silently
      ev_slot[brow + j] = -1;
      atomicOr(A.errflag, 128);
      continue;
    }
    if (!eligible(b, j)) {
      ev_slot[brow + j] = -1;
      continue;
    }
    const int blk = A.ev_blk[brow + j];
    int r = 0;  // rank of the block id among the sequence's offloaded evictions
    for (int i = 0; i < kb; ++i) r += (A.ev_blk[brow + i] < blk && eligible(b, i)) ? 1 : 0;
    const int gidx = off + r - (E - kept);  // index among the offloaded ones
    if (gidx < 0) {                         // dropped: a later eviction of this step takes its slot
      ev_slot[brow + j] = -1;
      continue;
    }
    const int slot = static_cast<int>((static_cast<int64_t>(ring) + gidx) % C);
    ev_slot[brow + j] = slot;
    const int key = b * A.maxblk + blk;
    const int prev = A.sowner[slot];
    if (prev >= 0 && A.hslot[prev] == slot) A.hslot[prev] = -1;
    A.sowner[slot] = key;
    A.hslot[key] = slot;
  }
}

// pool slot layout: K pages then V pages, each [L][Hkv][page_vec] 16-byte vectors
__global__ __launch_bounds__(256) void offload_copy_kernel(BlockArgs A, const int* __restrict__ ev_slot,
                                                           uint4* __restrict__ pool,
                                                           const uint4* __restrict__ kpool,
                                                           const uint4* __restrict__ vpool, int64_t page_vec,
                                                           int64_t P) {
  const int j = blockIdx.x, b = blockIdx.y, l = blockIdx.z, tid = threadIdx.x;
  if (j == 0 && b == 0 && l == 0 && tid == 0) A.oring[0] = A.oring[1];  // the slot kernel has read oring[0]
  if (j >= A.ev_n[b]) return;
  const int64_t brow = static_cast<int64_t>(b) * A.maxpages;
  const int slot = ev_slot[brow + j];
  if (slot < 0) return;
  const int64_t per_half = static_cast<int64_t>(A.L) * A.Hkv * page_vec;
  uint4* dst = pool + static_cast<int64_t>(slot) * 2 * per_half + static_cast<int64_t>(l) * A.Hkv * page_vec;
  const int64_t n = static_cast<int64_t>(A.Hkv) * page_vec;
  for (int64_t i = tid; i < n; i += 256) {
    const int h = static_cast<int>(i / page_vec), x = static_cast<int>(i % page_vec);
    const int page = A.ev_page[static_cast<int64_t>(b * A.Hkv + h) * A.maxpages + j];
    const int64_t src = (static_cast<int64_t>(l) * P + page) * page_vec + x;
    const uint4 kv = kpool[src], vv = vpool[src];
    dst[i] = kv;
    dst[per_half + i] = vv;
  }
}

// Re-admission from the host pool: after blk_readmit_kernel gave the n blocks
// table entries [e0, e0 + n), copy block i's slot into entry e0 + i's pages;
// src[i] >= 0 is a device staging slot (a prefetched copy), -1 - s pool
// slot s.  Grid (n, Hkv * L).
__global__ __launch_bounds__(256) void restore_kernel(BlockArgs A, const uint4* __restrict__ pool,
                                                      const uint4* __restrict__ stage,
                                                      uint4* __restrict__ kpool, uint4* __restrict__ vpool,
                                                      int64_t page_vec, int64_t P, int b, int e0,
                                                      const int* __restrict__ slots) {
  const int i = blockIdx.x, lh = blockIdx.y, tid = threadIdx.x;
  const int l = lh / A.Hkv, h = lh % A.Hkv;
  const int v = slots[i];
  const int page = A.ptab[static_cast<int64_t>(b * A.Hkv + h) * A.maxpages + e0 + i];
  const int64_t per_half = static_cast<int64_t>(A.L) * A.Hkv * page_vec;
  const uint4* base = v >= 0 ? stage : pool;
  const int slot = v >= 0 ? v : -1 - v;
  const uint4* src = base + static_cast<int64_t>(slot) * 2 * per_half + static_cast<int64_t>(lh) * page_vec;
  const int64_t dst = (static_cast<int64_t>(l) * P + page) * page_vec;
  for (int x = tid; x < page_vec; x += 256) {
    kpool[dst + x] = src[x];
    vpool[dst + x] = src[per_half + x];
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static BlockArgs block_args(kvev_ctx* c, float* out, int n_max) {
  const auto& cf = c->cfg;
  BlockArgs A;
  A.count = c->d.count;
  A.pos = c->d.pos;
  A.nextpos = c->d.nextpos;
  A.ptab = c->d.ptab;
  A.btab = c->d.btab;
  A.nres = c->d.nres;
  A.bscore = c->d.bscore;
  A.btref = c->d.btref;
  A.bres = c->d.bres;
  A.bcnt = c->d.bcnt;
  A.fstack = c->d.fstack;
  A.ftop = c->d.ftop;
  A.bmass = c->d.bmass;
  A.bbudget = c->d.bbudget;
  A.errflag = c->d.errflag;
  A.logits = c->d.logits;
  A.ml = c->d.ml;
  A.part_ml = c->d.part_ml;
  A.part_o = c->d.part_o;
  A.out = out;
  A.ev_n = c->d.ev_n;
  A.ev_blk = c->d.ev_blk;
  A.ev_page = c->d.ev_page;
  A.hslot = c->d.hslot;
  A.sowner = c->d.sowner;
  A.oring = c->d.oring;
  A.omin = cf.offload_min_score;
  A.L = cf.n_layers;
  A.G = c->G;
  A.Hkv = cf.n_kv_heads;
  A.Hq = cf.n_q_heads;
  A.HG = c->HG;
  A.D = cf.head_dim;
  A.maxpages = c->maxpages;
  A.maxblk = c->maxblk;
  A.S = (n_max + kAttnChunk - 1) / kAttnChunk;
  A.batch = cf.batch;
  A.cap = c->cap;
  A.lstride = c->lstride;
  A.alpha = cf.alpha_new;
  A.beta = cf.beta;
  A.tau = cf.access_tau_mult;
  for (int r = 0; r < kRegions; ++r) A.lam[r] = c->lam[r];
  A.pinned_mask = cf.pinned_region_mask;
  A.decode_region = cf.decode_region;
  A.t = static_cast<int>(c->t);
  return A;
}

hipError_t launch_block_open(kvev_ctx* c, int n_max, int t) {
  BlockArgs A = block_args(c, nullptr, n_max);
  A.t = t;
  return timed_launch(c, "open", blk_open_kernel, dim3(c->cfg.batch), dim3(64), 0, A, n_max);
}

hipError_t launch_block_merge(kvev_ctx* c, float* out, int n_max) {
  BlockArgs A = block_args(c, out, n_max);
  dim3 grid(c->cfg.n_layers, c->G);
  const size_t shm = (static_cast<size_t>(c->HG) * A.S * 3 + c->HG * 2) * sizeof(float);
  return timed_launch(c, "merge", blk_merge_kernel<256>, grid, dim3(256), shm, A);
}

hipError_t launch_block_mass(kvev_ctx* c, int n_max) {
  BlockArgs A = block_args(c, nullptr, n_max);
  if (c->d.bpart) {  // the attention wrote per-block sums
    dim3 grid((n_max + 4 * kPageTokens - 1) / (4 * kPageTokens), c->cfg.batch);
    const size_t shm = static_cast<size_t>(c->cfg.n_layers) * c->cfg.n_kv_heads * 4 * sizeof(float);
    return timed_launch(c, "mass", blk_mass_part_kernel, grid, dim3(256), shm, A,
                        static_cast<const float*>(c->d.bpart));
  }
  dim3 grid((n_max + 63) / 64, c->cfg.batch);
  const size_t shm = (static_cast<size_t>(c->cfg.n_layers) * c->cfg.n_kv_heads * 8 + 256) * sizeof(float);
  return timed_launch(c, "mass", blk_mass_kernel, grid, dim3(kMassNT), shm, A);
}

hipError_t launch_block_entry_mass(kvev_ctx* c, int n_max) {
  BlockArgs A = block_args(c, nullptr, n_max);
  dim3 grid((n_max + 64 * kPageTokens - 1) / (64 * kPageTokens), c->cfg.batch);
  return timed_launch(c, "mass", blk_entry_mass_kernel, grid, dim3(256), 0, A, static_cast<const float*>(c->d.bpart));
}

hipError_t launch_block_policy(kvev_ctx* c, int t, int update, int do_select, int appended,
                               int budget_override) {
  BlockArgs A = block_args(c, nullptr, 1);
  A.t = t;
  const size_t shm = static_cast<size_t>(c->maxpages) * (8 + 4);
  return timed_launch(c, "policy", blk_policy_kernel, dim3(c->cfg.batch), dim3(kPolNT), shm, A, update, do_select,
                      appended, budget_override);
}

hipError_t launch_offload(kvev_ctx* c, int k_max, int e_host) {
  BlockArgs A = block_args(c, nullptr, 1);
  const int64_t page_vec = static_cast<int64_t>(c->PT) * c->cfg.head_dim * c->elem / 16;
  hipError_t e = timed_launch(c, "offload", offload_slot_kernel, dim3(c->cfg.batch), dim3(256), 0, A, c->d.ev_slot,
                              static_cast<int>(c->cfg.offload_blocks), e_host);
  if (e != hipSuccess) return e;
  dim3 grid(k_max, c->cfg.batch, c->cfg.n_layers);
  return timed_launch(c, "offload", offload_copy_kernel, grid, dim3(256), 0, A, c->d.ev_slot,
                      static_cast<uint4*>(c->hpool_dev), static_cast<const uint4*>(c->d.kpool),
                      static_cast<const uint4*>(c->d.vpool), page_vec, c->P);
}

hipError_t launch_restore(kvev_ctx* c, int b, int n, int e0, const int* src_dev) {
  BlockArgs A = block_args(c, nullptr, 1);
  const int64_t page_vec = static_cast<int64_t>(c->PT) * c->cfg.head_dim * c->elem / 16;
  dim3 grid(n, c->cfg.n_layers * c->cfg.n_kv_heads);
  restore_kernel<<<grid, 256, 0, c->stream>>>(A, static_cast<const uint4*>(c->hpool_dev),
                                              static_cast<const uint4*>(c->dstage),
                                              static_cast<uint4*>(c->d.kpool), static_cast<uint4*>(c->d.vpool),
                                              page_vec, c->P, b, e0, src_dev);
  return hipGetLastError();
}

hipError_t launch_block_readmit(kvev_ctx* c, int b, int n, const int* ids_dev, int t) {
  BlockArgs A = block_args(c, nullptr, 1);
  A.t = t;
  blk_readmit_kernel<<<1, 64, 0, c->stream>>>(A, b, n, ids_dev);
  return hipGetLastError();
}

}  // namespace kvev
