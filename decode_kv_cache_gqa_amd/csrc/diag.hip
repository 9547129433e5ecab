// Rank-trace diagnostics of the token policies ("What Matters ...",
// appendix I, Table 13; the "QEvict" review, section 3) and the future
// missed mass of a compressed cache against a full one.
//
// After a step's post kernel, one block per (sequence, KV head) group reads
// the step's per-slot inputs (position, observation summed over layers,
// utility after the fold) and the retained state, and:
//  * stamps every retained position with the step (retained-set overlap
//    with the previous step: the positions whose stamp was that step's);
//  * finds the k-th largest 64-bit key (order-preserving score key << 32 |
//    position; keys are unique because positions are) of the raw and of
//    the utility values with an LDS radix select, 8 bits a pass from the
//    top, stopping once the selected bucket holds one key;
//  * marks the top-k members the same way, counts the overlaps, records
//    the step that evicted each position that is no longer retained, and
//    adds the step's statistics to the group's sums.
// Every per-position stamp array has one entry per position a sequence can
// reach, so nothing is cleared between steps.
#include "post_common.h"
#include "host_util.h"

#include <mutex>

namespace kvev {

constexpr int kDiagNT = 1024;

__device__ __forceinline__ unsigned long long diag_key(float v, int p) {
  return (static_cast<unsigned long long>(float_key(v)) << 32) | static_cast<uint32_t>(p);
}

// Block sums of N counters, returned to thread 0.
template <int N>
__device__ __forceinline__ void block_sum_ints(int (&v)[N], int (*red)[N]) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int j = 0; j < N; ++j) v[j] = wave_sum_int(v[j]);
  if (lane == 0)
#pragma unroll
    for (int j = 0; j < N; ++j) red[wave][j] = v[j];
  __syncthreads();
  if (threadIdx.x == 0)
#pragma unroll
    for (int j = 0; j < N; ++j) {
      int t = 0;
      for (int w = 0; w < static_cast<int>(blockDim.x) / kWave; ++w) t += red[w][j];
      v[j] = t;
    }
}

// Keys per thread held in registers; steps of more tokens read them again
// from memory on every pass.
constexpr int kDiagKPT = 8;

// The k-th largest key of the raw (set 0) and utility (set 1) values over
// slots [0, n), 1 <= k <= n.  cached: slot tid + u * kDiagNT's keys are
// kr[u], ku[u] (n <= kDiagNT * kDiagKPT).
__device__ void kth_largest_pair(int n, int k, const int* pos, const float* raw, const float* util,
                                 bool cached, const unsigned long long* kr_c,
                                 const unsigned long long* ku_c, unsigned long long* thr) {
  __shared__ int hist[2][256];
  __shared__ int excl[256];
  __shared__ int wsum[4];
  __shared__ int sel[2][2];
  __shared__ unsigned long long found[2];
  const int tid = threadIdx.x;
  unsigned long long pre[2] = {0ull, 0ull}, mask[2] = {0ull, 0ull};
  int rem[2] = {k, k};
  bool done[2] = {false, false}, unique[2] = {false, false};
  for (int shift = 56; shift >= 0 && !(done[0] && done[1]); shift -= 8) {
    for (int i = tid; i < 512; i += kDiagNT) hist[i / 256][i % 256] = 0;
    __syncthreads();
    // bins in descending digit order, so the scan counts larger keys first
    auto count = [&](unsigned long long kr, unsigned long long ku) {
      if (!done[0] && (kr & mask[0]) == pre[0]) atomicAdd(&hist[0][255 - ((kr >> shift) & 255u)], 1);
      if (!done[1] && (ku & mask[1]) == pre[1]) atomicAdd(&hist[1][255 - ((ku >> shift) & 255u)], 1);
    };
    if (cached) {
#pragma unroll
      for (int u = 0; u < kDiagKPT; ++u)
        if (tid + u * kDiagNT < n) count(kr_c[u], ku_c[u]);
    } else {
      for (int i = tid; i < n; i += kDiagNT) {
        const int p = pos[i];
        count(diag_key(raw[i], p), diag_key(util[i], p));
      }
    }
    __syncthreads();
    for (int s = 0; s < 2; ++s) {
      if (done[s]) continue;  // uniform across the block
      scan_256<kDiagNT>(hist[s], excl, wsum, tid);
      if (tid < 256 && excl[tid] < rem[s] && rem[s] <= excl[tid] + hist[s][tid]) {
        sel[s][0] = 255 - tid;
        sel[s][1] = excl[tid];
      }
      __syncthreads();
      const int digit = sel[s][0] & 255;  // a bin always holds the k-th key
      const int above = sel[s][1];
      const int cnt = hist[s][255 - digit];
      pre[s] |= static_cast<unsigned long long>(digit) << shift;
      mask[s] |= 255ull << shift;
      rem[s] -= above;
      if (shift == 0) done[s] = true;
      if (cnt == 1) done[s] = unique[s] = true;
      __syncthreads();
    }
  }
  // a bucket of one key: that key is the threshold
  if (unique[0] || unique[1]) {
    auto match = [&](unsigned long long kr, unsigned long long ku) {
      if (unique[0] && (kr & mask[0]) == pre[0]) found[0] = kr;
      if (unique[1] && (ku & mask[1]) == pre[1]) found[1] = ku;
    };
    if (cached) {
#pragma unroll
      for (int u = 0; u < kDiagKPT; ++u)
        if (tid + u * kDiagNT < n) match(kr_c[u], ku_c[u]);
    } else {
      for (int i = tid; i < n; i += kDiagNT) {
        const int p = pos[i];
        match(diag_key(raw[i], p), diag_key(util[i], p));
      }
    }
    __syncthreads();
    if (unique[0]) pre[0] = found[0];
    if (unique[1]) pre[1] = found[1];
    __syncthreads();
  }
  thr[0] = pre[0];
  thr[1] = pre[1];
}

struct DiagArgs {
  const int* dg_n;
  const int* dg_pos;
  const float* dg_raw;
  const float* dg_util;
  const int* count;
  const int* hole;
  const int* pos;
  int* st_raw;
  int* st_util;
  int* st_kept;
  int* ev_step;
  int* prev;
  int* cnt;
  double* acc;
  int* errflag;
  int64_t cap, maxpos;
  int K, t;
};

__global__ __launch_bounds__(kDiagNT) void diag_kernel(DiagArgs A) {
  __shared__ int red[kDiagNT / kWave][8];
  const int g = blockIdx.x, tid = threadIdx.x;
  const int64_t go = static_cast<int64_t>(g) * A.cap, so = static_cast<int64_t>(g) * A.maxpos;
  const int n = A.dg_n[g];
  const int* dpos = A.dg_pos + go;
  const float* draw = A.dg_raw + go;
  const float* dutil = A.dg_util + go;
  const int* gp = A.pos + go;
  int* st_raw = A.st_raw + so;
  int* st_util = A.st_util + so;
  int* st_kept = A.st_kept + so;
  int* ev_step = A.ev_step + so;
  const int tp = A.prev[g * 4 + 0];  // the previous recorded step (0: none)
  const int kprev = A.prev[g * 4 + 1], sprev = A.prev[g * 4 + 2];
  const int k = n < A.K ? n : A.K;
  // the step's keys, held in registers when they fit (loads issued first)
  const bool cached = n <= kDiagNT * kDiagKPT;
  unsigned long long kr_c[kDiagKPT], ku_c[kDiagKPT];
  int pos_c[kDiagKPT];
  if (cached) {
#pragma unroll
    for (int u = 0; u < kDiagKPT; ++u) {
      const int i = tid + u * kDiagNT;
      const bool in = i < n;
      pos_c[u] = in ? dpos[i] : -1;
      const float r = in ? draw[i] : 0.f, v = in ? dutil[i] : 0.f;
      kr_c[u] = diag_key(r, pos_c[u]);
      ku_c[u] = diag_key(v, pos_c[u]);
    }
  }

  // ---- the retained set: slots [0, count] except the free slot ------------------
  const int cnt = A.count[g], hl = A.hole[g];
  int i_s = 0, n_s = 0, bad = 0;
  auto keep_slot = [&](int p, int old) {
    if (p < 0 || p >= A.maxpos) {
      bad = 1;
      return;
    }
    i_s += (tp > 0 && old == tp) ? 1 : 0;
    st_kept[p] = A.t;
    ++n_s;
  };
  if (cnt + 1 <= kDiagNT * kDiagKPT) {
    // every position load, then every stamp load, then the stores
    int pk[kDiagKPT], old[kDiagKPT];
    bool in[kDiagKPT];
#pragma unroll
    for (int u = 0; u < kDiagKPT; ++u) {
      const int j = tid + u * kDiagNT;
      in[u] = j <= cnt && j != hl && j < A.cap;
      pk[u] = in[u] ? gp[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < kDiagKPT; ++u)
      old[u] = (in[u] && pk[u] >= 0 && pk[u] < A.maxpos) ? st_kept[pk[u]] : 0;
#pragma unroll
    for (int u = 0; u < kDiagKPT; ++u)
      if (in[u]) keep_slot(pk[u], old[u]);
  } else {
    for (int j = tid; j <= cnt; j += kDiagNT) {
      if (j == hl || j >= A.cap) continue;
      const int p = gp[j];
      keep_slot(p, (p >= 0 && p < A.maxpos) ? st_kept[p] : 0);
    }
  }

  // ---- top-k thresholds --------------------------------------------------------
  unsigned long long thr[2];
  kth_largest_pair(n, k, dpos, draw, dutil, cached, kr_c, ku_c, thr);  // synchronises the block

  // ---- membership, overlaps and evictions ------------------------------------------
  int i_r = 0, i_u = 0, i_ru = 0, i_rev = 0, n_ev = 0;
  // the stamps of a step token p: kept after this step, in the previous raw
  // and utility top-k
  auto visit = [&](int p, unsigned long long kr, unsigned long long ku, int skept, int sraw, int sutil) {
    if (p < 0 || p >= A.maxpos) {
      bad = 1;
      return;
    }
    const bool inr = kr >= thr[0];
    const bool inu = ku >= thr[1];
    const bool ev = skept != A.t;
    if (ev) {
      ev_step[p] = A.t;
      ++n_ev;
    }
    if (inr) {
      i_r += (tp > 0 && sraw == tp) ? 1 : 0;
      st_raw[p] = A.t;
    }
    if (inu) {
      i_u += (tp > 0 && sutil == tp) ? 1 : 0;
      st_util[p] = A.t;
    }
    i_ru += (inr && inu) ? 1 : 0;
    i_rev += (inr && ev) ? 1 : 0;
  };
  auto ok = [&](int p) { return p >= 0 && p < A.maxpos; };
  if (cached) {
    int sk[kDiagKPT], sr[kDiagKPT], su[kDiagKPT];
#pragma unroll
    for (int u = 0; u < kDiagKPT; ++u) {
      const int p = pos_c[u];
      const bool in = tid + u * kDiagNT < n && ok(p);
      sk[u] = in ? st_kept[p] : 0;
      sr[u] = in && kr_c[u] >= thr[0] ? st_raw[p] : 0;
      su[u] = in && ku_c[u] >= thr[1] ? st_util[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < kDiagKPT; ++u)
      if (tid + u * kDiagNT < n) visit(pos_c[u], kr_c[u], ku_c[u], sk[u], sr[u], su[u]);
  } else {
    for (int i = tid; i < n; i += kDiagNT) {
      const int p = dpos[i];
      const bool in = ok(p);
      visit(p, diag_key(draw[i], p), diag_key(dutil[i], p), in ? st_kept[p] : 0, in ? st_raw[p] : 0,
            in ? st_util[p] : 0);
    }
  }
  int sums[8] = {i_s, n_s, bad, i_r, i_u, i_ru, i_rev, n_ev};
  block_sum_ints(sums, red);
  if (tid != 0) return;
  i_s = sums[0];
  n_s = sums[1];
  bad = sums[2];
  i_r = sums[3];
  i_u = sums[4];
  i_ru = sums[5];
  i_rev = sums[6];
  n_ev = sums[7];
  if (bad) atomicOr(A.errflag, 64);
  const bool pair = tp > 0;
  int* c = A.cnt + static_cast<int64_t>(g) * kDiagCounts;
  c[0] = n;
  c[1] = k;
  c[2] = i_r;
  c[3] = pair ? kprev : 0;
  c[4] = i_u;
  c[5] = pair ? kprev : 0;
  c[6] = i_ru;
  c[7] = i_rev;
  c[8] = n_ev;
  c[9] = n_s;
  c[10] = i_s;
  c[11] = pair ? sprev : 0;
  double* a = A.acc + static_cast<int64_t>(g) * kDiagAcc;
  a[0] += 1.0;
  if (pair) {
    a[1] += 1.0;
    a[2] += 1.0 - static_cast<double>(i_r) / static_cast<double>(k + kprev - i_r);
    a[3] += 1.0 - static_cast<double>(i_u) / static_cast<double>(k + kprev - i_u);
    a[6] += 1.0 - static_cast<double>(i_s) / static_cast<double>(n_s + sprev - i_s);
  }
  a[4] += static_cast<double>(i_ru) / static_cast<double>(2 * k - i_ru);
  a[5] += static_cast<double>(i_rev) / static_cast<double>(k);
  A.prev[g * 4 + 0] = A.t;
  A.prev[g * 4 + 1] = k;
  A.prev[g * 4 + 2] = n_s;
}

// Missed mass per group: the full cache's last observation on positions the
// compressed cache evicted before step t, over the full observation's total.
__global__ __launch_bounds__(kDiagNT) void fmm_kernel(const int* __restrict__ full_n,
                                                      const int* __restrict__ full_pos,
                                                      const float* __restrict__ full_raw,
                                                      const int* __restrict__ ev_step, int64_t cap,
                                                      int64_t maxpos, int t, double* __restrict__ fmm) {
  __shared__ double red[2][kDiagNT / kWave];
  const int g = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int n = full_n[g];
  const int64_t go = static_cast<int64_t>(g) * cap;
  const int* ev = ev_step + static_cast<int64_t>(g) * maxpos;
  double miss = 0.0, tot = 0.0;
  for (int i = tid; i < n; i += kDiagNT) {
    const int p = full_pos[go + i];
    const double w = full_raw[go + i];
    tot += w;
    const int e = (p >= 0 && p < maxpos) ? ev[p] : 0;
    if (e > 0 && e < t) miss += w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    miss += __shfl_xor(miss, o, kWave);
    tot += __shfl_xor(tot, o, kWave);
  }
  if (lane == 0) {
    red[0][wave] = miss;
    red[1][wave] = tot;
  }
  __syncthreads();
  if (tid == 0) {
    double m = 0.0, s = 0.0;
    for (int w = 0; w < kDiagNT / kWave; ++w) {
      m += red[0][w];
      s += red[1][w];
    }
    fmm[g] = s > 0.0 ? m / s : 0.0;
  }
}

hipError_t launch_diag(kvev_ctx* c, int t) {
  DiagArgs A;
  A.dg_n = c->d.dg_n;
  A.dg_pos = c->d.dg_pos;
  A.dg_raw = c->d.dg_raw;
  A.dg_util = c->d.dg_util;
  A.count = c->d.count;
  A.hole = c->d.hole;
  A.pos = c->d.pos;
  A.st_raw = c->d.st_raw;
  A.st_util = c->d.st_util;
  A.st_kept = c->d.st_kept;
  A.ev_step = c->d.ev_step;
  A.prev = c->d.dprev;
  A.cnt = c->d.dcnt;
  A.acc = c->d.dacc;
  A.errflag = c->d.errflag;
  A.cap = c->cap;
  A.maxpos = c->cfg.max_tokens;
  A.K = c->cfg.diag_topk;
  A.t = t;
  diag_kernel<<<c->G, kDiagNT, 0, c->stream>>>(A);
  return hipGetLastError();
}

hipError_t launch_fmm(kvev_ctx* full, kvev_ctx* comp, double* fmm_dev) {
  fmm_kernel<<<comp->G, kDiagNT, 0, comp->stream>>>(full->d.dg_n, full->d.dg_pos, full->d.dg_raw,
                                                    comp->d.ev_step, full->cap, comp->cfg.max_tokens,
                                                    static_cast<int>(comp->t), fmm_dev);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Missed mass without any allocation, for callers that cannot allocate
// (graph capture, serving loops): the per-group results are staged in a
// file-scope device array of kFmmScratchGroups doubles (32 KiB), which each
// GPU holds until the process ends.  Host code never passes the array's name
// to a kernel or a copy: it uses the device address that hipGetSymbolAddress
// returns, fetched once per device with that device current.
// ---------------------------------------------------------------------------
constexpr int kFmmScratchGroups = 4096;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) double scratch[kFmmScratchGroups];

static std::mutex g_scratch_mu;
static double* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on `device` (the current device).
static hipError_t scratch_address(int device, double** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[device] = static_cast<double*>(p);
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace kvev

using namespace kvev;

extern "C" kvev_status kvev_diag_fmm_noalloc(kvev_ctx* full, kvev_ctx* comp, double* fmm) {
  KVEV_LIVE(full);
  KVEV_LIVE(comp);
  if (kvev_status s = fmm_check(full, comp, fmm)) return s;
  if (comp->G > kFmmScratchGroups)
    return fail(comp, KVEV_ERANGE, "more groups than the missed-mass scratch holds (4096)");
  int cur = -1;
  KVEV_HIP(comp, hipGetDevice(&cur));
  if (cur != comp->device || cur != full->device)
    return fail(comp, KVEV_EINVAL, "call with the contexts' device current");
  double* dev = nullptr;
  KVEV_HIP(comp, scratch_address(cur, &dev));
  // the full context's step must be complete before its per-token values
  // are read on the compressed context's stream (no event: nothing allocated)
  KVEV_HIP(comp, hipStreamSynchronize(full->stream));
  // every group's entry g < G is written by its own block: nothing to clear
  KVEV_HIP(comp, launch_fmm(full, comp, dev));
  KVEV_HIP(comp, hipMemcpyAsync(fmm, dev, sizeof(double) * comp->G, hipMemcpyDeviceToHost, comp->stream));
  KVEV_HIP(comp, hipStreamSynchronize(comp->stream));
  return KVEV_OK;
}
