// Host side of the kvev C ABI: validation, allocation, step sequencing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "host_util.h"

using namespace kvev;

namespace {

std::string g_create_error;

void prof_drain(kvev_ctx* c) {
  for (auto& r : c->prof.pending) {
    hipEventSynchronize(r.b);
    float ms = 0.f;
    hipEventElapsedTime(&ms, r.a, r.b);
    bool found = false;
    for (auto& t : c->prof.totals)
      if (t.first == r.name) {
        t.second.first += ms;
        t.second.second += 1;
        found = true;
      }
    if (!found) c->prof.totals.push_back({r.name, {ms, 1}});
    c->prof.pool.push_back(r.a);
    c->prof.pool.push_back(r.b);
  }
  c->prof.pending.clear();
}

void free_all(kvev_ctx* c) {
  auto& d = c->d;
  if (c->pf_stream) {  // copies may still read the pinned pool
    hipStreamSynchronize(c->pf_stream);
    hipStreamDestroy(c->pf_stream);
    c->pf_stream = nullptr;
  }
  if (c->pf_done) hipEventDestroy(c->pf_done);
  c->pf_done = nullptr;
  if (c->dstage) hipFree(c->dstage);
  c->dstage = nullptr;
  void* ptrs[] = {d.kpool, d.vpool, d.ptab, d.pos, d.score, d.count, d.nextpos, d.logits,
                  d.part_ml, d.part_o, d.ml, d.mv_src, d.mv_dst, d.nmoves, d.errflag,
                  d.grpctr, d.blk_key, d.blk_slot, d.blk_sum, d.btab, d.nres,
                  d.bscore, d.btref, d.bres, d.bcnt, d.fstack, d.ftop, d.bmass, d.bbudget,
                  d.rd_ids, d.part_u, d.vnorm, d.part_vn, d.hole, d.dg_n, d.dg_pos, d.dg_raw,
                  d.dg_util, d.st_raw, d.st_util, d.st_kept, d.ev_step, d.dprev, d.dcnt, d.dacc,
                  d.ev_n, d.ev_blk, d.ev_page, d.hslot, d.sowner, d.rd_slots, d.ev_slot, d.oring, d.bpart,
                  d.gnew};
  for (void* p : ptrs)
    if (p) hipFree(p);
  if (c->hpool) hipHostFree(c->hpool);
  c->hpool = c->hpool_dev = nullptr;
  d = DevState{};
  tier_free(c);
  for (auto& r : c->prof.pending) {
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  for (auto e : c->prof.pool) hipEventDestroy(e);
  c->prof.pending.clear();
  c->prof.pool.clear();
}

// Token modes: group g's logical page i is the pool page g * maxpages + i,
// a fixed contiguous region per group (the page table holds this mapping
// from kvev_create on), so a step streams each group's pages in address
// order.  The pool holds maxpages pages for every group; a group fits
// `n_slots` slots when they need at most maxpages pages.
bool ensure_pages(kvev_ctx* c, int g, int64_t n_slots, std::vector<int>& upd) {
  (void)g;
  (void)upd;
  return (n_slots + c->PT - 1) / c->PT <= c->maxpages;
}

void release_pages(kvev_ctx* c, int g, int64_t n_slots) {
  (void)c;
  (void)g;
  (void)n_slots;
}

}  // namespace

// Tiered mode: windows of 32 positions, storage for every window the
// sequence can reach, chunk partials for two lists of them.
static kvev_status tier_create(const kvev_config& f, void* hip_stream, kvev_ctx** out) {
  kvev_ctx* c = new (std::nothrow) kvev_ctx();
  if (!c) {
    g_create_error = "out of host memory";
    return KVEV_EINVAL;
  }
  c->cfg = f;
  c->stream = static_cast<hipStream_t>(hip_stream);
  hipGetDevice(&c->device);
  c->G = f.n_kv_heads;
  c->HG = f.n_q_heads / f.n_kv_heads;
  c->cap = f.max_tokens;
  c->elem = 2;
  c->count.assign(c->G, 0);
  c->hole_in.assign(c->G, 0);
  c->prefilled.assign(1, 0);
  c->tier_mode = true;
  c->tw.W = f.window_tokens;
  c->tw.rope = f.rope_theta > 0.f;
  c->tw.kgroups = f.int2_key_groups == 1;
  c->tw.mat = c->tw.W == 8 || c->tw.rope || c->tw.kgroups;
  c->tw.NW = static_cast<int>((c->cap + c->tw.W - 1) / c->tw.W);
  c->tw.maxch = 2 * ((c->tw.NW + 7) / 8);
  const hipError_t e = tier_alloc(c);
  if (e != hipSuccess) {
    g_create_error = std::string("device allocation failed: ") + hipGetErrorString(e);
    free_all(c);
    delete c;
    return e == hipErrorOutOfMemory ? KVEV_ENOMEM : KVEV_EHIP;
  }
  *out = c;
  return KVEV_OK;
}

extern "C" {

void kvev_config_init(kvev_config* cfg) {
  if (!cfg) return;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->page_tokens = kPageTokens;
  cfg->policy = KVEV_EMA;
  cfg->alpha_new = 0.05f;
  cfg->refresh_interval = 1;
  cfg->dtype = KVEV_BF16;
  cfg->beta = 0.001f;
  cfg->decode_region = 4;
  cfg->access_tau_mult = 2.0f;
  cfg->window_tokens = kTierWin;
  cfg->rope_theta = 0.f;
}

kvev_status kvev_create(const kvev_config* cfg, void* hip_stream, kvev_ctx** out) {
  if (!cfg || !out) {
    g_create_error = "null argument";
    return KVEV_EINVAL;
  }
  *out = nullptr;
  const kvev_config& f = *cfg;
  auto bad = [&](const char* m) {
    g_create_error = m;
    return KVEV_EINVAL;
  };
  if (f.n_layers < 1 || f.n_q_heads < 1 || f.n_kv_heads < 1 || f.batch < 1)
    return bad("n_layers, n_q_heads, n_kv_heads and batch must be >= 1");
  if (f.n_q_heads % f.n_kv_heads != 0) return bad("n_q_heads must be a multiple of n_kv_heads");
  const int hg = f.n_q_heads / f.n_kv_heads;
  if (hg < 1 || hg > kMaxGroupSize) return bad("query group size must be 1..8");
  if ((f.policy == KVEV_LRFU_BLOCK || f.policy == KVEV_TIERED_INT2) && hg != 4)
    return bad("block and tiered modes: query group size must be 4");
  if (f.scorer & ~(KVEV_SCORE_VNORM | KVEV_SCORE_ENTROPY)) return bad("unknown scorer bits");
  if (f.route_interval < 0) return bad("route_interval must be >= 0");
  if (f.granularity != KVEV_PER_KV_HEAD && f.granularity != KVEV_PER_SEQUENCE)
    return bad("unknown granularity");
  if ((f.policy == KVEV_LRFU_BLOCK || f.policy == KVEV_TIERED_INT2) &&
      (f.scorer != 0 || f.granularity != KVEV_PER_KV_HEAD))
    return bad("scorer variants and granularity apply to the token policies only");
  if (f.revival_gap < 0) return bad("revival_gap must be >= 0");
  if (f.revival_gap > 0 && f.policy != KVEV_TIERED_INT2) return bad("revival_gap applies to the tiered mode only");
  if (f.offload_blocks < 0) return bad("offload_blocks must be >= 0");
  if (f.offload_blocks > 0 && f.policy != KVEV_LRFU_BLOCK) return bad("offload_blocks applies to the block mode only");
  if (f.prefetch_blocks < 0) return bad("prefetch_blocks must be >= 0");
  if (f.prefetch_blocks > 0 && f.offload_blocks <= 0) return bad("prefetch_blocks needs the host-offload tier");
  if (!std::isfinite(f.offload_min_score)) return bad("offload_min_score must be finite");
  if (f.attn_path < KVEV_ATTN_AUTO || f.attn_path > KVEV_ATTN_WHOLE) return bad("unknown attn_path");
  if (f.rope_theta != 0.f && f.policy != KVEV_TIERED_INT2) return bad("rope_theta applies to the tiered mode only");
  if (f.int2_key_groups != 0 && f.policy != KVEV_TIERED_INT2)
    return bad("int2_key_groups applies to the tiered mode only");
  if (f.int2_key_groups != 0 && f.int2_key_groups != 1) return bad("int2_key_groups must be 0 or 1");
  if (f.new_token_init != KVEV_NEW_TOKEN_ZERO && f.new_token_init != KVEV_NEW_TOKEN_MEAN)
    return bad("new_token_init must be 0 or 1");
  if (f.new_token_init != KVEV_NEW_TOKEN_ZERO && f.policy != KVEV_EMA && f.policy != KVEV_CUMULATIVE)
    return bad("new_token_init applies to the token policies only");
  if (f.evict_interval < 0) return bad("evict_interval must be >= 0");
  if (f.evict_interval > 1 && f.policy != KVEV_EMA && f.policy != KVEV_CUMULATIVE)
    return bad("evict_interval applies to the token policies only");
  if (f.evict_interval > 1 && f.diag_topk > 0) return bad("diagnostics need evict_interval 0 or 1");
  if (f.diag_topk < 0) return bad("diag_topk must be >= 0");
  if (f.diag_topk > 0 && f.policy != KVEV_EMA && f.policy != KVEV_CUMULATIVE)
    return bad("diagnostics apply to the token policies only");
  if (f.diag_topk > 0 && (f.granularity != KVEV_PER_KV_HEAD || f.refresh_interval != 1 || f.score_free != 0))
    return bad("diagnostics need per-KV-head granularity, refresh_interval 1 and score_free 0");
  if (f.head_dim != 64 && f.head_dim != 128) return bad("head_dim must be 64 or 128");
  if (f.dtype != KVEV_F32 && f.dtype != KVEV_BF16) return bad("dtype must be KVEV_F32 or KVEV_BF16");
  if (f.page_tokens != kPageTokens) return bad("page_tokens must be 16");
  if (f.policy != KVEV_EMA && f.policy != KVEV_CUMULATIVE && f.policy != KVEV_LRFU_BLOCK &&
      f.policy != KVEV_TIERED_INT2)
    return bad("unsupported policy");
  const bool tiered = f.policy == KVEV_TIERED_INT2;
  if (tiered) {
    if (f.dtype != KVEV_BF16 || f.head_dim != kTierD) return bad("tiered mode: bf16 and head_dim 128 only");
    if (f.batch != 1) return bad("tiered mode: batch must be 1");
    if (f.window_tokens != 8 && f.window_tokens != 32) return bad("tiered mode: window_tokens must be 8 or 32");
    if (f.fp_windows < 0 || f.int2_windows < 0) return bad("tiered mode: tier capacities must be >= 0");
    if (f.max_tokens > static_cast<int64_t>(kTierMaxWin) * f.window_tokens)
      return bad("tiered mode: max_tokens must be <= 12288 windows");
    if (!(f.rope_theta >= 0.f) || !std::isfinite(f.rope_theta)) return bad("rope_theta must be finite and >= 0");
    if (f.refresh_interval != 1 || f.score_free != 0)
      return bad("tiered mode: refresh_interval must be 1 and score_free 0");
    if (f.n_sink < 0 || f.n_recent < 0) return bad("n_sink and n_recent must be >= 0");
    if (f.n_layers > 64) return bad("n_layers must be <= 64");
    if (f.max_tokens < 2) return bad("max_tokens out of range");
  }
  if ((f.policy == KVEV_EMA || f.policy == KVEV_LRFU_BLOCK) && !(f.alpha_new > 0.f && f.alpha_new <= 1.f))
    return bad("alpha_new must be in (0, 1]");
  const bool block = f.policy == KVEV_LRFU_BLOCK;
  if (block) {
    if (f.max_tokens > static_cast<int64_t>(kMaxBlockEntries) * kPageTokens)
      return bad("block mode: max_tokens must be <= 65536");
    if (f.n_sink != 0 || f.n_recent != 0) return bad("block mode: n_sink and n_recent must be 0");
    if (f.refresh_interval != 1 || f.score_free != 0)
      return bad("block mode: refresh_interval must be 1 and score_free 0");
    if (!(f.beta >= 0.f) || !std::isfinite(f.beta)) return bad("block mode: beta must be finite and >= 0");
    if (f.decode_region < 0 || f.decode_region >= kRegions) return bad("block mode: decode_region out of range");
    if ((f.pinned_region_mask >> f.decode_region) & 1u) return bad("block mode: decode_region is pinned");
    if (f.pinned_region_mask >> kRegions) return bad("block mode: pinned_region_mask has bits above 7");
    if (!(f.access_tau_mult > 0.f) || !std::isfinite(f.access_tau_mult))
      return bad("block mode: access_tau_mult must be > 0");
    if (f.n_kv_heads > 64 || f.n_layers * f.n_kv_heads > 1024)
      return bad("block mode: at most 64 KV heads and 1024 (layer, KV head) pairs");
  }
  if (tiered) return tier_create(f, hip_stream, out);
  if (f.refresh_interval < 1) return bad("refresh_interval must be >= 1");
  if (f.n_sink < 0 || f.n_recent < 0) return bad("n_sink and n_recent must be >= 0");
  if (f.budget < 1) return bad("budget must be >= 1");
  if (block && f.budget > kMaxBlockEntries) return bad("block mode: budget must be <= 4096 blocks");
  if (f.n_sink + f.n_recent > f.budget) return bad("n_sink + n_recent exceeds the budget");
  if (f.max_tokens < 2 || f.max_tokens > (1ll << 30)) return bad("max_tokens out of range");
  if (f.n_layers > 64) return bad("n_layers must be <= 64");
  {
    // the post kernel stages per-layer statistics and one layer's split
    // weights in LDS: (3 L HG + HG S + 65 L) floats must fit 56 KiB (the
    // rest of the 64 KiB is the kernels' static arrays, < 8 KiB)
    const int64_t S = (f.max_tokens + kAttnChunk - 1) / kAttnChunk;
    const int64_t lds = (3ll * f.n_layers * hg + hg * S + 65ll * f.n_layers) * 4;
    if (!block && lds > 57344) return bad("max_tokens too large for this layer count and group size");
    if (f.granularity == KVEV_PER_SEQUENCE &&
        pool_post_shm(f.n_layers, f.n_q_heads, f.n_kv_heads, S) * 4 > 57344)
      return bad("per-sequence granularity: too many (layer, query head) pairs or max_tokens too large");
  }

  kvev_ctx* c = new (std::nothrow) kvev_ctx();
  if (!c) return bad("out of host memory");
  c->cfg = f;
  c->stream = static_cast<hipStream_t>(hip_stream);
  hipGetDevice(&c->device);
  if (hipDeviceGetAttribute(&c->max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, c->device) != hipSuccess)
    c->max_lds = 65536;
  c->G = f.batch * f.n_kv_heads;
  c->HG = f.n_q_heads / f.n_kv_heads;
  c->cap = f.max_tokens;
  c->maxpages = static_cast<int>((c->cap + c->PT - 1) / c->PT);
  c->P = static_cast<int64_t>(c->G) * c->maxpages;
  c->max_splits = static_cast<int>((c->cap + kAttnChunk - 1) / kAttnChunk);
  c->pooled = f.granularity == KVEV_PER_SEQUENCE;
  c->max_post_blocks = c->pooled ? std::max(static_cast<int>((c->cap + kPoolTokens - 1) / kPoolTokens),
                                            f.n_layers * f.n_kv_heads)
                                 : std::max(static_cast<int>((c->cap + 63) / 64), f.n_layers);
  c->elem = f.dtype == KVEV_BF16 ? 2 : 4;
  c->count.assign(c->G, 0);
  c->hole_in.assign(c->G, 0);
  c->prefilled.assign(f.batch, 0);
  c->seq_next.assign(f.batch, 0);
  if (c->pooled) c->pool_import.assign(f.batch, {});
  c->block_mode = block;
  if (block) {
    c->maxblk = c->maxpages;
    for (int r = 0; r < kRegions; ++r) {
      const double hl = f.region_half_life[r];
      c->lam[r] = (hl > 0.0 && std::isfinite(hl)) ? static_cast<float>(std::log(2.0) / hl) : 0.f;
    }
    c->nres.assign(f.batch, 0);
    c->npos.assign(f.batch, 0);
    c->bbudget.assign(f.batch, static_cast<int>(f.budget));
    c->npinned.assign(f.batch, 0);
  }

  auto& d = c->d;
  const int64_t L = f.n_layers, D = f.head_dim, G = c->G, HG = c->HG;
  const size_t pool_bytes = static_cast<size_t>(L) * c->P * c->PT * D * c->elem;
  hipError_t e = hipSuccess;
  auto A = [&](hipError_t r) {
    if (e == hipSuccess && r != hipSuccess) e = r;
  };
  A(hipMalloc(&d.kpool, pool_bytes));
  A(hipMalloc(&d.vpool, pool_bytes));
  A(dalloc(&d.ptab, static_cast<size_t>(G) * c->maxpages));
  A(dalloc(&d.pos, static_cast<size_t>(G) * c->cap));
  A(dalloc(&d.score, static_cast<size_t>(G) * c->cap));
  A(dalloc(&d.count, G));
  if (!block) A(dalloc(&d.hole, G));  // token modes: the free slot the next token takes
  A(dalloc(&d.nextpos, G));
  // the logit stride is the step's slot count rounded up to 16, which can
  // exceed a capacity that is not a multiple of 16.  The block mode's
  // matrix-core attention writes per-block sums (bpart) instead of logits.
  const bool block_sums = block && f.dtype == KVEV_BF16 && f.head_dim == 128;
  if (!block_sums) A(dalloc(&d.logits, static_cast<size_t>(G) * L * ((c->cap + 15) / 16 * 16) * HG));
  A(dalloc(&d.part_ml, static_cast<size_t>(L) * G * c->max_splits * HG * 2));
  A(dalloc(&d.part_o, static_cast<size_t>(L) * G * c->max_splits * HG * D));
  A(dalloc(&d.ml, static_cast<size_t>(L) * G * HG * 2));
  if (f.scorer & KVEV_SCORE_ENTROPY) A(dalloc(&d.part_u, static_cast<size_t>(L) * G * c->max_splits * HG));
  if (f.scorer & KVEV_SCORE_VNORM) {
    A(dalloc(&d.vnorm, static_cast<size_t>(G) * L * ((c->cap + 15) / 16 * 16)));
    A(dalloc(&d.part_vn, static_cast<size_t>(L) * G * c->max_splits));
  }
  A(dalloc(&d.mv_src, static_cast<size_t>(G) * c->cap));
  A(dalloc(&d.mv_dst, static_cast<size_t>(G) * c->cap));
  A(dalloc(&d.nmoves, G));
  A(dalloc(&d.errflag, 1));
  A(dalloc(&d.grpctr, G));
  A(dalloc(&d.blk_key, static_cast<size_t>(G) * c->max_post_blocks));
  A(dalloc(&d.blk_slot, static_cast<size_t>(G) * c->max_post_blocks));
  A(dalloc(&d.blk_sum, static_cast<size_t>(G) * c->max_post_blocks));
  A(dalloc(&d.gnew, G));
  const bool diag = f.diag_topk > 0;
  const size_t npos = static_cast<size_t>(G) * f.max_tokens;  // per-position stamps
  if (diag) {
    A(dalloc(&d.dg_n, G));
    A(dalloc(&d.dg_pos, static_cast<size_t>(G) * c->cap));
    A(dalloc(&d.dg_raw, static_cast<size_t>(G) * c->cap));
    A(dalloc(&d.dg_util, static_cast<size_t>(G) * c->cap));
    A(dalloc(&d.st_raw, npos));
    A(dalloc(&d.st_util, npos));
    A(dalloc(&d.st_kept, npos));
    A(dalloc(&d.ev_step, npos));
    A(dalloc(&d.dprev, static_cast<size_t>(G) * 4));
    A(dalloc(&d.dcnt, static_cast<size_t>(G) * kDiagCounts));
    A(dalloc(&d.dacc, static_cast<size_t>(G) * kDiagAcc));
  }
  if (block) {
    const size_t Bs = f.batch;
    A(dalloc(&d.btab, Bs * c->maxpages));
    A(dalloc(&d.nres, Bs));
    A(dalloc(&d.bscore, Bs * c->maxblk));
    A(dalloc(&d.btref, Bs * c->maxblk));
    A(dalloc(&d.bres, Bs * c->maxblk));
    // the matrix-core attention writes per-block sums instead of per-slot logits
    if (block_sums) A(dalloc(&d.bpart, static_cast<size_t>(L) * G * c->maxpages * HG));
    A(dalloc(&d.bcnt, Bs * c->maxblk * kRegions));
    A(dalloc(&d.fstack, static_cast<size_t>(G) * c->maxpages));
    A(dalloc(&d.ftop, G));
    A(dalloc(&d.bmass, Bs * c->maxpages));
    A(dalloc(&d.bbudget, Bs));
    A(dalloc(&d.rd_ids, c->maxpages));
    if (f.offload_blocks > 0) {
      A(dalloc(&d.ev_n, Bs));
      A(dalloc(&d.ev_blk, Bs * c->maxpages));
      A(dalloc(&d.ev_page, static_cast<size_t>(G) * c->maxpages));
      A(dalloc(&d.hslot, Bs * c->maxblk));
      A(dalloc(&d.sowner, static_cast<size_t>(f.offload_blocks)));
      A(dalloc(&d.rd_slots, c->maxpages));
      A(dalloc(&d.ev_slot, Bs * c->maxpages));
      A(dalloc(&d.oring, 2));
      // K and V pages of every layer and KV head per slot
      const size_t slot_bytes = 2ull * L * f.n_kv_heads * c->PT * D * c->elem;
      A(hipHostMalloc(&c->hpool, slot_bytes * f.offload_blocks, hipHostMallocDefault));
      if (c->hpool) A(hipHostGetDevicePointer(&c->hpool_dev, c->hpool, 0));
      if (f.prefetch_blocks > 0) {
        A(hipMalloc(&c->dstage, slot_bytes * f.prefetch_blocks));
        A(hipStreamCreateWithFlags(&c->pf_stream, hipStreamNonBlocking));
        A(hipEventCreateWithFlags(&c->pf_done, hipEventDisableTiming));
        c->pf_key.assign(f.prefetch_blocks, -1);
        c->pf_src.assign(f.prefetch_blocks, -1);
      }
    }
  }
  if (e != hipSuccess) {
    g_create_error = std::string("device allocation failed: ") + hipGetErrorString(e);
    free_all(c);
    delete c;
    return e == hipErrorOutOfMemory ? KVEV_ENOMEM : KVEV_EHIP;
  }
  // zero everything so unused slots hold finite values
  A(hipMemsetAsync(d.kpool, 0, pool_bytes, c->stream));
  A(hipMemsetAsync(d.vpool, 0, pool_bytes, c->stream));
  if (block) {
    A(hipMemsetAsync(d.ptab, 0, sizeof(int) * G * c->maxpages, c->stream));
  } else {
    // token modes: the fixed mapping of logical page i of group g to pool page g * maxpages + i
    std::vector<int> idmap(static_cast<size_t>(G) * c->maxpages);
    for (size_t i = 0; i < idmap.size(); ++i) idmap[i] = static_cast<int>(i);
    A(hipMemcpy(d.ptab, idmap.data(), sizeof(int) * idmap.size(), hipMemcpyHostToDevice));
  }
  A(hipMemsetAsync(d.score, 0, sizeof(float) * G * c->cap, c->stream));
  A(hipMemsetAsync(d.pos, 0, sizeof(int) * G * c->cap, c->stream));
  A(hipMemsetAsync(d.count, 0, sizeof(int) * G, c->stream));
  if (d.hole) A(hipMemsetAsync(d.hole, 0, sizeof(int) * G, c->stream));
  A(hipMemsetAsync(d.nextpos, 0, sizeof(int) * G, c->stream));
  A(hipMemsetAsync(d.nmoves, 0, sizeof(int) * G, c->stream));
  A(hipMemsetAsync(d.errflag, 0, sizeof(int), c->stream));
  A(hipMemsetAsync(d.grpctr, 0, sizeof(unsigned) * G, c->stream));
  A(hipMemsetAsync(d.mv_src, 0, sizeof(int) * G * c->cap, c->stream));
  A(hipMemsetAsync(d.mv_dst, 0, sizeof(int) * G * c->cap, c->stream));
  if (diag) {
    A(hipMemsetAsync(d.dg_n, 0, sizeof(int) * G, c->stream));
    A(hipMemsetAsync(d.st_raw, 0, sizeof(int) * npos, c->stream));
    A(hipMemsetAsync(d.st_util, 0, sizeof(int) * npos, c->stream));
    A(hipMemsetAsync(d.st_kept, 0, sizeof(int) * npos, c->stream));
    A(hipMemsetAsync(d.ev_step, 0, sizeof(int) * npos, c->stream));
    A(hipMemsetAsync(d.dprev, 0, sizeof(int) * G * 4, c->stream));
    A(hipMemsetAsync(d.dcnt, 0, sizeof(int) * G * kDiagCounts, c->stream));
    A(hipMemsetAsync(d.dacc, 0, sizeof(double) * G * kDiagAcc, c->stream));
  }
  if (block) {
    const size_t Bs = f.batch;
    A(hipMemsetAsync(d.btab, 0, sizeof(int) * Bs * c->maxpages, c->stream));
    A(hipMemsetAsync(d.nres, 0, sizeof(int) * Bs, c->stream));
    A(hipMemsetAsync(d.bscore, 0, sizeof(float) * Bs * c->maxblk, c->stream));
    A(hipMemsetAsync(d.btref, 0, sizeof(int) * Bs * c->maxblk, c->stream));
    A(hipMemsetAsync(d.bres, 0, sizeof(int) * Bs * c->maxblk, c->stream));
    A(hipMemsetAsync(d.bcnt, 0, Bs * c->maxblk * kRegions, c->stream));
    A(hipMemsetAsync(d.bmass, 0, sizeof(float) * Bs * c->maxpages, c->stream));
    A(hipMemsetAsync(d.rd_ids, 0, sizeof(int) * c->maxpages, c->stream));
    if (f.offload_blocks > 0) {
      A(hipMemsetAsync(d.ev_n, 0, sizeof(int) * Bs, c->stream));
      A(hipMemsetAsync(d.ev_blk, 0, sizeof(int) * Bs * c->maxpages, c->stream));
      A(hipMemsetAsync(d.ev_page, 0, sizeof(int) * G * c->maxpages, c->stream));
      A(hipMemsetAsync(d.hslot, 0xff, sizeof(int) * Bs * c->maxblk, c->stream));  // -1
      A(hipMemsetAsync(d.sowner, 0xff, sizeof(int) * f.offload_blocks, c->stream));
      A(hipMemsetAsync(d.rd_slots, 0, sizeof(int) * c->maxpages, c->stream));
      A(hipMemsetAsync(d.ev_slot, 0xff, sizeof(int) * Bs * c->maxpages, c->stream));
      A(hipMemsetAsync(d.oring, 0, sizeof(int) * 2, c->stream));
    }
    std::vector<int> stack(static_cast<size_t>(G) * c->maxpages), top(G, c->maxpages);
    for (int64_t g = 0; g < G; ++g)
      for (int i = 0; i < c->maxpages; ++i)  // popped from the top: lowest page first
        stack[g * c->maxpages + i] = static_cast<int>(g * c->maxpages + (c->maxpages - 1 - i));
    std::vector<int> bud(Bs, static_cast<int>(f.budget));
    A(hipMemcpyAsync(d.fstack, stack.data(), sizeof(int) * stack.size(), hipMemcpyHostToDevice, c->stream));
    A(hipMemcpyAsync(d.ftop, top.data(), sizeof(int) * G, hipMemcpyHostToDevice, c->stream));
    A(hipMemcpyAsync(d.bbudget, bud.data(), sizeof(int) * Bs, hipMemcpyHostToDevice, c->stream));
    A(hipStreamSynchronize(c->stream));  // host vectors above are local
  }
  A(hipStreamSynchronize(c->stream));
  if (e != hipSuccess) {
    g_create_error = std::string("device initialisation failed: ") + hipGetErrorString(e);
    free_all(c);
    delete c;
    return KVEV_EHIP;
  }
  *out = c;
  return KVEV_OK;
}

kvev_status kvev_destroy(kvev_ctx* c) {
  if (!c) return KVEV_OK;
  hipStreamSynchronize(c->stream);
  free_all(c);
  delete c;
  return KVEV_OK;
}

// Block mode: install a sequence's block table, page tables, free-page
// stacks and block state for blocks 0..nb-1 of which `resident` are cached
// (ascending ids, the last one the block holding the newest token), then
// scatter the resident tokens' K/V.  Shared by prefill and import.
static kvev_status block_install(kvev_ctx* c, int seq, int64_t npos, const std::vector<int>& resident,
                                 const float* score, const int32_t* tref, const void* k,
                                 const void* v) {
  const int Hkv = c->cfg.n_kv_heads;
  const int nb = static_cast<int>((npos + c->PT - 1) / c->PT);
  const int nr = static_cast<int>(resident.size());
  const int fill = static_cast<int>(npos - static_cast<int64_t>(c->PT) * (nb - 1));
  const int64_t cnt = static_cast<int64_t>(c->PT) * (nr - 1) + fill;
  std::vector<int> btab(resident), top(Hkv, c->maxpages - nr);
  std::vector<int> ptab(static_cast<size_t>(Hkv) * c->maxpages), stack(ptab.size());
  for (int h = 0; h < Hkv; ++h) {
    const int g = seq * Hkv + h;
    for (int i = 0; i < c->maxpages; ++i) {
      const int page = g * c->maxpages + i;
      if (i < nr) ptab[static_cast<size_t>(h) * c->maxpages + i] = page;
      else stack[static_cast<size_t>(h) * c->maxpages + (c->maxpages - 1 - i)] = page;
    }
  }
  std::vector<float> bscore(c->maxblk, 0.f);
  std::vector<int> btref(c->maxblk, 0), bres(c->maxblk, 0), posv(cnt);
  for (int j = 0; j < nb; ++j) {
    bscore[j] = score ? score[j] : 0.f;
    btref[j] = tref ? tref[j] : 0;
  }
  for (int i = 0; i < nr; ++i) {
    bres[resident[i]] = 1;
    const int len = i == nr - 1 ? fill : c->PT;
    for (int r = 0; r < len; ++r) posv[static_cast<size_t>(i) * c->PT + r] = resident[i] * c->PT + r;
  }
  const int64_t brow = static_cast<int64_t>(seq) * c->maxpages, bblk = static_cast<int64_t>(seq) * c->maxblk;
  const int nr32 = nr, cnt32 = static_cast<int>(cnt), np32 = static_cast<int>(npos);
  auto H2D = [&](void* dst, const void* src, size_t bytes) {
    return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, c->stream);
  };
  KVEV_HIP(c, H2D(c->d.btab + brow, btab.data(), sizeof(int) * nr));
  KVEV_HIP(c, H2D(c->d.nres + seq, &nr32, sizeof(int)));
  KVEV_HIP(c, H2D(c->d.bscore + bblk, bscore.data(), sizeof(float) * c->maxblk));
  KVEV_HIP(c, H2D(c->d.btref + bblk, btref.data(), sizeof(int) * c->maxblk));
  KVEV_HIP(c, H2D(c->d.bres + bblk, bres.data(), sizeof(int) * c->maxblk));
  for (int h = 0; h < Hkv; ++h) {
    const int g = seq * Hkv + h;
    KVEV_HIP(c, H2D(c->d.ptab + static_cast<int64_t>(g) * c->maxpages,
                    ptab.data() + static_cast<size_t>(h) * c->maxpages, sizeof(int) * c->maxpages));
    KVEV_HIP(c, H2D(c->d.fstack + static_cast<int64_t>(g) * c->maxpages,
                    stack.data() + static_cast<size_t>(h) * c->maxpages, sizeof(int) * c->maxpages));
    KVEV_HIP(c, H2D(c->d.ftop + g, &top[h], sizeof(int)));
    KVEV_HIP(c, H2D(c->d.pos + static_cast<int64_t>(g) * c->cap, posv.data(), sizeof(int) * cnt));
    KVEV_HIP(c, H2D(c->d.count + g, &cnt32, sizeof(int)));
    KVEV_HIP(c, H2D(c->d.nextpos + g, &np32, sizeof(int)));
  }
  KVEV_HIP(c, launch_prefill_scatter(c, seq, k, v, cnt));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));  // host vectors above are local
  for (int h = 0; h < Hkv; ++h) c->count[seq * Hkv + h] = cnt;
  c->nres[seq] = nr;
  c->npos[seq] = npos;
  return KVEV_OK;
}

static kvev_status block_prefill(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n,
                                 const uint8_t* labels) {
  const int nb = static_cast<int>((n + c->PT - 1) / c->PT);
  std::vector<uint8_t> cnt8(static_cast<size_t>(c->maxblk) * kRegions, 0);
  int pinned = 0;
  for (int j = 0; j < nb; ++j) {
    bool pin = false;
    for (int64_t i = static_cast<int64_t>(j) * c->PT; i < std::min<int64_t>(n, (j + 1) * c->PT); ++i) {
      const int r = labels ? labels[i] : c->cfg.decode_region;
      if (r < 0 || r >= kRegions) return fail(c, KVEV_EINVAL, "region label out of range");
      cnt8[static_cast<size_t>(j) * kRegions + r] += 1;
      if ((c->cfg.pinned_region_mask >> r) & 1u) pin = true;
    }
    pinned += pin;
  }
  KVEV_HIP(c, hipMemcpyAsync(c->d.bcnt + static_cast<int64_t>(seq) * c->maxblk * kRegions, cnt8.data(),
                             cnt8.size(), hipMemcpyHostToDevice, c->stream));
  std::vector<int> resident(nb);
  for (int j = 0; j < nb; ++j) resident[j] = j;
  if (kvev_status s = block_install(c, seq, n, resident, nullptr, nullptr, k, v)) return s;
  c->npinned[seq] = pinned;
  c->prefilled[seq] = 1;
  return KVEV_OK;
}

kvev_status kvev_prefill(kvev_ctx* c, int32_t seq, const void* k, const void* v, int64_t n,
                         const uint8_t* labels) {
  KVEV_LIVE(c);
  if (seq < 0 || seq >= c->cfg.batch) return fail(c, KVEV_EINVAL, "sequence index out of range");
  if (!k || !v) return fail(c, KVEV_EINVAL, "null k or v");
  if (c->t > 0) return fail(c, KVEV_ESTATE, "prefill after the first decode step");
  if (n < 1 || n + 1 > c->cap) return fail(c, KVEV_EINVAL, "n_tokens out of range for max_tokens");
  if (c->block_mode) return block_prefill(c, seq, k, v, n, labels);
  if (c->tier_mode) return tier_prefill(c, seq, k, v, n);
  const int Hkv = c->cfg.n_kv_heads;
  std::vector<int> upd;
  for (int h = 0; h < Hkv; ++h) {
    const int g = seq * Hkv + h;
    release_pages(c, g, 0);
  }
  for (int h = 0; h < Hkv; ++h)
    if (!ensure_pages(c, seq * Hkv + h, n, upd)) return fail(c, KVEV_ENOMEM, "page pool exhausted");
  KVEV_HIP(c, launch_prefill_scatter(c, seq, k, v, n));
  // positions 0..n-1, utilities 0, count n, next position n
  std::vector<int> posv(n);
  for (int64_t i = 0; i < n; ++i) posv[i] = static_cast<int>(i);
  for (int h = 0; h < Hkv; ++h) {
    const int g = seq * Hkv + h;
    KVEV_HIP(c, hipMemcpyAsync(c->d.pos + static_cast<int64_t>(g) * c->cap, posv.data(),
                               sizeof(int) * n, hipMemcpyHostToDevice, c->stream));
    KVEV_HIP(c, hipMemsetAsync(c->d.score + static_cast<int64_t>(g) * c->cap, 0,
                               sizeof(float) * n, c->stream));
    const int cnt = static_cast<int>(n);
    KVEV_HIP(c, hipMemcpyAsync(c->d.count + g, &cnt, sizeof(int), hipMemcpyHostToDevice, c->stream));
    KVEV_HIP(c, hipMemcpyAsync(c->d.hole + g, &cnt, sizeof(int), hipMemcpyHostToDevice, c->stream));
    KVEV_HIP(c, hipMemcpyAsync(c->d.nextpos + g, &cnt, sizeof(int), hipMemcpyHostToDevice, c->stream));
    KVEV_HIP(c, hipStreamSynchronize(c->stream));  // host buffers above are stack-local
    c->count[g] = n;
  }
  c->prefilled[seq] = 1;
  c->seq_next[seq] = n;
  return KVEV_OK;
}

// Block mode: the per-sequence budget a selection uses, checked against the
// blocks it must keep (pinned by region labels, plus the block being filled).
static kvev_status block_budget(kvev_ctx* c, int b, int64_t override_budget, int* B) {
  const int64_t bb = override_budget > 0 ? override_budget : c->bbudget[b];
  if (bb > kMaxBlockEntries) return fail(c, KVEV_EINVAL, "budget out of range");
  if (bb < c->npinned[b] + 1) return fail(c, KVEV_EINVAL, "budget below the pinned blocks of a sequence");
  *B = static_cast<int>(bb);
  return KVEV_OK;
}

static int block_fill(const kvev_ctx* c, int64_t npos) {
  return static_cast<int>(npos - static_cast<int64_t>(c->PT) * ((npos - 1) / c->PT));
}

// Block mode step: open (slot and block of the new token), attention,
// split merge, block mass, policy (score and clock update; selection and
// table compaction when do_select).
// Host-offload tier: after a selection that evicted ev[b] blocks of each
// sequence, copy them into the pool's next ring slots (the last
// offload_blocks of them when more were evicted).
static hipError_t offload_evicted(kvev_ctx* c, const std::vector<int>& ev) {
  int E = 0, kmax = 0;
  for (int k : ev) {
    E += k;
    kmax = std::max(kmax, k);
  }
  if (E == 0) return hipSuccess;
  if (c->pf_pending) {  // prefetch copies still read the slots about to be written
    if (hipError_t w = hipStreamWaitEvent(c->stream, c->pf_done, 0)) return w;
    c->pf_pending = false;
  }
  return launch_offload(c, kmax, E);
}

// The whole-cache attention over the block tables (bf16, head_dim 128; the
// block mode has no scorer variants): under the same rule as the token
// modes' (at least 224 (group, layer) pairs unless attn_path asks for it,
// the step's slots within its bound and its LDS).
static bool block_whole_attention(const kvev_ctx* c, int64_t n_max) {
  const auto& f = c->cfg;
  if (f.attn_path == KVEV_ATTN_SPLIT || !c->d.bpart || f.scorer != 0) return false;
  if (n_max > kSeqMaxSlots || seq_attn_lds_bytes(c->HG, n_max, true, true) + 1024 > c->max_lds) return false;
  return f.attn_path == KVEV_ATTN_WHOLE || static_cast<int64_t>(c->G) * f.n_layers >= 224;
}

static kvev_status block_step(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                              float* out, bool do_select, int64_t override_budget) {
  if (!q || !k_new || !v_new || !out) return fail(c, KVEV_EINVAL, "null argument");
  const int Bsz = c->cfg.batch, Hkv = c->cfg.n_kv_heads;
  std::vector<int> Bs(Bsz, 0);
  int64_t n_max = 0;
  for (int b = 0; b < Bsz; ++b) {
    if (!c->prefilled[b]) return fail(c, KVEV_ESTATE, "a sequence has no prefill");
    if (c->npos[b] + 1 > c->cap) return fail(c, KVEV_ESTATE, "position capacity exhausted");
    if (do_select)
      if (kvev_status s = block_budget(c, b, override_budget, &Bs[b])) return s;
    const bool opens = c->npos[b] % c->PT == 0;
    if (opens && c->nres[b] + 1 > c->maxpages) return fail(c, KVEV_ESTATE, "block table full");
    n_max = std::max(n_max, c->count[b * Hkv] + 1);
  }
  const int64_t t = c->t + 1;
  c->lstride = (n_max + 15) / 16 * 16;
  const int nm = static_cast<int>(n_max);
  // every launch of the step times itself from its own dispatch (kvev_profile_*)
  KVEV_HIP(c, launch_block_open(c, nm, static_cast<int>(t)));
  if (block_whole_attention(c, n_max)) {
    // one workgroup per (group, layer): outputs and entry masses directly
    KVEV_HIP(c, launch_attention_seq_blocks(c, q, k_new, v_new, out, nm));
    KVEV_HIP(c, launch_block_entry_mass(c, nm));
  } else {
    KVEV_HIP(c, launch_attention(c, q, k_new, v_new, nm, 1, "attn"));
    KVEV_HIP(c, launch_block_merge(c, out, nm));
    KVEV_HIP(c, launch_block_mass(c, nm));
  }
  KVEV_HIP(c, launch_block_policy(c, static_cast<int>(t), 1, do_select ? 1 : 0, 1,
                                  static_cast<int>(override_budget > 0 ? override_budget : 0)));
  if (c->cfg.offload_blocks > 0 && do_select) {
    std::vector<int> ev(Bsz, 0);
    for (int b = 0; b < Bsz; ++b) {
      const int open = c->nres[b] + (c->npos[b] % c->PT == 0 ? 1 : 0);
      ev[b] = std::max(0, open - Bs[b]);
    }
    KVEV_HIP(c, offload_evicted(c, ev));
  }
  for (int b = 0; b < Bsz; ++b) {
    if (c->npos[b] % c->PT == 0) c->nres[b] += 1;
    c->npos[b] += 1;
    if (do_select && c->nres[b] > Bs[b]) c->nres[b] = Bs[b];
    const int64_t cnt = static_cast<int64_t>(c->PT) * (c->nres[b] - 1) + block_fill(c, c->npos[b]);
    for (int h = 0; h < Hkv; ++h) c->count[b * Hkv + h] = cnt;
  }
  c->t = t;
  return KVEV_OK;
}

static kvev_status block_evict(kvev_ctx* c, int64_t override_budget) {
  const int Bsz = c->cfg.batch, Hkv = c->cfg.n_kv_heads;
  std::vector<int> Bs(Bsz, 0);
  bool any = false;
  for (int b = 0; b < Bsz; ++b) {
    if (kvev_status s = block_budget(c, b, override_budget, &Bs[b])) return s;
    any = any || c->nres[b] > Bs[b];
  }
  if (!any) return KVEV_OK;
  KVEV_HIP(c, launch_block_policy(c, static_cast<int>(c->t), 0, 1, 0,
                                  static_cast<int>(override_budget > 0 ? override_budget : 0)));
  if (c->cfg.offload_blocks > 0) {
    std::vector<int> ev(Bsz, 0);
    for (int b = 0; b < Bsz; ++b) ev[b] = std::max(0, c->nres[b] - Bs[b]);
    KVEV_HIP(c, offload_evicted(c, ev));
  }
  for (int b = 0; b < Bsz; ++b) {
    if (c->nres[b] > Bs[b]) c->nres[b] = Bs[b];
    const int64_t cnt = static_cast<int64_t>(c->PT) * (c->nres[b] - 1) + block_fill(c, c->npos[b]);
    for (int h = 0; h < Hkv; ++h) c->count[b * Hkv + h] = cnt;
  }
  return KVEV_OK;
}

// Shared by kvev_decode_step and kvev_step: pages for the new token, the
// attention launch and the post launch.
// Per-sequence granularity: a sequence whose KV heads were only partly
// imported (kvev_import_group) holds inconsistent slots.
static kvev_status check_pool_import(kvev_ctx* c) {
  for (const auto& pi : c->pool_import)
    if (!pi.done.empty())
      return fail(c, KVEV_ESTATE, "per-sequence granularity: a sequence's KV heads were only partly imported");
  return KVEV_OK;
}

// The whole-cache attention kernel applies to the token policies with bf16,
// head_dim 128 and the attention scorer (per KV head or per sequence: the
// fold kernel then pools a sequence's groups), when the step's slots fit
// its bound and its LDS (the logits of an observation step, the per-wave
// outputs and about 1 KiB of fixed arrays).
static bool whole_cache_attention(const kvev_ctx* c, int64_t n_max) {
  const auto& f = c->cfg;
  if (f.attn_path == KVEV_ATTN_SPLIT || c->block_mode || c->tier_mode) return false;
  if (f.dtype != KVEV_BF16 || f.head_dim != 128 || f.scorer != 0) return false;
  if (n_max > kSeqMaxSlots || seq_attn_lds_bytes(c->HG, n_max, true, false) + 1024 > c->max_lds) return false;
  return f.attn_path == KVEV_ATTN_WHOLE || static_cast<int64_t>(c->G) * f.n_layers >= 224;
}

static kvev_status run_step(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                            float* out, bool do_select, int64_t B) {
  if (!q || !k_new || !v_new || !out) return fail(c, KVEV_EINVAL, "null argument");
  if (kvev_status s = check_pool_import(c)) return s;
  for (int b = 0; b < c->cfg.batch; ++b)
    if (!c->prefilled[b]) return fail(c, KVEV_ESTATE, "a sequence has no prefill");
  const int64_t t = c->t + 1;
  const bool refresh = c->cfg.score_free ? (t == 1) : ((t - 1) % c->cfg.refresh_interval == 0);
  const bool diag = c->cfg.diag_topk > 0;
  if (diag)  // the diagnostics stamp positions below max_tokens
    for (int b = 0; b < c->cfg.batch; ++b)
      if (c->seq_next[b] >= c->cfg.max_tokens)
        return fail(c, KVEV_ESTATE, "diagnostics: positions would reach max_tokens");
  auto& upd = c->ptab_upd;
  upd.clear();
  int64_t n_max = 0, max_moves = 0;
  for (int g = 0; g < c->G; ++g) {
    if (c->count[g] + 1 > c->cap) return fail(c, KVEV_ESTATE, "slot capacity exhausted");
    n_max = std::max(n_max, c->count[g] + 1);
    // one token over budget frees a slot (no move); more plan a hole fill
    if (c->count[g] + 1 > B + 1) max_moves = std::max(max_moves, std::min(B, c->count[g] + 1 - B));
  }
  for (int g = 0; g < c->G; ++g)
    if (!ensure_pages(c, g, c->count[g] + 1, upd)) return fail(c, KVEV_ENOMEM, "page pool exhausted");
  if (!upd.empty()) KVEV_HIP(c, launch_set_pages(c, upd.data(), static_cast<int>(upd.size() / 2)));
  c->lstride = (n_max + 15) / 16 * 16;
  const bool whole = whole_cache_attention(c, n_max);
  // the launches time themselves ("attn_whole", "attn", "post") when
  // profiling; after the whole-cache attention the fold kernel folds,
  // selects and commits each group's state
  if (whole) {
    KVEV_HIP(c, launch_attention_seq(c, q, k_new, v_new, out, static_cast<int>(n_max), refresh ? 1 : 0));
    KVEV_HIP(c, launch_fold(c, static_cast<int>(n_max), refresh ? 1 : 0, do_select ? 1 : 0, B));
  } else {
    KVEV_HIP(c, launch_attention(c, q, k_new, v_new, static_cast<int>(n_max), refresh ? 1 : 0, "attn"));
    KVEV_HIP(c, launch_post(c, out, k_new, v_new, static_cast<int>(n_max), refresh ? 1 : 0,
                            do_select ? 1 : 0, B, 0));
  }
  // the post kernel plans the compaction; the move kernel copies the rows
  // (its blocks spread the scattered stores of the channel-major V columns)
  if (do_select && max_moves > 0) {
    ProfScope p(c, "move");
    KVEV_HIP(c, launch_moves(c, static_cast<int>(max_moves)));
  }
  if (diag && refresh) {
    ProfScope p(c, "diag");
    KVEV_HIP(c, launch_diag(c, static_cast<int>(t)));
  }
  for (int b = 0; b < c->cfg.batch; ++b) c->seq_next[b] += 1;
  for (int g = 0; g < c->G; ++g) {
    c->count[g] += 1;
    // a single-token eviction leaves its slot free inside the cache
    c->hole_in[g] = do_select && c->count[g] == B + 1;
    if (do_select && c->count[g] > B) c->count[g] = B;
    // the cache spans count + 1 slots (the free slot may lie inside)
    if (do_select) release_pages(c, g, c->count[g] + 1);
  }
  c->t = t;
  return KVEV_OK;
}

static kvev_status check_budget(kvev_ctx* c, int64_t budget, int64_t* B) {
  *B = budget > 0 ? budget : c->cfg.budget;
  if (*B < c->cfg.n_sink + c->cfg.n_recent || *B < 1)
    return fail(c, KVEV_EINVAL, "budget below the protected token count");
  if (*B > (1ll << 30)) return fail(c, KVEV_EINVAL, "budget out of range");
  return KVEV_OK;
}

kvev_status kvev_decode_step(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                             float* out) {
  KVEV_LIVE(c);
  if (c->block_mode) return block_step(c, q, k_new, v_new, out, false, 0);
  if (c->tier_mode) return tier_decode(c, q, k_new, v_new, out);
  if (c->cfg.diag_topk > 0) return fail(c, KVEV_ESTATE, "diagnostics on: use kvev_step");
  return run_step(c, q, k_new, v_new, out, false, c->cfg.budget);
}

kvev_status kvev_step(kvev_ctx* c, const void* q, const void* k_new, const void* v_new, float* out,
                      int64_t budget) {
  KVEV_LIVE(c);
  if (c->block_mode) return block_step(c, q, k_new, v_new, out, true, budget);
  if (c->tier_mode) {
    if (kvev_status s = tier_decode(c, q, k_new, v_new, out)) return s;
    const int omega = c->cfg.route_interval > 1 ? c->cfg.route_interval : 1;
    return c->t % omega == 0 ? tier_route(c) : KVEV_OK;  // routing events at t = 0 mod Omega
  }
  int64_t B;
  if (kvev_status s = check_budget(c, budget, &B)) return s;
  // selection only after the steps t with (t - 1) % evict_interval == 0
  const int64_t ei = c->cfg.evict_interval > 1 ? c->cfg.evict_interval : 1;
  return run_step(c, q, k_new, v_new, out, c->t % ei == 0, B);
}

kvev_status kvev_evict(kvev_ctx* c, int64_t budget) {
  KVEV_LIVE(c);
  if (c->block_mode) return block_evict(c, budget);
  if (c->tier_mode) return tier_route(c);
  if (c->cfg.diag_topk > 0) return fail(c, KVEV_ESTATE, "diagnostics on: use kvev_step");
  int64_t B;
  if (kvev_status s = check_budget(c, budget, &B)) return s;
  if (kvev_status s = check_pool_import(c)) return s;
  int64_t max_moves = 0;
  bool any = false, inner = false;
  for (int g = 0; g < c->G; ++g) {
    if (c->count[g] > B) {
      any = true;
      inner = inner || c->hole_in[g];
      // one token over budget frees a slot (no move); more plan a hole fill
      if (c->count[g] > B + 1) max_moves = std::max(max_moves, std::min(B, c->count[g] - B));
    }
  }
  if (!any) return KVEV_OK;
  if (inner) {
    // a free slot inside the cache: the last token moves into it first
    ProfScope p(c, "move");
    KVEV_HIP(c, launch_close_holes(c, B));
    KVEV_HIP(c, launch_moves(c, 1));
  }
  {
    ProfScope p(c, "select");
    KVEV_HIP(c, launch_select(c, B));
  }
  if (max_moves > 0) {
    ProfScope p(c, "move");
    KVEV_HIP(c, launch_moves(c, static_cast<int>(max_moves)));
  }
  for (int g = 0; g < c->G; ++g) {
    if (c->count[g] > B) {
      c->hole_in[g] = c->count[g] == B + 1;
      c->count[g] = B;
    }
    release_pages(c, g, c->count[g] + 1);
  }
  return KVEV_OK;
}

// The free slot of group g (token modes; block mode: count, the end).
// Synchronises.
static kvev_status read_hole(kvev_ctx* c, int g, int* hole) {
  *hole = static_cast<int>(c->count[g]);
  if (!c->d.hole) return KVEV_OK;
  KVEV_HIP(c, hipMemcpyAsync(hole, c->d.hole + g, sizeof(int), hipMemcpyDeviceToHost, c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  if (*hole < 0 || *hole > c->count[g]) return fail(c, KVEV_ESTATE, "inconsistent free slot");
  return KVEV_OK;
}

// Copy the count[g] live entries (elem bytes each) of a per-slot array
// (slots [0, count], the free slot skipped) to host memory.
static kvev_status copy_live(kvev_ctx* c, int g, const void* base, size_t elem, void* dst) {
  int h;
  if (kvev_status s = read_hole(c, g, &h)) return s;
  const int64_t n = c->count[g];
  const char* src = static_cast<const char*>(base) + static_cast<int64_t>(g) * c->cap * elem;
  char* out = static_cast<char*>(dst);
  if (h > 0) KVEV_HIP(c, hipMemcpyAsync(out, src, elem * h, hipMemcpyDeviceToHost, c->stream));
  if (n > h)
    KVEV_HIP(c, hipMemcpyAsync(out + elem * h, src + elem * (h + 1), elem * (n - h), hipMemcpyDeviceToHost,
                               c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  return KVEV_OK;
}

static kvev_status group_index(kvev_ctx* c, int32_t seq, int32_t h, int* g) {
  if (seq < 0 || seq >= c->cfg.batch || h < 0 || h >= c->cfg.n_kv_heads)
    return fail(c, KVEV_ERANGE, "group index out of range");
  *g = seq * c->cfg.n_kv_heads + h;
  return KVEV_OK;
}

kvev_status kvev_block_state(kvev_ctx* c, int32_t seq, float* score, int32_t* tref,
                             uint8_t* resident, int64_t cap, int64_t* n_blocks) {
  KVEV_LIVE(c);
  if (!c->block_mode) return fail(c, KVEV_EINVAL, "not in block mode");
  if (seq < 0 || seq >= c->cfg.batch) return fail(c, KVEV_ERANGE, "sequence index out of range");
  const int64_t nb = (c->npos[seq] + c->PT - 1) / c->PT;
  if (n_blocks) *n_blocks = nb;
  if (cap < nb) return fail(c, KVEV_ERANGE, "destination too small");
  const int64_t bblk = static_cast<int64_t>(seq) * c->maxblk;
  std::vector<int> res(nb);
  if (score)
    KVEV_HIP(c, hipMemcpyAsync(score, c->d.bscore + bblk, sizeof(float) * nb, hipMemcpyDeviceToHost, c->stream));
  if (tref)
    KVEV_HIP(c, hipMemcpyAsync(tref, c->d.btref + bblk, sizeof(int) * nb, hipMemcpyDeviceToHost, c->stream));
  if (resident && nb)
    KVEV_HIP(c, hipMemcpyAsync(res.data(), c->d.bres + bblk, sizeof(int) * nb, hipMemcpyDeviceToHost, c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  if (resident)
    for (int64_t j = 0; j < nb; ++j) resident[j] = res[j] ? 1 : 0;
  return KVEV_OK;
}

kvev_status kvev_set_budget(kvev_ctx* c, int32_t seq, int64_t budget) {
  KVEV_LIVE(c);
  if (!c->block_mode) return fail(c, KVEV_EINVAL, "not in block mode");
  if (seq < 0 || seq >= c->cfg.batch) return fail(c, KVEV_EINVAL, "sequence index out of range");
  if (budget < c->npinned[seq] + 1 || budget > kMaxBlockEntries)
    return fail(c, KVEV_EINVAL, "budget below the pinned blocks or out of range");
  const int b32 = static_cast<int>(budget);
  KVEV_HIP(c, hipMemcpyAsync(c->d.bbudget + seq, &b32, sizeof(int), hipMemcpyHostToDevice, c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  c->bbudget[seq] = b32;
  return KVEV_OK;
}

kvev_status kvev_readmit(kvev_ctx* c, int32_t seq, int64_t n, const int64_t* ids, const void* k,
                         const void* v) {
  KVEV_LIVE(c);
  if (!c->block_mode) return fail(c, KVEV_EINVAL, "not in block mode");
  if (seq < 0 || seq >= c->cfg.batch) return fail(c, KVEV_EINVAL, "sequence index out of range");
  if (!c->prefilled[seq]) return fail(c, KVEV_ESTATE, "sequence has no prefill");
  if (n < 1 || !ids || !k || !v) return fail(c, KVEV_EINVAL, "null argument or n < 1");
  if (c->nres[seq] + n > c->maxpages || c->count[seq * c->cfg.n_kv_heads] + c->PT * n + 1 > c->cap)
    return fail(c, KVEV_ENOMEM, "block table full");
  const int64_t tail = (c->npos[seq] - 1) / c->PT;
  std::vector<int> res(tail + 1);
  KVEV_HIP(c, hipMemcpyAsync(res.data(), c->d.bres + static_cast<int64_t>(seq) * c->maxblk,
                             sizeof(int) * (tail + 1), hipMemcpyDeviceToHost, c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  std::vector<int> id32(n);
  for (int64_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= tail) return fail(c, KVEV_EINVAL, "block id unknown or still being filled");
    if (res[ids[i]]) return fail(c, KVEV_EINVAL, "block is resident (or listed twice)");
    res[ids[i]] = 1;
    id32[i] = static_cast<int>(ids[i]);
  }
  const int e0 = c->nres[seq] - 1;
  KVEV_HIP(c, hipMemcpyAsync(c->d.rd_ids, id32.data(), sizeof(int) * n, hipMemcpyHostToDevice, c->stream));
  {
    ProfScope p(c, "readmit");
    KVEV_HIP(c, launch_block_readmit(c, seq, static_cast<int>(n), c->d.rd_ids, static_cast<int>(c->t)));
    KVEV_HIP(c, launch_scatter_at(c, seq, k, v, c->PT * n, e0));
  }
  KVEV_HIP(c, hipStreamSynchronize(c->stream));  // id32 is local
  c->nres[seq] += static_cast<int>(n);
  for (int h = 0; h < c->cfg.n_kv_heads; ++h) c->count[seq * c->cfg.n_kv_heads + h] += c->PT * n;
  return KVEV_OK;
}

kvev_status kvev_readmit_offloaded(kvev_ctx* c, int32_t seq, int64_t n, const int64_t* ids) {
  KVEV_LIVE(c);
  if (!c->block_mode) return fail(c, KVEV_EINVAL, "not in block mode");
  if (c->cfg.offload_blocks <= 0) return fail(c, KVEV_ESTATE, "the host-offload tier is off");
  if (seq < 0 || seq >= c->cfg.batch) return fail(c, KVEV_EINVAL, "sequence index out of range");
  if (!c->prefilled[seq]) return fail(c, KVEV_ESTATE, "sequence has no prefill");
  if (n < 1 || !ids) return fail(c, KVEV_EINVAL, "null argument or n < 1");
  if (c->nres[seq] + n > c->maxpages || c->count[seq * c->cfg.n_kv_heads] + c->PT * n + 1 > c->cap)
    return fail(c, KVEV_ENOMEM, "block table full");
  const int64_t tail = (c->npos[seq] - 1) / c->PT;
  std::vector<int> res(tail + 1), slot(tail + 1);
  const int64_t row = static_cast<int64_t>(seq) * c->maxblk;
  KVEV_HIP(c, hipMemcpyAsync(res.data(), c->d.bres + row, sizeof(int) * (tail + 1), hipMemcpyDeviceToHost,
                             c->stream));
  KVEV_HIP(c, hipMemcpyAsync(slot.data(), c->d.hslot + row, sizeof(int) * (tail + 1), hipMemcpyDeviceToHost,
                             c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  std::vector<int> id32(n), sl(n);
  for (int64_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= tail) return fail(c, KVEV_EINVAL, "block id unknown or still being filled");
    if (res[ids[i]]) return fail(c, KVEV_EINVAL, "block is resident (or listed twice)");
    if (slot[ids[i]] < 0 || slot[ids[i]] >= c->cfg.offload_blocks)
      return fail(c, KVEV_ESTATE, "block is not in the host pool");
    res[ids[i]] = 1;
    id32[i] = static_cast<int>(ids[i]);
    // a prefetched copy in device staging (valid while the block still owns
    // the pool slot it was copied from), else the pool slot (encoded -1 - slot)
    const int s = slot[ids[i]];
    const int key = static_cast<int>(seq * c->maxblk + ids[i]);
    int st = -1;
    for (int x = 0; x < static_cast<int>(c->pf_key.size()); ++x)
      if (c->pf_key[x] == key && c->pf_src[x] == s) st = x;
    sl[i] = st >= 0 ? st : -1 - s;
  }
  if (c->pf_pending) {
    KVEV_HIP(c, hipStreamWaitEvent(c->stream, c->pf_done, 0));
    c->pf_pending = false;
  }
  for (int64_t i = 0; i < n; ++i)  // consumed
    if (sl[i] >= 0) c->pf_key[sl[i]] = -1;
  const int e0 = c->nres[seq] - 1;
  KVEV_HIP(c, hipMemcpyAsync(c->d.rd_ids, id32.data(), sizeof(int) * n, hipMemcpyHostToDevice, c->stream));
  KVEV_HIP(c, hipMemcpyAsync(c->d.rd_slots, sl.data(), sizeof(int) * n, hipMemcpyHostToDevice, c->stream));
  {
    ProfScope p(c, "readmit");
    KVEV_HIP(c, launch_block_readmit(c, seq, static_cast<int>(n), c->d.rd_ids, static_cast<int>(c->t)));
    KVEV_HIP(c, launch_restore(c, seq, static_cast<int>(n), e0, c->d.rd_slots));
  }
  KVEV_HIP(c, hipStreamSynchronize(c->stream));  // id32 and sl are local
  c->nres[seq] += static_cast<int>(n);
  for (int h = 0; h < c->cfg.n_kv_heads; ++h) c->count[seq * c->cfg.n_kv_heads + h] += c->PT * n;
  return KVEV_OK;
}

kvev_status kvev_prefetch_offloaded(kvev_ctx* c, int32_t seq, int64_t n, const int64_t* ids) {
  KVEV_LIVE(c);
  if (!c->block_mode || c->cfg.prefetch_blocks <= 0 || !c->pf_stream)
    return fail(c, KVEV_ESTATE, "prefetch is off");
  if (seq < 0 || seq >= c->cfg.batch) return fail(c, KVEV_EINVAL, "sequence index out of range");
  if (n < 1 || !ids || n > c->cfg.prefetch_blocks) return fail(c, KVEV_EINVAL, "n outside 1..prefetch_blocks");
  const int64_t tail = (c->npos[seq] - 1) / c->PT;
  std::vector<int> slot(tail + 1);
  // the stream's earlier work (restores from staging, offloads into the pool) completes here
  KVEV_HIP(c, hipMemcpyAsync(slot.data(), c->d.hslot + static_cast<int64_t>(seq) * c->maxblk,
                             sizeof(int) * (tail + 1), hipMemcpyDeviceToHost, c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  for (int64_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= tail) return fail(c, KVEV_EINVAL, "block id unknown or still being filled");
    if (slot[ids[i]] < 0 || slot[ids[i]] >= c->cfg.offload_blocks)
      return fail(c, KVEV_ESTATE, "block is not in the host pool");
  }
  const size_t sb = 2ull * c->cfg.n_layers * c->cfg.n_kv_heads * c->PT * c->cfg.head_dim * c->elem;
  for (int64_t i = 0; i < n; ++i) {
    const int s = slot[ids[i]];
    const int key = static_cast<int>(seq * c->maxblk + ids[i]);
    bool staged = false;
    for (int x = 0; x < static_cast<int>(c->pf_key.size()); ++x)
      staged = staged || (c->pf_key[x] == key && c->pf_src[x] == s);
    if (staged) continue;
    const int st = c->pf_next;
    c->pf_next = (c->pf_next + 1) % c->cfg.prefetch_blocks;
    KVEV_HIP(c, hipMemcpyAsync(static_cast<char*>(c->dstage) + sb * st, static_cast<char*>(c->hpool) + sb * s, sb,
                               hipMemcpyHostToDevice, c->pf_stream));
    c->pf_key[st] = key;
    c->pf_src[st] = s;
  }
  KVEV_HIP(c, hipEventRecord(c->pf_done, c->pf_stream));
  c->pf_pending = true;
  return KVEV_OK;
}

kvev_status kvev_offload_state(kvev_ctx* c, int32_t seq, int32_t* slot, int64_t cap, int64_t* n_blocks) {
  KVEV_LIVE(c);
  if (!c->block_mode || c->cfg.offload_blocks <= 0) return fail(c, KVEV_ESTATE, "the host-offload tier is off");
  if (seq < 0 || seq >= c->cfg.batch) return fail(c, KVEV_ERANGE, "sequence index out of range");
  const int64_t nb = (c->npos[seq] + c->PT - 1) / c->PT;
  if (n_blocks) *n_blocks = nb;
  if (!slot) return KVEV_OK;
  if (nb > cap) return fail(c, KVEV_ERANGE, "cap too small");
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  if (nb > 0)
    KVEV_HIP(c, hipMemcpy(slot, c->d.hslot + static_cast<int64_t>(seq) * c->maxblk, sizeof(int) * nb,
                          hipMemcpyDeviceToHost));
  return KVEV_OK;
}

kvev_status kvev_import_blocks(kvev_ctx* c, int32_t seq, int64_t n_blocks, const float* score,
                               const int32_t* tref, const uint8_t* resident, int64_t n_tokens,
                               const void* k, const void* v) {
  KVEV_LIVE(c);
  if (!c->block_mode) return fail(c, KVEV_EINVAL, "not in block mode");
  if (c->cfg.offload_blocks > 0)
    return fail(c, KVEV_ESTATE, "host-offload tier on: the block state changes only by steps and readmissions");
  if (seq < 0 || seq >= c->cfg.batch) return fail(c, KVEV_EINVAL, "sequence index out of range");
  if (!c->prefilled[seq]) return fail(c, KVEV_ESTATE, "sequence has no prefill");
  if (!score || !tref || !resident || !k || !v) return fail(c, KVEV_EINVAL, "null argument");
  const int64_t nb = (c->npos[seq] + c->PT - 1) / c->PT;
  if (n_blocks != nb) return fail(c, KVEV_EINVAL, "n_blocks must equal the blocks seen");
  if (!resident[nb - 1]) return fail(c, KVEV_EINVAL, "the block being filled must be resident");
  std::vector<int> ids;
  for (int64_t j = 0; j < nb; ++j)
    if (resident[j]) ids.push_back(static_cast<int>(j));
  if (static_cast<int64_t>(ids.size()) > c->maxpages) return fail(c, KVEV_EINVAL, "too many resident blocks");
  const int64_t want = static_cast<int64_t>(c->PT) * (static_cast<int64_t>(ids.size()) - 1) +
                       block_fill(c, c->npos[seq]);
  if (n_tokens != want) return fail(c, KVEV_EINVAL, "n_tokens does not match the resident blocks");
  return block_install(c, seq, c->npos[seq], ids, score, tref, k, v);
}

kvev_status kvev_scores(kvev_ctx* c, int32_t seq, int32_t h, float* dst, int64_t cap,
                        int64_t* n_written) {
  KVEV_LIVE(c);
  if (c->tier_mode) {
    if (seq != 0) return fail(c, KVEV_ERANGE, "tiered mode: the only sequence is 0");
    return tier_scores(c, h, dst, cap, n_written);
  }
  int g;
  if (kvev_status s = group_index(c, seq, h, &g)) return s;
  if (c->block_mode) return kvev_block_state(c, seq, dst, nullptr, nullptr, cap, n_written);
  if (c->pooled) g = seq * c->cfg.n_kv_heads;  // the sequence's utilities
  const int64_t n = c->count[g];
  if (n_written) *n_written = n;
  if (!dst || cap < n) return fail(c, KVEV_ERANGE, "destination too small");
  return copy_live(c, g, c->d.score, sizeof(float), dst);
}

kvev_status kvev_retained(kvev_ctx* c, int32_t seq, int32_t h, int32_t* positions, int64_t cap,
                          int64_t* n_out) {
  KVEV_LIVE(c);
  if (c->tier_mode) return fail(c, KVEV_EINVAL, "tiered mode: use the kvev_tier_* calls");
  int g;
  if (kvev_status s = group_index(c, seq, h, &g)) return s;
  if (c->pooled) g = seq * c->cfg.n_kv_heads;  // one retained set per sequence
  const int64_t n = c->count[g];
  if (n_out) *n_out = n;
  if (!positions || cap < n) return fail(c, KVEV_ERANGE, "destination too small");
  return copy_live(c, g, c->d.pos, sizeof(int), positions);
}

kvev_status kvev_export_kv(kvev_ctx* c, int32_t seq, int32_t h, void* k_out, void* v_out,
                           int64_t cap, int64_t* n_out) {
  KVEV_LIVE(c);
  if (c->tier_mode) return fail(c, KVEV_EINVAL, "tiered mode: use the kvev_tier_* calls");
  int g;
  if (kvev_status s = group_index(c, seq, h, &g)) return s;
  const int64_t n = c->count[g];
  if (n_out) *n_out = n;
  if (!k_out || !v_out || cap < n) return fail(c, KVEV_ERANGE, "destination too small");
  int hole;
  if (kvev_status s = read_hole(c, g, &hole)) return s;
  KVEV_HIP(c, launch_export(c, g, k_out, v_out, n, cap, hole));
  return KVEV_OK;
}

kvev_status kvev_import_group(kvev_ctx* c, int32_t seq, int32_t h, int64_t n,
                              const int32_t* positions, const float* scores, const void* k,
                              const void* v) {
  KVEV_LIVE(c);
  if (c->tier_mode) return fail(c, KVEV_EINVAL, "tiered mode: use the kvev_tier_* calls");
  int g;
  if (kvev_status s = group_index(c, seq, h, &g)) return s;
  if (c->block_mode) return fail(c, KVEV_EINVAL, "block mode: use kvev_import_blocks");
  if (c->cfg.diag_topk > 0) return fail(c, KVEV_ESTATE, "diagnostics on: the state changes only by kvev_step");
  if (!positions || !scores || !k || !v) return fail(c, KVEV_EINVAL, "null argument");
  if (n < 1 || n + 1 > c->cap) return fail(c, KVEV_ERANGE, "n out of range");
  if (c->pooled) {
    // every KV head of a sequence holds the same slots: the sequence's
    // import completes once each of its KV heads was imported with the same
    // positions (in the same slot order); until then the step calls refuse
    auto& pi = c->pool_import[seq];
    if (pi.done.empty()) {
      pi.done.assign(c->cfg.n_kv_heads, 0);
      pi.pos.assign(positions, positions + n);
    } else if (static_cast<int64_t>(pi.pos.size()) != n || !std::equal(pi.pos.begin(), pi.pos.end(), positions)) {
      return fail(c, KVEV_EINVAL,
                  "per-sequence granularity: every KV head of a sequence must be imported with the same positions");
    }
  }
  int maxp = 0;
  for (int64_t i = 0; i < n; ++i) maxp = std::max(maxp, positions[i]);
  std::vector<int> upd;
  if (!ensure_pages(c, g, n, upd)) return fail(c, KVEV_ENOMEM, "page pool exhausted");
  if (!upd.empty()) KVEV_HIP(c, launch_set_pages(c, upd.data(), static_cast<int>(upd.size() / 2)));
  KVEV_HIP(c, launch_import(c, g, k, v, n));
  KVEV_HIP(c, hipMemcpyAsync(c->d.pos + static_cast<int64_t>(g) * c->cap, positions,
                             sizeof(int) * n, hipMemcpyHostToDevice, c->stream));
  KVEV_HIP(c, hipMemcpyAsync(c->d.score + static_cast<int64_t>(g) * c->cap, scores,
                             sizeof(float) * n, hipMemcpyHostToDevice, c->stream));
  const int cnt = static_cast<int>(n);
  KVEV_HIP(c, hipMemcpyAsync(c->d.count + g, &cnt, sizeof(int), hipMemcpyHostToDevice, c->stream));
  KVEV_HIP(c, hipMemcpyAsync(c->d.hole + g, &cnt, sizeof(int), hipMemcpyHostToDevice, c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  release_pages(c, g, n + 1);
  c->count[g] = n;
  c->hole_in[g] = 0;
  if (c->pooled) {
    auto& pi = c->pool_import[seq];
    pi.done[h] = 1;
    if (std::all_of(pi.done.begin(), pi.done.end(), [](uint8_t x) { return x != 0; })) {
      pi.done.clear();
      pi.pos.clear();
    }
  }
  return KVEV_OK;
}

kvev_status kvev_diag_read(kvev_ctx* c, kvev_diag_group* out, int32_t n_groups) {
  KVEV_LIVE(c);
  if (c->cfg.diag_topk <= 0 || !c->d.dcnt) return fail(c, KVEV_ESTATE, "diagnostics are off");
  if (!out || n_groups < 1 || n_groups > c->G) return fail(c, KVEV_ERANGE, "n_groups out of range");
  std::vector<int> cnt(static_cast<size_t>(n_groups) * kDiagCounts);
  std::vector<double> acc(static_cast<size_t>(n_groups) * kDiagAcc);
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  KVEV_HIP(c, hipMemcpy(cnt.data(), c->d.dcnt, sizeof(int) * cnt.size(), hipMemcpyDeviceToHost));
  KVEV_HIP(c, hipMemcpy(acc.data(), c->d.dacc, sizeof(double) * acc.size(), hipMemcpyDeviceToHost));
  for (int g = 0; g < n_groups; ++g) {
    const int* k = &cnt[static_cast<size_t>(g) * kDiagCounts];
    const double* a = &acc[static_cast<size_t>(g) * kDiagAcc];
    kvev_diag_group& o = out[g];
    o.n = k[0];
    o.k = k[1];
    o.raw_overlap = k[2];
    o.raw_prev = k[3];
    o.util_overlap = k[4];
    o.util_prev = k[5];
    o.raw_util_overlap = k[6];
    o.raw_top_evicted = k[7];
    o.evicted = k[8];
    o.retained = k[9];
    o.retained_overlap = k[10];
    o.retained_prev = k[11];
    o.steps = static_cast<int64_t>(a[0]);
    o.pairs = static_cast<int64_t>(a[1]);
    o.sum_raw_churn = a[2];
    o.sum_util_churn = a[3];
    o.sum_raw_util_jaccard = a[4];
    o.sum_raw_top_evicted = a[5];
    o.sum_selection_churn = a[6];
  }
  return KVEV_OK;
}

kvev_status kvev_diag_trace(kvev_ctx* c, int32_t seq, int32_t h, int32_t* positions, float* raw,
                            float* util, int64_t cap, int64_t* n) {
  KVEV_LIVE(c);
  if (c->cfg.diag_topk <= 0 || !c->d.dg_n) return fail(c, KVEV_ESTATE, "diagnostics are off");
  int g;
  if (kvev_status s = group_index(c, seq, h, &g)) return s;
  int cnt = 0;
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  KVEV_HIP(c, hipMemcpy(&cnt, c->d.dg_n + g, sizeof(int), hipMemcpyDeviceToHost));
  if (n) *n = cnt;
  if (cnt > cap && (positions || raw || util)) return fail(c, KVEV_ERANGE, "cap too small");
  const int64_t off = static_cast<int64_t>(g) * c->cap;
  if (positions && cnt > 0)
    KVEV_HIP(c, hipMemcpy(positions, c->d.dg_pos + off, sizeof(int) * cnt, hipMemcpyDeviceToHost));
  if (raw && cnt > 0)
    KVEV_HIP(c, hipMemcpy(raw, c->d.dg_raw + off, sizeof(float) * cnt, hipMemcpyDeviceToHost));
  if (util && cnt > 0)
    KVEV_HIP(c, hipMemcpy(util, c->d.dg_util + off, sizeof(float) * cnt, hipMemcpyDeviceToHost));
  return KVEV_OK;
}

}  // extern "C"

namespace kvev {
// The argument checks shared by the two missed-mass entry points.
kvev_status fmm_check(kvev_ctx* full, kvev_ctx* comp, const double* fmm) {
  if (!fmm || full == comp) return fail(comp, KVEV_EINVAL, "null output or the same context twice");
  if (full->cfg.diag_topk <= 0 || comp->cfg.diag_topk <= 0)
    return fail(comp, KVEV_ESTATE, "diagnostics are off");
  const kvev_config &a = full->cfg, &b = comp->cfg;
  if (a.n_layers != b.n_layers || a.n_q_heads != b.n_q_heads || a.n_kv_heads != b.n_kv_heads ||
      a.batch != b.batch || a.head_dim != b.head_dim || a.max_tokens != b.max_tokens)
    return fail(comp, KVEV_EINVAL, "contexts of different shapes");
  if (a.budget < a.max_tokens || a.scorer != 0)
    return fail(comp, KVEV_EINVAL, "the full context must never evict and use the attention scorer");
  if (full->t != comp->t) return fail(comp, KVEV_EINVAL, "contexts at different steps");
  if (comp->t < 1) return fail(comp, KVEV_ESTATE, "no step yet");
  for (int s = 0; s < a.batch; ++s)
    if (full->seq_next[s] != comp->seq_next[s]) return fail(comp, KVEV_EINVAL, "different prefill lengths");
  return KVEV_OK;
}
}  // namespace kvev

extern "C" {

kvev_status kvev_diag_fmm(kvev_ctx* full, kvev_ctx* comp, double* fmm) {
  KVEV_LIVE(full);
  KVEV_LIVE(comp);
  if (kvev_status s = fmm_check(full, comp, fmm)) return s;
  double* dev = nullptr;
  KVEV_HIP(comp, hipMalloc(&dev, sizeof(double) * comp->G));
  hipEvent_t ev = nullptr;
  hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventRecord(ev, full->stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(comp->stream, ev, 0);
  if (e == hipSuccess) e = launch_fmm(full, comp, dev);
  if (e == hipSuccess)
    e = hipMemcpyAsync(fmm, dev, sizeof(double) * comp->G, hipMemcpyDeviceToHost, comp->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(comp->stream);
  if (ev) hipEventDestroy(ev);
  hipFree(dev);
  if (e != hipSuccess) return hip_fail(comp, e, "kvev_diag_fmm");
  return KVEV_OK;
}

kvev_status kvev_sync(kvev_ctx* c) {
  KVEV_LIVE(c);
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  KVEV_HIP(c, hipGetLastError());
  int flag = 0;
  KVEV_HIP(c, hipMemcpy(&flag, c->d.errflag, sizeof(int), hipMemcpyDeviceToHost));
  if (flag) {
    c->sticky = true;
    c->err = "device consistency check failed (flag " + std::to_string(flag) + ")";
    return KVEV_ESTATE;
  }
  if (c->tier_mode) return KVEV_OK;
  // the host's slot counts size every launch: they must match the device's
  std::vector<int> dc(c->G);
  KVEV_HIP(c, hipMemcpy(dc.data(), c->d.count, sizeof(int) * c->G, hipMemcpyDeviceToHost));
  for (int g = 0; g < c->G; ++g)
    if (dc[g] != c->count[g]) {
      c->sticky = true;
      c->err = "device slot count of group " + std::to_string(g) + " differs from the host's";
      return KVEV_ESTATE;
    }
  return KVEV_OK;
}

int64_t kvev_step_index(const kvev_ctx* c) { return c ? c->t : -1; }

kvev_status kvev_profile_enable(kvev_ctx* c, int32_t enable) {
  KVEV_LIVE(c);
  c->prof.enabled = enable != 0;
  return KVEV_OK;
}

kvev_status kvev_profile_reset(kvev_ctx* c) {
  KVEV_LIVE(c);
  prof_drain(c);
  c->prof.totals.clear();
  return KVEV_OK;
}

kvev_status kvev_profile_read(kvev_ctx* c, const char* kernel, double* total_ms,
                              int64_t* launches) {
  KVEV_LIVE(c);
  if (!kernel) return fail(c, KVEV_EINVAL, "null kernel name");
  prof_drain(c);
  double ms = 0;
  long long nl = 0;
  for (auto& t : c->prof.totals)
    if (t.first == kernel) {
      ms = t.second.first;
      nl = t.second.second;
    }
  if (total_ms) *total_ms = ms;
  if (launches) *launches = nl;
  return KVEV_OK;
}

const char* kvev_last_error(const kvev_ctx* c) {
  if (!c) return g_create_error.c_str();
  return c->err.c_str();
}

}  // extern "C"
