// Internal state of a kvev context and the kernel launchers (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <string>
#include <type_traits>
#include <vector>

#include "../../include/kvev.h"
#include "common.h"

namespace kvev {

constexpr int kAttnChunk = 256;   // slots per attention split
constexpr int kPostTokens = 64;   // slots per post-attention block
constexpr int kPoolTokens = 16;   // slots per block of the sequence-pooled post kernel
constexpr int kMaxGroupSize = 8;  // query heads per KV head supported
constexpr int kRegions = 8;       // region labels of the block-granular mode
constexpr int kMaxBlockEntries = 4096;  // block-table entries per sequence (block mode)
// two-tier window mode
constexpr int kTierWin = 32;            // tokens per routing window
constexpr int kTierD = 128;             // head dim of the tiered mode
constexpr int kTierLedgerBytes = 3072;  // INT2 record per (layer, KV head, window)
constexpr int kTierMaxWin = 12288;      // windows per sequence (393216 positions at 32 tokens a window)
constexpr int kTierLedgerBytes8 = 1152; // INT2 record of an 8-token window
inline int tier_rec_bytes(int w) { return w == 8 ? kTierLedgerBytes8 : kTierLedgerBytes; }
constexpr int kTierXferBlocks = 512;    // blocks of the transition kernel (all layers)
constexpr int kTierWinBits = 14;        // a list entry is slot << kTierWinBits | window
// rank-trace diagnostics
constexpr int kDiagCounts = 12;  // the int32 counts of kvev_diag_group, in order
constexpr int kDiagAcc = 7;      // steps, pairs and the five sums

// Device buffers of one context.  Groups are (sequence, KV head) pairs,
// g = seq * Hkv + kv_head; slots of a group are its cached tokens in order.
struct DevState {
  void* kpool = nullptr;   // [L][P][PT][D] cfg.dtype
  void* vpool = nullptr;
  int* ptab = nullptr;     // [G][maxpages] physical page of each logical page
  int* pos = nullptr;      // [G][cap] position of each slot
  float* score = nullptr;  // [G][cap] utility of each slot
  int* count = nullptr;    // [G] tokens in the group
  int* hole = nullptr;     // [G] the free slot the next token takes (token modes): count, or the
                           // slot a single-token eviction freed (the cache then spans count + 1 slots)
  int* nextpos = nullptr;  // [G] position the next appended token takes
  float* logits = nullptr; // [G][L][lstride][HG] fp32 logits of the current step
  float* part_ml = nullptr;// [L][G][S][HG][2] per-split (max, sum), S = splits of the step
  float* part_o = nullptr; // [L][G][S][HG][D] per-split unnormalised output
  float* ml = nullptr;     // [L][G][HG][2] global (max, sum)
  float* part_u = nullptr; // [L][G][S][HG] entropy partials (entropy scorer only)
  float* vnorm = nullptr;  // [G][L][lstride] value-row norms (VNorm scorer only)
  float* part_vn = nullptr;// [L][G][S] per-split sums of vnorm (VNorm scorer only)
  int* mv_src = nullptr;   // [G][cap] compaction moves
  int* mv_dst = nullptr;   // [G][cap]
  int* nmoves = nullptr;   // [G]
  int* errflag = nullptr;  // [1] device-side consistency failures (bit mask)
  unsigned* grpctr = nullptr;  // [G] arrival counters of the post kernel (0 between launches)
  unsigned long long* blk_key = nullptr;  // [G][max_post_blocks] per-block minimum eviction key
  int* blk_slot = nullptr;                // [G][max_post_blocks] its slot
  float* blk_sum = nullptr;               // [G][max_post_blocks] per-block utility sum
  float* gnew = nullptr;                  // [G] the new token's folded utility (fold kernel)
  // rank-trace diagnostics (cfg.diag_topk > 0)
  int* dg_n = nullptr;      // [G] tokens the last step attended
  int* dg_pos = nullptr;    // [G][cap] their positions, in the step's slot order
  float* dg_raw = nullptr;  // [G][cap] the step's observation summed over layers
  float* dg_util = nullptr; // [G][cap] the utility after the step's fold
  int* st_raw = nullptr;    // [G][max_tokens] last step whose raw top-k held the position
  int* st_util = nullptr;   // [G][max_tokens] ... utility top-k
  int* st_kept = nullptr;   // [G][max_tokens] last step after which the position was kept
  int* ev_step = nullptr;   // [G][max_tokens] step that evicted the position (0: never)
  int* dprev = nullptr;     // [G][4] last recorded step, its k, its retained count
  int* dcnt = nullptr;      // [G][kDiagCounts] the last step's counts
  double* dacc = nullptr;   // [G][kDiagAcc] sums over the recorded steps
  // host-offload tier (block mode, cfg.offload_blocks > 0)
  int* ev_n = nullptr;      // [batch] blocks the last selection evicted
  int* ev_blk = nullptr;    // [batch][maxpages] their ids
  int* ev_page = nullptr;   // [G][maxpages] their pages
  int* hslot = nullptr;     // [batch][maxblk] pool slot of an evicted block, or -1
  int* sowner = nullptr;    // [offload_blocks] owner b * maxblk + block, or -1
  int* rd_slots = nullptr;  // [maxpages] slots of a re-admission
  int* ev_slot = nullptr;   // [batch][maxpages] pool slot of each evicted block, or -1 (dropped)
  int* oring = nullptr;     // [2] the pool's next ring slot, and its value after the current selection
  // block-granular mode
  int* btab = nullptr;      // [batch][maxpages] logical block of each table entry
  int* nres = nullptr;      // [batch] table entries (resident blocks)
  float* bscore = nullptr;  // [batch][maxblk] score of every logical block (kept when evicted)
  int* btref = nullptr;     // [batch][maxblk] step of the last access / insertion
  int* bres = nullptr;      // [batch][maxblk] 1 while resident
  float* bpart = nullptr;   // [L][G][maxpages][HG] per-block sums of exp(s - M_split) (matrix-core path)
  uint8_t* bcnt = nullptr;  // [batch][maxblk][kRegions] tokens of each region in the block
  int* fstack = nullptr;    // [G][maxpages] free pages of each group
  int* ftop = nullptr;      // [G] free pages on the stack
  float* bmass = nullptr;   // [batch][maxpages] step mass per table entry (unnormalised)
  int* bbudget = nullptr;   // [batch] retained blocks per sequence
  int* rd_ids = nullptr;    // [maxpages] block ids of one re-admission call
};

// Device buffers of the two-tier window mode ([L][Hkv][NW] windows).
struct TierDev {
  // full-precision slot pool: SF window slots per (layer, KV head)
  uint16_t* kfp = nullptr;   // [L][Hkv][SF][W][128] bf16 keys, token-major (rotated in rotary mode)
  uint16_t* vfp = nullptr;   // [L][Hkv][SF][128][W] bf16 values, channel-major
  uint16_t* kpre = nullptr;  // rotary mode: [L][Hkv][SF][W][128] bf16 keys before the rotation
  // INT2 record pool: SQ records per (layer, KV head)
  uint8_t* ledger = nullptr; // [L][Hkv][SQ][record bytes] INT2 codes and parameters
  // prefill staging (until the first routing event has placed every prefill
  // window): NWS windows in the layout of the pool; slot SF + w is window w
  uint16_t* kst = nullptr;
  uint16_t* vst = nullptr;
  uint16_t* kpst = nullptr;
  int* fslot = nullptr;      // [L][NW] full-precision slot of each window (-1: none)
  int* lslot = nullptr;      // [L][NW] record slot of each window (-1: none)
  int* ffree = nullptr;      // [L][SF] the free full-precision slots after the last routing event, ascending
  double* rcs = nullptr;     // rotary mode: [max_tokens][64][2] cos and sin of position * frequency
  double* ifreq = nullptr;   // rotary mode: [64] frequencies theta^(-2i/128)
  uint8_t* tier = nullptr;   // [L][NW] 0 full precision, 1 INT2, 2 evicted
  uint8_t* hasled = nullptr; // [L][NW] 1 once the window has been quantized
  uint8_t* forced = nullptr; // [L][NW] tiers imported by kvev_tier_import
  float* S = nullptr;        // [L][NW] cumulative window score
  // routing diagnostics (cfg.revival_gap > 0)
  int* rd_fstamp = nullptr;  // [L][NW] last event that routed the window to full precision
  int* rd_rstamp = nullptr;  // [L][NW] last event that kept it (full precision or INT2)
  int* rd_run = nullptr;     // [L][NW] consecutive events outside full precision
  int* rd_cnt = nullptr;     // [L][6] the last event's set sizes and overlaps
  double* rd_acc = nullptr;  // [L][6] events, pairs, churn sums, sustained, revived
  int* fplist = nullptr;     // [L][NW] full-precision windows (pinned, local, routed)
  int* qlist = nullptr;      // [L][NW] INT2 windows
  int4* jobs = nullptr;      // [L][NW] transition jobs: (window << 2 | kind, source slot, slot, record slot)
  int* njobs = nullptr;      // [L]
  float* emass = nullptr;    // [L][Hkv][NW][4] per listed window and head: sum exp(s - chunk max)
};

// Host mirror of the tiered mode (the list lengths are equal in every
// layer: every layer routes the same number of candidates).
struct TierHost {
  int NW = 0, maxch = 0;
  int SF = 0, SQ = 0;  // full-precision and record slots per (layer, KV head)
  int NWS = 0;         // prefill windows in the staging buffers (0: none allocated)
  bool stage_done = false;  // every prefill window placed: the staging buffers may be freed
  int held = 0;        // full-precision slots held after the last routing event
  int opened = 0;      // windows opened since then (each took the next free slot)
  int W = 32;          // tokens per window
  bool rope = false;   // rotary mode (cfg.rope_theta > 0)
  bool mat = false;    // INT2 windows are attended through their bf16 reconstruction, kept in the
                       // full-precision storage (8-token windows, rotary mode or key groups)
  bool kgroups = false;  // keys quantized per token and 32-channel group
  int64_t npos = 0;  // positions 0 .. npos-1 exist
  int n_fp = 0;      // full-precision windows listed (pinned + local + routed F)
  int n_q = 0;       // INT2 windows listed
  int n_kept = 0;    // routed windows in F or Q after the last routing event
  int na_prev = 0;   // aged windows at the last routing event
  int events = 0;    // routing events so far
};

// Kernel arguments of the tiered mode.
struct TierArgs {
  uint16_t* kfp;
  uint16_t* vfp;
  uint8_t* ledger;
  uint8_t* tier;
  uint8_t* hasled;
  float* S;
  int* fplist;
  int* qlist;
  int4* jobs;
  int* njobs;
  float* part_ml;  // [L][Hkv][maxch][4][2]
  float* part_o;   // [L][Hkv][maxch][4][128]
  float* ml;       // [L][Hkv][4][2]
  float* emass;
  int* errflag;
  int* rd_fstamp;  // routing diagnostics, or null
  int* rd_rstamp;
  int* rd_run;
  int* rd_cnt;
  double* rd_acc;
  int rd_gap, rd_event;
  int L, Hkv, Hq, NW, maxch;
  int W, rope, mat, recb;  // window tokens, rotary mode, bf16 reconstruction, record bytes
  uint16_t* kpre;
  double* rcs;
  const double* ifreq;
  uint16_t* kst;
  uint16_t* vst;
  uint16_t* kpst;
  int* fslot;
  int* lslot;
  int* ffree;
  int SF, SQ, NWS;
  int kgroups;  // keys quantized per token and 32-channel group (else per channel)
};

struct Profiler {
  bool enabled = false;
  // name under which the next timed_launch() records the kernel's own
  // dispatch start and end (set by the caller around one launch)
  struct Rec {
    std::string name;
    hipEvent_t a, b;
  };
  std::vector<Rec> pending;
  std::vector<std::pair<std::string, std::pair<double, long long>>> totals;
  std::vector<hipEvent_t> pool;
};

}  // namespace kvev

struct kvev_ctx {
  kvev_config cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  int G = 0, HG = 0, PT = kvev::kPageTokens, maxpages = 0;
  int max_lds = 65536;  // LDS bytes a workgroup may allocate on the device
  bool pooled = false;  // one retained set per sequence (KVEV_PER_SEQUENCE)
  int64_t cap = 0, P = 0;
  int64_t lstride = 0;  // slot stride of the logit scratch in the current step
  int max_splits = 0;
  int max_post_blocks = 0;
  size_t elem = 0;
  kvev::DevState d;
  // host mirrors (kept exact: every count change is deterministic)
  std::vector<int64_t> count;
  std::vector<uint8_t> hole_in;             // token modes: the free slot may lie inside (after a
                                            // single-token eviction; an append fills it)
  std::vector<int> prefilled;               // per sequence
  std::vector<int64_t> seq_next;            // per sequence: the next position (token modes)
  struct PoolImport {                       // per-sequence granularity: an import in progress
    std::vector<uint8_t> done;              // KV heads imported so far (empty: none pending)
    std::vector<int> pos;                   // the positions every KV head must take
  };
  std::vector<PoolImport> pool_import;      // per sequence
  void* hpool = nullptr;                    // pinned host pool of the offload tier
  void* hpool_dev = nullptr;                // its device mapping
  // background prefetch of pool blocks into device staging
  hipStream_t pf_stream = nullptr;          // the copies' stream (default priority)
  hipEvent_t pf_done = nullptr;             // recorded after each batch of copies
  bool pf_pending = false;                  // the context's stream has not waited for pf_done yet
  void* dstage = nullptr;                   // [prefetch_blocks] device copies of pool slots
  std::vector<int> pf_key;                  // staging slot -> block key b * maxblk + block, or -1
  std::vector<int> pf_src;                  // staging slot -> the pool slot it was copied from
  int pf_next = 0;                          // next staging slot
  int64_t t = 0;
  bool sticky = false;
  std::string err;
  kvev::Profiler prof;
  std::vector<int> ptab_upd;                // scratch for page-table updates
  // block-granular mode
  bool block_mode = false;
  int maxblk = 0;
  float lam[kvev::kRegions] = {};
  std::vector<int> nres;                    // host mirror of resident blocks per sequence
  std::vector<int64_t> npos;                // next position per sequence
  std::vector<int> bbudget;                 // per-sequence block budget
  std::vector<int> npinned;                 // blocks pinned by region labels per sequence
  // two-tier window mode
  bool tier_mode = false;
  kvev::TierDev td;
  kvev::TierHost tw;
};

namespace kvev {

// Dynamic LDS floats of the sequence-pooled post kernel: per (layer, query
// head) statistics and entropies, one output's split weights, the per
// (layer, KV head) and per layer slot masses, the layer factors and the per
// (layer, KV head) norm factors.
inline int64_t pool_post_shm(int L, int Hq, int Hkv, int64_t S) {
  return 3ll * L * Hq + (Hq / Hkv) * S + static_cast<int64_t>(L) * Hkv * (kPoolTokens + 1) +
         static_cast<int64_t>(L) * (kPoolTokens + 1);
}
// Calls fn(std::integral_constant<int, HG>) for a query group size 1..8.
template <typename Fn>
inline hipError_t with_group(int hg, Fn&& fn) {
  switch (hg) {
    case 1: return fn(std::integral_constant<int, 1>{});
    case 2: return fn(std::integral_constant<int, 2>{});
    case 3: return fn(std::integral_constant<int, 3>{});
    case 4: return fn(std::integral_constant<int, 4>{});
    case 5: return fn(std::integral_constant<int, 5>{});
    case 6: return fn(std::integral_constant<int, 6>{});
    case 7: return fn(std::integral_constant<int, 7>{});
    case 8: return fn(std::integral_constant<int, 8>{});
    default: return hipErrorInvalidValue;
  }
}
// Pops a profiling event from the context's pool (or creates one).
inline hipEvent_t prof_event(kvev_ctx* c);
// Launch of `kern` on the context's stream.  With profiling on and a name,
// the launch records its own dispatch start and end timestamps into an
// event pair (hipExtLaunchKernelGGL: no separate event packets between the
// step's kernels, so the durations are not inflated), accumulated under
// `name`.
template <typename F, typename... Args>
hipError_t timed_launch(kvev_ctx* c, const char* name, F kern, dim3 grid, dim3 block, size_t shm,
                        Args... args);
// Launchers (defined in the .hip translation units).  All are stream-ordered.
hipError_t launch_prefill_scatter(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n);
// scatter into table entries [e0, e0 + ceil(n/16)) of every KV head of `seq`
hipError_t launch_scatter_at(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n, int e0);
hipError_t launch_set_pages(kvev_ctx* c, const int* upd, int n_upd);
// prof: the profiling name of the matrix-core launch (nullptr: the caller
// times the launch itself)
hipError_t launch_attention(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                            int n_max, int write_logits, const char* prof = nullptr);
hipError_t launch_post(kvev_ctx* c, float* out, const void* k_new, const void* v_new, int n_max,
                       int refresh, int do_select, int64_t budget, int seq);
// whole-cache attention: one workgroup per (group, layer) (attn_seq.hip);
// writes out and, with obs, the per-slot group masses into d.logits
// ([G][L][lstride]); token modes only (group g's logical page i is pool
// page g * maxpages + i)
hipError_t launch_attention_seq(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                                float* out, int n_max, int obs);
// the same kernel over the block mode's page tables: writes out and the
// group mass of every table entry into d.bpart ([batch][L][Hkv][maxpages]);
// launch_block_entry_mass then sums it per entry into bmass
hipError_t launch_attention_seq_blocks(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                                       float* out, int n_max);
// after it: fold of the masses, the new token's state and the selection
// (policy.hip)
hipError_t launch_fold(kvev_ctx* c, int n_max, int refresh, int do_select, int64_t budget);
int64_t seq_attn_lds_bytes(int hg, int64_t n_max, bool obs, bool paged);
constexpr int kSeqMaxSlots = 8192;  // the whole-cache kernel's slot bound (64 pages per wave)
hipError_t launch_select(kvev_ctx* c, int64_t budget);
// plans the move of each over-budget group's last token into its inner free slot
hipError_t launch_close_holes(kvev_ctx* c, int64_t budget);
hipError_t launch_moves(kvev_ctx* c, int max_moves);
// the n rows of slots [0, n] other than slot `skip` (n + 1 > skip: the free slot)
hipError_t launch_export(kvev_ctx* c, int g, void* k_out, void* v_out, int64_t n, int64_t cap, int64_t skip);
hipError_t launch_import(kvev_ctx* c, int g, const void* k, const void* v, int64_t n);
// rank-trace diagnostics (diag.hip): after a step's post kernel, at step t
hipError_t launch_diag(kvev_ctx* c, int t);
// missed mass of `comp` against `full`, into device fmm[G]
hipError_t launch_fmm(kvev_ctx* full, kvev_ctx* comp, double* fmm_dev);
kvev_status fmm_check(kvev_ctx* full, kvev_ctx* comp, const double* fmm);
// block-granular mode (block.hip)
hipError_t launch_block_open(kvev_ctx* c, int n_max, int t);
hipError_t launch_block_merge(kvev_ctx* c, float* out, int n_max);
hipError_t launch_block_mass(kvev_ctx* c, int n_max);
hipError_t launch_block_entry_mass(kvev_ctx* c, int n_max);
hipError_t launch_block_policy(kvev_ctx* c, int t, int update, int do_select, int appended,
                               int budget_override);
hipError_t launch_block_readmit(kvev_ctx* c, int b, int n, const int* ids_dev, int t);
// host-offload tier: copy the last selection's evicted blocks into the pool;
// copy pool slots into the entries [e0, e0 + n) of sequence b
hipError_t launch_offload(kvev_ctx* c, int k_max, int e_host);
// src_dev[i] >= 0: staging slot; -1 - s: pool slot s
hipError_t launch_restore(kvev_ctx* c, int b, int n, int e0, const int* src_dev);
// two-tier window mode (tier.hip)
hipError_t launch_tier_prefill(kvev_ctx* c, const void* k, const void* v, int64_t n);
hipError_t launch_tier_rope_table(kvev_ctx* c, int64_t p0, int64_t n);
hipError_t launch_tier_append(kvev_ctx* c, const void* k_new, const void* v_new, int kslot);
hipError_t launch_tier_attention(kvev_ctx* c, const void* q);
hipError_t launch_tier_merge(kvev_ctx* c, float* out);
hipError_t launch_tier_route(kvev_ctx* c, int nw, int np, int recent_lo, int exp_fp, int exp_q,
                             const uint8_t* forced_dev, int layer);  // layer < 0: every layer
hipError_t launch_tier_export(kvev_ctx* c, int l, int h, void* k_out, void* v_out, int nwin);
// host side of the tiered mode (tier_api.cpp)
hipError_t tier_alloc(kvev_ctx* c);
void tier_free(kvev_ctx* c);
kvev_status tier_prefill(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n);
kvev_status tier_decode(kvev_ctx* c, const void* q, const void* k_new, const void* v_new, float* out);
kvev_status tier_route(kvev_ctx* c);
kvev_status tier_scores(kvev_ctx* c, int layer, float* dst, int64_t cap, int64_t* n);

inline hipEvent_t prof_event(kvev_ctx* c) {
  if (!c->prof.pool.empty()) {
    hipEvent_t e = c->prof.pool.back();
    c->prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <typename F, typename... Args>
hipError_t timed_launch(kvev_ctx* c, const char* name, F kern, dim3 grid, dim3 block, size_t shm,
                        Args... args) {
  if (!c->prof.enabled || name == nullptr) {
    kern<<<grid, block, shm, c->stream>>>(args...);
    return hipGetLastError();
  }
  hipEvent_t a = prof_event(c), b = prof_event(c);
  if (!a || !b) {  // no events to be had: launch untimed
    kern<<<grid, block, shm, c->stream>>>(args...);
    return hipGetLastError();
  }
  hipExtLaunchKernelGGL(kern, grid, block, static_cast<uint32_t>(shm), c->stream, a, b, 0, args...);
  c->prof.pending.push_back({name, a, b});
  return hipGetLastError();
}

}  // namespace kvev
