// Host side of the two-tier window mode: allocation, step sequencing, the
// per-layer tier counts, and the copy-out / import calls.
//
// The counts of the routing state machine are a function of positions
// alone, so the host knows every launch shape without reading the device:
// windows [0, np) hold sink positions (pinned), windows [np, na + np) are
// aged (full and older than the n_recent newest positions) and the rest are
// local.  Aged windows not evicted are the candidates of a routing event:
// those kept by the previous event plus the windows aged since.  Of them
// min(K_f, n) stay full precision and min(K_q, n - that) go to INT2
// ("QEvict" review, section 4.4, Eq.4-5).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "host_util.h"

namespace kvev {

namespace {

struct Counts {
  int nw, np, recent_lo, na;
};

Counts tier_counts(const kvev_ctx* c) {
  Counts k;
  const int64_t npos = c->tw.npos;
  const int W = c->tw.W;
  k.nw = static_cast<int>((npos + W - 1) / W);
  k.np = c->cfg.n_sink > 0 ? std::min(k.nw, (c->cfg.n_sink + W - 1) / W) : 0;
  const int64_t rl = npos - c->cfg.n_recent;
  k.recent_lo = static_cast<int>(std::max<int64_t>(rl, -1));
  const int64_t full = rl >= 0 ? rl / W : 0;
  k.na = static_cast<int>(std::max<int64_t>(0, full - k.np));
  return k;
}

}  // namespace

void tier_free(kvev_ctx* c) {
  auto& t = c->td;
  void* ptrs[] = {t.kfp, t.vfp, t.ledger, t.tier, t.hasled, t.forced, t.S,
                  t.fplist, t.qlist, t.jobs, t.njobs, t.emass, t.rd_fstamp, t.rd_rstamp,
                  t.rd_run, t.rd_cnt, t.rd_acc, t.kpre, t.rcs, t.ifreq, t.kst, t.vst, t.kpst,
                  t.fslot, t.lslot, t.ffree};
  for (void* p : ptrs)
    if (p) hipFree(p);
  t = TierDev{};
}

namespace {

// Releases the prefill staging buffers (every prefill window has been placed
// by the first routing event).  Synchronises once.
hipError_t tier_release_staging(kvev_ctx* c) {
  auto& t = c->td;
  if (!t.kst) return hipSuccess;
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return e;
  for (uint16_t** p : {&t.kst, &t.vst, &t.kpst})
    if (*p) {
      hipFree(*p);
      *p = nullptr;
    }
  c->tw.NWS = 0;
  c->tw.stage_done = false;
  return hipSuccess;
}

// The free full-precision slots 0 .. SF-1 of every layer, ascending, and
// no window holding a slot or a record.
hipError_t tier_reset_slots(kvev_ctx* c) {
  auto& t = c->td;
  const size_t L = c->cfg.n_layers, lw = L * c->tw.NW, SF = c->tw.SF;
  std::vector<int> fr(L * SF);
  for (size_t l = 0; l < L; ++l)
    for (size_t i = 0; i < SF; ++i) fr[l * SF + i] = static_cast<int>(i);
  hipError_t e = hipMemcpyAsync(t.ffree, fr.data(), fr.size() * sizeof(int), hipMemcpyHostToDevice, c->stream);
  if (e == hipSuccess) e = hipMemsetAsync(t.fslot, 0xff, lw * sizeof(int), c->stream);
  if (e == hipSuccess) e = hipMemsetAsync(t.lslot, 0xff, lw * sizeof(int), c->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);  // fr is a host buffer
  c->tw.held = 0;
  c->tw.opened = 0;
  return e;
}

}  // namespace

hipError_t tier_alloc(kvev_ctx* c) {
  const auto& f = c->cfg;
  auto& t = c->td;
  auto& d = c->d;
  const int64_t L = f.n_layers, H = f.n_kv_heads, NW = c->tw.NW;
  const size_t win = static_cast<size_t>(L) * H * NW;
  const size_t lw = static_cast<size_t>(L) * NW;
  hipError_t e = hipSuccess;
  auto A = [&](hipError_t r) {
    if (e == hipSuccess && r != hipSuccess) e = r;
  };
  const size_t W = c->tw.W, recb = tier_rec_bytes(c->tw.W);
  // Slot pools ("QEvict" review, section 4.1 (Budget), section 4.3 Eq.3):
  // full-precision slots for the pinned windows, the local and not yet
  // routed ones (the n_recent newest positions plus a routing interval of
  // new tokens) and K_f routed windows (and the K_q INT2 windows when they
  // are read through bf16 reconstructions); records for the K_f + K_q routed
  // windows kept (a promoted window keeps its record for its next demotion).
  {
    const int Wi = c->tw.W, nwi = c->tw.NW;
    const int np = f.n_sink > 0 ? (f.n_sink + Wi - 1) / Wi : 0;
    const int omega = std::max(f.route_interval, 1);
    const int64_t reserve = (static_cast<int64_t>(f.n_recent) + omega + Wi - 1) / Wi + 4;
    const int64_t sf = np + reserve + f.fp_windows + (c->tw.mat ? static_cast<int64_t>(f.int2_windows) : 0);
    const int64_t sq = static_cast<int64_t>(f.fp_windows) + f.int2_windows;
    c->tw.SF = static_cast<int>(std::min<int64_t>(nwi, sf));
    c->tw.SQ = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(nwi, sq)));
  }
  const size_t fpw = static_cast<size_t>(L) * H * c->tw.SF, qw = static_cast<size_t>(L) * H * c->tw.SQ;
  A(dalloc(&t.kfp, fpw * W * kTierD));
  A(dalloc(&t.vfp, fpw * W * kTierD));
  A(dalloc(&t.ledger, qw * recb));
  A(dalloc(&t.fslot, lw));
  A(dalloc(&t.lslot, lw));
  A(dalloc(&t.ffree, static_cast<size_t>(L) * c->tw.SF));
  if (c->tw.rope) {
    A(dalloc(&t.kpre, fpw * W * kTierD));
    A(dalloc(&t.rcs, static_cast<size_t>(c->cap) * 64 * 2));
    A(dalloc(&t.ifreq, 64));
  }
  A(dalloc(&t.tier, lw));
  A(dalloc(&t.hasled, lw));
  A(dalloc(&t.forced, lw));
  A(dalloc(&t.S, lw));
  A(dalloc(&t.fplist, lw));
  A(dalloc(&t.qlist, lw));
  A(dalloc(&t.jobs, lw));
  A(dalloc(&t.njobs, L));
  A(dalloc(&t.emass, win * 4));
  const size_t parts = static_cast<size_t>(L) * H * c->tw.maxch * 4;
  A(dalloc(&d.part_ml, parts * 2));
  A(dalloc(&d.part_o, parts * kTierD));
  A(dalloc(&d.ml, static_cast<size_t>(L) * H * 4 * 2));
  A(dalloc(&d.errflag, 1));
  if (f.revival_gap > 0) {
    A(dalloc(&t.rd_fstamp, lw));
    A(dalloc(&t.rd_rstamp, lw));
    A(dalloc(&t.rd_run, lw));
    A(dalloc(&t.rd_cnt, static_cast<size_t>(L) * 6));
    A(dalloc(&t.rd_acc, static_cast<size_t>(L) * 6));
  }
  if (e != hipSuccess) return e;
  if (f.revival_gap > 0) {
    A(hipMemsetAsync(t.rd_fstamp, 0, lw * sizeof(int), c->stream));
    A(hipMemsetAsync(t.rd_rstamp, 0, lw * sizeof(int), c->stream));
    A(hipMemsetAsync(t.rd_run, 0, lw * sizeof(int), c->stream));
    A(hipMemsetAsync(t.rd_cnt, 0, L * 6 * sizeof(int), c->stream));
    A(hipMemsetAsync(t.rd_acc, 0, L * 6 * sizeof(double), c->stream));
  }
  // zero the storage so that unwritten rows are finite
  A(hipMemsetAsync(t.kfp, 0, fpw * W * kTierD * 2, c->stream));
  A(hipMemsetAsync(t.vfp, 0, fpw * W * kTierD * 2, c->stream));
  A(hipMemsetAsync(t.ledger, 0, qw * recb, c->stream));
  if (c->tw.rope) {
    // the rotary frequencies theta^(-2i/128), i < 64, in fp64 on the host
    double fr[64];
    for (int i = 0; i < 64; ++i) fr[i] = std::pow(static_cast<double>(f.rope_theta), -2.0 * i / 128.0);
    A(hipMemsetAsync(t.kpre, 0, fpw * W * kTierD * 2, c->stream));
    A(hipMemcpyAsync(t.ifreq, fr, sizeof(fr), hipMemcpyHostToDevice, c->stream));
  }
  A(hipMemsetAsync(t.tier, 0, lw, c->stream));
  A(hipMemsetAsync(t.hasled, 0, lw, c->stream));
  A(hipMemsetAsync(t.S, 0, lw * sizeof(float), c->stream));
  A(hipMemsetAsync(t.njobs, 0, L * sizeof(int), c->stream));
  // list entries past the live lengths stay valid window ids (0)
  A(hipMemsetAsync(t.fplist, 0, lw * sizeof(int), c->stream));
  A(hipMemsetAsync(t.qlist, 0, lw * sizeof(int), c->stream));
  A(hipMemsetAsync(t.jobs, 0, lw * sizeof(int4), c->stream));
  A(hipMemsetAsync(d.errflag, 0, sizeof(int), c->stream));
  A(hipStreamSynchronize(c->stream));
  if (e == hipSuccess) e = tier_reset_slots(c);
  return e;
}

kvev_status tier_prefill(kvev_ctx* c, int seq, const void* k, const void* v, int64_t n) {
  if (seq != 0) return fail(c, KVEV_EINVAL, "tiered mode: the only sequence is 0");
  if (n < 1 || n + 1 > c->cap) return fail(c, KVEV_EINVAL, "n_tokens out of range for max_tokens");
  auto& tw = c->tw;
  // the prefill windows go to staging buffers until the first routing event
  // places them (full precision into the pool, INT2 into records, or evicted)
  KVEV_HIP(c, tier_release_staging(c));
  KVEV_HIP(c, tier_reset_slots(c));
  {
    const int nwin = static_cast<int>((n + tw.W - 1) / tw.W);
    const size_t sw = static_cast<size_t>(c->cfg.n_layers) * c->cfg.n_kv_heads * nwin * tw.W * kTierD;
    hipError_t e = dalloc(&c->td.kst, sw);
    if (e == hipSuccess) e = dalloc(&c->td.vst, sw);
    if (e == hipSuccess && tw.rope) e = dalloc(&c->td.kpst, sw);
    if (e != hipSuccess) {
      (void)tier_release_staging(c);
      return fail(c, KVEV_ENOMEM, "out of device memory for the prefill staging buffers");
    }
    tw.NWS = nwin;
  }
  if (c->tw.rope) KVEV_HIP(c, launch_tier_rope_table(c, 0, n));
  KVEV_HIP(c, launch_tier_prefill(c, k, v, n));
  tw.npos = n;
  tw.n_fp = static_cast<int>((n + tw.W - 1) / tw.W);
  tw.n_q = 0;
  tw.n_kept = 0;
  tw.na_prev = 0;
  c->prefilled[0] = 1;
  return KVEV_OK;
}

kvev_status tier_decode(kvev_ctx* c, const void* q, const void* k_new, const void* v_new, float* out) {
  if (!q || !k_new || !v_new || !out) return fail(c, KVEV_EINVAL, "null argument");
  if (!c->prefilled[0]) return fail(c, KVEV_ESTATE, "the sequence has no prefill");
  auto& tw = c->tw;
  if (tw.npos + 1 > c->cap) return fail(c, KVEV_ESTATE, "position capacity exhausted");
  const bool opens = tw.npos % tw.W == 0;
  if (opens && tw.opened >= tw.SF - tw.held)
    return fail(c, KVEV_ESTATE, "full-precision slot pool exhausted: route at least every route_interval steps");
  if (tw.stage_done) KVEV_HIP(c, tier_release_staging(c));
  // every launch of the step times itself from its own dispatch (kvev_profile_*)
  if (tw.rope) KVEV_HIP(c, launch_tier_rope_table(c, tw.npos, 1));
  KVEV_HIP(c, launch_tier_append(c, k_new, v_new, opens ? tw.opened : 0));
  if (opens) {
    tw.n_fp += 1;
    tw.opened += 1;
  }
  tw.npos += 1;
  KVEV_HIP(c, launch_tier_attention(c, q));
  KVEV_HIP(c, launch_tier_merge(c, out));
  c->t += 1;
  return KVEV_OK;
}

kvev_status tier_route(kvev_ctx* c) {
  if (!c->prefilled[0]) return fail(c, KVEV_ESTATE, "the sequence has no prefill");
  auto& tw = c->tw;
  const Counts k = tier_counts(c);
  const int cand = tw.n_kept + (k.na - tw.na_prev);
  const int nF = std::min(c->cfg.fp_windows, cand);
  const int nQ = std::min(c->cfg.int2_windows, cand - nF);
  const int exp_fp = k.np + (k.nw - k.np - k.na) + nF;
  KVEV_HIP(c, launch_tier_route(c, k.nw, k.np, k.recent_lo, exp_fp, nQ, nullptr, -1));
  tw.n_fp = exp_fp;
  tw.n_q = nQ;
  tw.held = exp_fp + (tw.mat ? nQ : 0);
  tw.opened = 0;
  if (tw.NWS) tw.stage_done = true;
  tw.n_kept = nF + nQ;
  tw.na_prev = k.na;
  tw.events += 1;
  return KVEV_OK;
}

kvev_status tier_scores(kvev_ctx* c, int layer, float* dst, int64_t cap, int64_t* n) {
  return kvev_tier_state(c, layer, dst, nullptr, nullptr, cap, n);
}

}  // namespace kvev

using namespace kvev;

extern "C" {

kvev_status kvev_tier_diag(kvev_ctx* c, int32_t layer, kvev_route_diag* out) {
  KVEV_LIVE(c);
  if (!c->tier_mode) return fail(c, KVEV_EINVAL, "not in tiered mode");
  if (c->cfg.revival_gap <= 0 || !c->td.rd_cnt) return fail(c, KVEV_ESTATE, "routing diagnostics are off");
  if (layer < 0 || layer >= c->cfg.n_layers || !out) return fail(c, KVEV_ERANGE, "layer out of range or null output");
  int cn[6];
  double ac[6];
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  KVEV_HIP(c, hipMemcpy(cn, c->td.rd_cnt + layer * 6, sizeof(cn), hipMemcpyDeviceToHost));
  KVEV_HIP(c, hipMemcpy(ac, c->td.rd_acc + layer * 6, sizeof(ac), hipMemcpyDeviceToHost));
  out->f_prev = cn[0];
  out->f_new = cn[1];
  out->f_overlap = cn[2];
  out->r_prev = cn[3];
  out->r_new = cn[4];
  out->r_overlap = cn[5];
  out->events = static_cast<int64_t>(ac[0]);
  out->pairs = static_cast<int64_t>(ac[1]);
  out->sum_f_churn = ac[2];
  out->sum_r_churn = ac[3];
  out->sustained = static_cast<int64_t>(ac[4]);
  out->revived = static_cast<int64_t>(ac[5]);
  return KVEV_OK;
}

kvev_status kvev_tier_state(kvev_ctx* c, int32_t layer, float* score, uint8_t* tier, uint8_t* ledger,
                            int64_t cap, int64_t* n_windows) {
  KVEV_LIVE(c);
  if (!c->tier_mode) return fail(c, KVEV_EINVAL, "not in tiered mode");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, KVEV_EINVAL, "layer out of range");
  const int64_t nw = (c->tw.npos + c->tw.W - 1) / c->tw.W;
  if (n_windows) *n_windows = nw;
  if (cap < nw) return fail(c, KVEV_ERANGE, "destination too small");
  const int64_t off = static_cast<int64_t>(layer) * c->tw.NW;
  if (score)
    KVEV_HIP(c, hipMemcpyAsync(score, c->td.S + off, sizeof(float) * nw, hipMemcpyDeviceToHost, c->stream));
  if (tier) KVEV_HIP(c, hipMemcpyAsync(tier, c->td.tier + off, nw, hipMemcpyDeviceToHost, c->stream));
  if (ledger)
    KVEV_HIP(c, hipMemcpyAsync(ledger, c->td.hasled + off, nw, hipMemcpyDeviceToHost, c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  return KVEV_OK;
}

kvev_status kvev_tier_export(kvev_ctx* c, int32_t layer, int32_t h, void* k_out, void* v_out,
                             int64_t cap, int64_t* n_rows) {
  KVEV_LIVE(c);
  if (!c->tier_mode) return fail(c, KVEV_EINVAL, "not in tiered mode");
  if (layer < 0 || layer >= c->cfg.n_layers || h < 0 || h >= c->cfg.n_kv_heads)
    return fail(c, KVEV_EINVAL, "layer or KV head out of range");
  const int nw = static_cast<int>((c->tw.npos + c->tw.W - 1) / c->tw.W);
  const int64_t rows = static_cast<int64_t>(nw) * c->tw.W;
  if (n_rows) *n_rows = rows;
  if (!k_out || !v_out || cap < rows) return fail(c, KVEV_ERANGE, "destination too small");
  if (nw > 0) KVEV_HIP(c, launch_tier_export(c, layer, h, k_out, v_out, nw));
  return KVEV_OK;
}

// The key parameters of a record: per channel [128], or with key groups
// stored [group][W] and exported [W][group].
static void tier_key_params(const kvev_ctx* c, const uint8_t* s_src, const uint8_t* z_src, int W,
                            uint16_t* k_scale, uint16_t* k_zero) {
  if (!c->tw.kgroups) {
    std::memcpy(k_scale, s_src, 256);
    std::memcpy(k_zero, z_src, 256);
    return;
  }
  uint16_t s[4 * kTierWin], z[4 * kTierWin];
  std::memcpy(s, s_src, 8 * W);
  std::memcpy(z, z_src, 8 * W);
  for (int r = 0; r < W; ++r)
    for (int g = 0; g < 4; ++g) {
      k_scale[r * 4 + g] = s[g * W + r];
      k_zero[r * 4 + g] = z[g * W + r];
    }
}

kvev_status kvev_tier_ledger(kvev_ctx* c, int32_t layer, int32_t h, int32_t w, uint8_t* k_codes,
                             uint16_t* k_scale, uint16_t* k_zero, uint8_t* v_codes, uint16_t* v_scale,
                             uint16_t* v_zero) {
  KVEV_LIVE(c);
  if (!c->tier_mode) return fail(c, KVEV_EINVAL, "not in tiered mode");
  const int W = c->tw.W, recb = tier_rec_bytes(W);
  const int nw = static_cast<int>((c->tw.npos + W - 1) / W);
  if (layer < 0 || layer >= c->cfg.n_layers || h < 0 || h >= c->cfg.n_kv_heads || w < 0 || w >= nw)
    return fail(c, KVEV_EINVAL, "layer, KV head or window out of range");
  if (!k_codes || !k_scale || !k_zero || !v_codes || !v_scale || !v_zero)
    return fail(c, KVEV_EINVAL, "null argument");
  uint8_t flag = 0;
  int slot = -1;
  const int64_t lw = static_cast<int64_t>(layer) * c->tw.NW + w;
  std::vector<uint8_t> rec(recb);
  KVEV_HIP(c, hipMemcpyAsync(&flag, c->td.hasled + lw, 1, hipMemcpyDeviceToHost, c->stream));
  KVEV_HIP(c, hipMemcpyAsync(&slot, c->td.lslot + lw, sizeof(int), hipMemcpyDeviceToHost, c->stream));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));
  if (!flag || slot < 0) return fail(c, KVEV_EINVAL, "window holds no INT2 record");
  const int64_t roff = ((static_cast<int64_t>(layer) * c->cfg.n_kv_heads + h) * c->tw.SQ + slot) * recb;
  KVEV_HIP(c, hipMemcpy(rec.data(), c->td.ledger + roff, recb, hipMemcpyDeviceToHost));
  if (W == 8) {
    // 8-token record: key / value codes [8][128] at 2 bits (element e at
    // byte e / 4, bits 2 (e % 4)), key scale / zero [128], value scale /
    // zero [4][8] (fp16)
    for (int e = 0; e < 8 * kTierD; ++e) {
      k_codes[e] = static_cast<uint8_t>((rec[e / 4] >> (2 * (e % 4))) & 3);
      v_codes[e] = static_cast<uint8_t>((rec[256 + e / 4] >> (2 * (e % 4))) & 3);
    }
    tier_key_params(c, rec.data() + 512, rec.data() + 768, 8, k_scale, k_zero);
    uint16_t vs8[4][8], vz8[4][8];
    std::memcpy(vs8, rec.data() + 1024, 64);
    std::memcpy(vz8, rec.data() + 1088, 64);
    for (int r = 0; r < 8; ++r)
      for (int g = 0; g < 4; ++g) {
        v_scale[r * 4 + g] = vs8[g][r];
        v_zero[r * 4 + g] = vz8[g][r];
      }
    return KVEV_OK;
  }
  uint32_t words[2][256];
  std::memcpy(words[0], rec.data(), 1024);
  std::memcpy(words[1], rec.data() + 1024, 1024);
  // element k of a 16-code word sits at bits 8 (k % 4) + 2 (k / 4); key word
  // 4 lane + 2 j + ks of lane (r16, q4) holds token 16 j + r16, channels
  // 64 ks + 16 q4 .. +16; value word (hf 16 + r16) 8 + ct holds channel
  // 16 ct + r16, tokens 16 hf .. +16 (layout in tier.hip)
  auto bit = [](int k) { return 8 * (k & 3) + 2 * (k >> 2); };
  for (int r = 0; r < kTierWin; ++r)
    for (int ch = 0; ch < kTierD; ++ch) {
      const int ln = ((ch >> 4) & 3) * 16 + (r & 15);
      k_codes[r * kTierD + ch] =
          static_cast<uint8_t>((words[0][4 * ln + 2 * (r >> 4) + (ch >> 6)] >> bit(ch & 15)) & 3u);
      v_codes[r * kTierD + ch] =
          static_cast<uint8_t>((words[1][((r >> 4) * 16 + (ch & 15)) * 8 + (ch >> 4)] >> bit(r & 15)) & 3u);
    }
  tier_key_params(c, rec.data() + 2048, rec.data() + 2304, kTierWin, k_scale, k_zero);
  // value scales and zero points are stored [group][token]; the export is [token][group]
  uint16_t vs[4][kTierWin], vz[4][kTierWin];
  std::memcpy(vs, rec.data() + 2560, 256);
  std::memcpy(vz, rec.data() + 2816, 256);
  for (int r = 0; r < kTierWin; ++r)
    for (int g = 0; g < 4; ++g) {
      v_scale[r * 4 + g] = vs[g][r];
      v_zero[r * 4 + g] = vz[g][r];
    }
  return KVEV_OK;
}

kvev_status kvev_tier_import(kvev_ctx* c, int32_t layer, int64_t n_windows, const float* score,
                             const uint8_t* tier) {
  KVEV_LIVE(c);
  if (!c->tier_mode) return fail(c, KVEV_EINVAL, "not in tiered mode");
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, KVEV_EINVAL, "layer out of range");
  if (!score || !tier) return fail(c, KVEV_EINVAL, "null argument");
  if (!c->prefilled[0]) return fail(c, KVEV_ESTATE, "the sequence has no prefill");
  const Counts k = tier_counts(c);
  if (n_windows != k.nw) return fail(c, KVEV_EINVAL, "n_windows must equal the windows seen");
  int nf = 0, nq = 0;
  for (int w = 0; w < k.nw; ++w) {
    if (tier[w] > 2) return fail(c, KVEV_EINVAL, "tier code out of range");
    nf += tier[w] == 0;
    nq += tier[w] == 1;
    const bool aged = w >= k.np && (w + 1) * c->tw.W <= k.recent_lo;
    if (!aged && tier[w] != 0) return fail(c, KVEV_EINVAL, "pinned and local windows must be full precision");
  }
  if (nf != c->tw.n_fp || nq != c->tw.n_q)
    return fail(c, KVEV_EINVAL, "tier counts differ from the context's");
  const int64_t off = static_cast<int64_t>(layer) * c->tw.NW;
  const size_t lw = static_cast<size_t>(c->cfg.n_layers) * c->tw.NW;
  KVEV_HIP(c, hipMemcpyAsync(c->td.forced, c->td.tier, lw, hipMemcpyDeviceToDevice, c->stream));
  KVEV_HIP(c, hipMemcpyAsync(c->td.forced + off, tier, k.nw, hipMemcpyHostToDevice, c->stream));
  KVEV_HIP(c, hipMemcpyAsync(c->td.S + off, score, sizeof(float) * k.nw, hipMemcpyHostToDevice, c->stream));
  KVEV_HIP(c, launch_tier_route(c, k.nw, k.np, k.recent_lo, c->tw.n_fp, c->tw.n_q, c->td.forced, -1));
  KVEV_HIP(c, hipStreamSynchronize(c->stream));  // host buffers are the caller's
  c->tw.held = c->tw.n_fp + (c->tw.mat ? c->tw.n_q : 0);
  c->tw.opened = 0;
  if (c->tw.NWS) c->tw.stage_done = true;
  int flag = 0;
  KVEV_HIP(c, hipMemcpy(&flag, c->d.errflag, sizeof(int), hipMemcpyDeviceToHost));
  if (flag & 64) return fail(c, KVEV_ESTATE, "an evicted window cannot be kept: its storage is released");
  return KVEV_OK;
}

}  // extern "C"

kvev_status kvev_tier_footprint(kvev_ctx* c, int64_t* fp_pool, int64_t* record_pool, int64_t* staging,
                                int32_t* fp_slots, int32_t* record_slots) {
  KVEV_LIVE(c);
  if (!c->tier_mode) return fail(c, KVEV_EINVAL, "not in tiered mode");
  const int64_t lh = static_cast<int64_t>(c->cfg.n_layers) * c->cfg.n_kv_heads;
  const int64_t win = static_cast<int64_t>(c->tw.W) * kTierD * 2;  // bytes of one window's keys (or values)
  const int64_t per = (c->tw.rope ? 3 : 2) * win;                 // keys, values, keys before the rotation
  if (fp_pool) *fp_pool = lh * c->tw.SF * per;
  if (record_pool) *record_pool = lh * c->tw.SQ * tier_rec_bytes(c->tw.W);
  if (staging) *staging = lh * c->tw.NWS * per;
  if (fp_slots) *fp_slots = c->tw.SF;
  if (record_slots) *record_slots = c->tw.SQ;
  return KVEV_OK;
}

kvev_status kvev_tier_capacities(double b_hist, double q, double m_f, double m_q, int32_t* k_f,
                                 int32_t* k_q) {
  if (!k_f || !k_q) return KVEV_EINVAL;
  if (!std::isfinite(b_hist) || !std::isfinite(q) || !std::isfinite(m_f) || !std::isfinite(m_q))
    return KVEV_EINVAL;
  if (q < 0.0 || q > 1.0 || b_hist < 0.0 || !(m_f > 0.0) || !(m_q > 0.0)) return KVEV_EINVAL;
  const double f = std::floor((1.0 - q) * b_hist / m_f);
  const double g = std::floor(q * b_hist / m_q);
  if (f > 2147483647.0 || g > 2147483647.0) return KVEV_EINVAL;
  *k_f = static_cast<int32_t>(f);
  *k_q = static_cast<int32_t>(g);
  return KVEV_OK;
}
