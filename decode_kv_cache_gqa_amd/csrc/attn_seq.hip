// Whole-cache GQA decode attention per (layer, group): one workgroup reads
// every retained slot of one (sequence, KV head) group at one layer, so the
// softmax statistics are final inside the workgroup.  It writes the
// attention output and, on an observation step, the group's probability
// mass per slot, G[t] = sum_{h in group} exp(s_h[t] - M_h) / Z_h
// ("QEvict" review, section 4.1 (Attention): s = q.k / sqrt(d); "What
// Matters ...", section 3.1 Eq.1 with appendix E's GQA sharing: the KV
// head's query group pooled by summation).  No split partials and no
// per-slot logits leave the chip: the logits stay in LDS until the
// probability pass.  The step's new token is appended on the way (it takes
// the group's free slot, hole[g]).
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16, 32 slots = two pages per
// iteration):
//   q.K^T  C[16 slots][16 heads] = K (A: lane (slot r16, k-group q4) holds
//          channels 32s + 8q4 .. +8 of a token-major K page row) x Q^T (B:
//          lane (head r16, q4) holds the same channels of query head r16;
//          heads >= HG are zero).  Lane (head r16, q4) receives the logits
//          of slots 4q4 .. 4q4+3 of the tile.
//   p.V    C[16 channels][16 heads] = V^T x P^T over a k-block of 32 slots
//          ordered sigma(8q4 + e) = 16 (e >> 2) + 4q4 + (e & 3): then the
//          probabilities a lane holds after q.K^T of the two tiles are
//          exactly its B operand, and its A operand is slots 4q4 .. 4q4+3 of
//          one channel in each of the two channel-major V pages (8 bytes
//          each).  P is split into bf16 high and low parts (two products),
//          so its rounding is at most 2^-18 relative.
// The online softmax keeps one running maximum and sum per lane (its head)
// and rescales the accumulator, whose lanes hold the same head.  Each wave
// streams a contiguous range of chunks with the next chunk's K and V loads
// in flight while the current one is computed.
#include "common.h"
#include "kvev_internal.h"

namespace kvev {

typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
typedef float f32x4s __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4s __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2s __attribute__((ext_vector_type(2)));

// bit casts between same-size vector types (registers only)
__device__ __forceinline__ bf16x8s to_bf16x8(u32x4s r) { return __builtin_bit_cast(bf16x8s, r); }

// replace 16-bit element e (0..3) of an 8-byte register pair (values
// selected, never an address: the pair stays in registers)
__device__ __forceinline__ u32x2s put16x4(u32x2s r, int e, uint32_t x) {
  const int sh = (e & 1) * 16;
  const uint32_t m = ~(0xffffu << sh);
  const uint32_t v = (x & 0xffffu) << sh;
  const bool hi = (e >> 1) != 0;
  u32x2s o;
  o.x = hi ? r.x : ((r.x & m) | v);
  o.y = hi ? ((r.y & m) | v) : r.y;
  return o;
}

// The registers of one 32-slot chunk: K rows of its two pages (A operands
// of q.K^T) and the V pieces of its two pages (A operands of p.V).
struct SeqChunk {
  u32x4s k[2][4];  // [page of the chunk][k-step]
  u32x2s v[2][8];  // [page of the chunk][channel tile]
};

// Loads of chunk c from the group's pages (slots past the group's count are
// masked, so their values never count).  The cache is read once per step:
// non-temporal loads keep it from displacing reused lines.
template <bool PG>
__device__ __forceinline__ void seq_load(SeqChunk& ch, const uint16_t* __restrict__ kpool,
                                         const uint16_t* __restrict__ vpool, int page0, const int* s_pt,
                                         int maxpages, int c, int l, int r16, int q4, int64_t P) {
  constexpr int D = 128;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int page = PG ? s_pt[2 * c + j] : page0 + min(2 * c + j, maxpages - 1);
    const uint16_t* kb = kpool + kidx(l, page, r16, 8 * q4, P, D);
    const uint16_t* vb = vpool + vidx(l, page, 4 * q4, r16, P, D);
#pragma unroll
    for (int s = 0; s < 4; ++s) ch.k[j][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4s*>(kb + 32 * s));
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      ch.v[j][ct] = __builtin_nontemporal_load(reinterpret_cast<const u32x2s*>(vb + ct * 16 * kPageTokens));
  }
}

// One chunk: append of the new token (when the chunk holds the free slot),
// q.K^T, online softmax, p.V.
template <int HG, bool OBS, bool PG>
__device__ __forceinline__ void seq_step(SeqChunk& ch, int c, int n, bool app, int tnew, const u32x4s (&knew)[4],
                                         const uint32_t (&vnew)[8], int page0, const int* s_pt,
                                         uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool, int l,
                                         int r16, int q4, int64_t P, bool head, const bf16x8s (&qb)[4],
                                         float scale, float* s_lg, float* s_mc, int nstride, f32x4s (&oacc)[8],
                                         float& m_run, float& l_run) {
  constexpr int D = 128;
  // append: the new token replaces the free slot's stale contents (per-lane
  // selects with constant indices) and is written into its page
  if (app && (tnew >> 5) == c) {  // wave-uniform
    const int jn = (tnew >> 4) & 1, rn = tnew & 15;
    const int page = PG ? s_pt[2 * c + jn] : page0 + 2 * c + jn;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool krow = j == jn && r16 == rn;
      const bool vcol = j == jn && q4 == (rn >> 2);
#pragma unroll
      for (int s = 0; s < 4; ++s) ch.k[j][s] = krow ? knew[s] : ch.k[j][s];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) ch.v[j][ct] = vcol ? put16x4(ch.v[j][ct], rn & 3, vnew[ct]) : ch.v[j][ct];
    }
    // block mode: the rows are written through to memory (sc1; measured 2%
    // shorter launches on the 64-sequence workload, where every one of the
    // 16,384 workgroups appends; 3% longer on the 32k workload, which keeps
    // plain stores)
    if (r16 == rn) {
      uint16_t* kd = kpool + kidx(l, page, rn, 8 * q4, P, D);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (PG) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __hip_atomic_store(reinterpret_cast<uint32_t*>(kd + 32 * s) + i, static_cast<uint32_t>(knew[s][i]),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          *reinterpret_cast<u32x4s*>(kd + 32 * s) = knew[s];
        }
      }
    }
    if (q4 == (rn >> 2)) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        uint16_t* vd = &vpool[vidx(l, page, rn, 16 * ct + r16, P, D)];
        if constexpr (PG)
          __hip_atomic_store(vd, static_cast<uint16_t>(vnew[ct]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *vd = static_cast<uint16_t>(vnew[ct]);
      }
    }
  }
  // q.K^T of the two 16-slot tiles
  float sv[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    f32x4s acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(to_bf16x8(ch.k[j][s]), qb[s], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 32 * c + 16 * j + 4 * q4 + i;
      sv[j][i] = (head && t < n) ? acc[i] * scale : -INFINITY;
    }
  }
  // online softmax (the four lane quarters of a head hold its 32 slots)
  float mc = fmaxf(fmaxf(fmaxf(sv[0][0], sv[0][1]), fmaxf(sv[0][2], sv[0][3])),
                   fmaxf(fmaxf(sv[1][0], sv[1][1]), fmaxf(sv[1][2], sv[1][3])));
  mc = fmaxf(mc, __shfl_xor(mc, 16, kWave));
  mc = fmaxf(mc, __shfl_xor(mc, 32, kWave));
  const float m_new = fmaxf(m_run, mc);
  const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = sv[j][i] == -INFINITY ? 0.f : __expf(sv[j][i] - m_new);
      sv[j][i] = p;
      psum += p;
    }
  l_run = l_run * alpha + psum;
  m_run = m_new;
  if constexpr (OBS && PG) {
    // block table: the chunk's two 16-slot tiles are table entries 2c and
    // 2c + 1; per head, each tile's probability sum relative to the running
    // maximum, and that maximum (the four lane quarters hold a tile's slots)
    float bs[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bs[j] = (sv[j][0] + sv[j][1]) + (sv[j][2] + sv[j][3]);
      bs[j] += __shfl_xor(bs[j], 16, kWave);
      bs[j] += __shfl_xor(bs[j], 32, kWave);
    }
    if (head && q4 == 0) {
      s_lg[(2 * c) * HG + r16] = bs[0];
      s_lg[(2 * c + 1) * HG + r16] = bs[1];
      s_mc[c * HG + r16] = m_new;
    }
  } else if (OBS && head) {
    // the chunk's probabilities relative to its running maximum, and that
    // maximum: the probability pass rescales them once M and Z are known
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *reinterpret_cast<float4*>(&s_lg[r16 * nstride + 32 * c + 16 * j + 4 * q4]) =
          make_float4(sv[j][0], sv[j][1], sv[j][2], sv[j][3]);
    if (q4 == 0) s_mc[c * HG + r16] = m_new;
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) oacc[ct][i] *= alpha;
  // p.V: B = P^T in the sigma order, split into bf16 high and low parts
  uint32_t h16[8], l16[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = sv[e >> 2][e & 3];
    h16[e] = bf16_rne(x);
    l16[e] = bf16_rne(x - __uint_as_float(h16[e] << 16));
  }
  const bf16x8s phi = to_bf16x8(u32x4s{h16[0] | (h16[1] << 16), h16[2] | (h16[3] << 16),
                                        h16[4] | (h16[5] << 16), h16[6] | (h16[7] << 16)});
  const bf16x8s plo = to_bf16x8(u32x4s{l16[0] | (l16[1] << 16), l16[2] | (l16[3] << 16),
                                        l16[4] | (l16[5] << 16), l16[6] | (l16[7] << 16)});
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const bf16x8s va = to_bf16x8(u32x4s{ch.v[0][ct].x, ch.v[0][ct].y, ch.v[1][ct].x, ch.v[1][ct].y});
    oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, oacc[ct], 0, 0, 0);
    oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, oacc[ct], 0, 0, 0);
  }
}

// A store written through the L2 to memory (relaxed agent-scope atomic
// store: global_store ... sc1).
__device__ __forceinline__ void st_through(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A head's overall maximum M and normaliser Z from the waves' (m, l).
template <int NW, int HG>
__device__ __forceinline__ void head_stats(const float (&wm)[NW][HG], const float (&wl)[NW][HG], int h, float& M,
                                           float& Z) {
  M = -INFINITY;
#pragma unroll
  for (int x = 0; x < NW; ++x) M = fmaxf(M, wm[x][h]);
  Z = 0.f;
#pragma unroll
  for (int x = 0; x < NW; ++x) Z += wm[x][h] == -INFINITY ? 0.f : wl[x][h] * __expf(wm[x][h] - M);
}

// PG (block mode): the group's slots lie in the pages its block table
// names, ptab[g][e] for table entry e = slot / 16, and the step's new token
// takes slot count[g] (the last entry).  On an observation step the kernel
// writes, instead of per-slot masses, the group mass of every table entry,
// gmass[((b * L + l) * Hkv + kvh) * maxpages + e] = the sum of G[t] over
// the entry's 16 slots.
template <int NW, int HG, bool OBS, bool PG>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(2))) void attn_seq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool,
    const int* __restrict__ count, const int* __restrict__ hole, float* __restrict__ out,
    float* __restrict__ gmass, int L, int G, int Hkv, int Hq, int64_t P, int maxpages, int64_t lstride,
    int nstride, float scale, int nmax, const int* __restrict__ ptab) {
  static_assert(HG >= 1 && HG <= 8, "group size");
  constexpr int D = 128, NT = NW * kWave;
  extern __shared__ float dyn[];
  // observation steps: the probabilities (token mode [HG][nstride] per
  // slot; block mode [nstride / 16][HG] per table entry) and
  // [nstride / 32][HG] chunk maxima; then [NW][HG][D] per-wave outputs;
  // then (block mode) the page of every table entry the loads can reach
  const int nchm = (nmax + 31) / 32;  // chunks of the launch's slot bound (nstride / 32)
  float* s_lg = dyn;
  float* s_mc = dyn + (OBS ? (PG ? HG * 2 * nchm : HG * nstride) : 0);
  float* o_m = s_mc + (OBS ? HG * (nstride / 32) : 0);
  int* s_pt = reinterpret_cast<int*>(o_m + NW * HG * D);
  __shared__ float wm[NW][HG], wl[NW][HG], sf[NW][HG];

  const int g = blockIdx.x, l = blockIdx.y;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int Bsz = G / Hkv, b = g / Hkv, kvh = g % Hkv;
  const int64_t new_off = (static_cast<int64_t>(l * Bsz + b) * Hkv + kvh) * D;
  const bool head = r16 < HG;  // the lane's column is a real query head
  const int page0 = g * maxpages;  // the group's first page

  // Token mode: the chunk ranges come from the launch's slot bound nmax
  // (>= every group's slot count), and a group's logical page i is the pool
  // page g * maxpages + i, so the first page loads issue at once; slots past
  // the group's count are masked.  Block mode: the table's pages (entries
  // past the group's own, which only masked loads reach, and any value
  // outside the pool become the group's first page) are staged in LDS
  // beside the count, and the ranges split the group's own chunks evenly.
  int c0, c1;
  if constexpr (!PG) {
    const int nch = nchm;
    const int cpw = (nch + NW - 1) / NW;
    c0 = min(nch, wave * cpw);
    c1 = min(nch, c0 + cpw);
  }
  const int n = count[g] + 1;  // slots including the new token
  const int tnew = PG ? n - 1 : hole[g];
  if constexpr (PG) {
    const int* pt = ptab + static_cast<int64_t>(g) * maxpages;
    const int npg = (n + 15) / 16;
    for (int i = tid; i < 2 * nchm + 2; i += NT) {
      const int v = (i < npg && i < maxpages) ? pt[i] : page0;
      s_pt[i] = (v >= 0 && v < P) ? v : page0;
    }
    __syncthreads();
    const int nch = min((n + 31) / 32, nchm);
    c0 = wave * nch / NW;
    c1 = (wave + 1) * nch / NW;
  }

  // B operand of q.K^T: query head r16, channels 32s + 8q4 .. +8.  Lanes
  // past the group's heads repeat its last head: their logits are masked
  // to -inf, so their probabilities and outputs never count.
  bf16x8s qb[4];
  {
    const uint16_t* qp = q + (static_cast<int64_t>(l * Bsz + b) * Hq + kvh * HG + min(r16, HG - 1)) * D + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = to_bf16x8(*reinterpret_cast<const u32x4s*>(qp + 32 * s));
  }

  // the new token's K row piece and V column elements, used by the wave
  // whose range holds the free slot.  Every wave loads them: no load here
  // or in the chunk loop sits on a branch, so each wait covers exactly the
  // loads it needs.
  const bool app = tnew >= 32 * c0 && tnew < 32 * c1;  // wave-uniform
  u32x4s knew[4];
  uint32_t vnew[8];
#pragma unroll
  for (int s = 0; s < 4; ++s) knew[s] = *reinterpret_cast<const u32x4s*>(k_new + new_off + 32 * s + 8 * q4);
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) vnew[ct] = v_new[new_off + 16 * ct + r16];

  f32x4s oacc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) oacc[ct] = f32x4s{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // two chunks per iteration, one per register buffer: the next chunk's
  // loads are in flight while the current one is computed.  Every load in
  // the loop body is unconditional (the loop runs while two chunks remain
  // after the current one), so the wait before each chunk covers that
  // chunk's loads only; the last one or two chunks are peeled.
  // (a wave without chunks loads one in bounds and leaves it unused).  The
  // query and new-token loads stay ahead of the first chunk's, so that
  // waiting for them never waits for the chunk.
  SeqChunk cur, nxt;
  int c = c0;
  __builtin_amdgcn_sched_barrier(0);
  seq_load<PG>(cur, kpool, vpool, page0, s_pt, maxpages, c0, l, r16, q4, P);
#pragma unroll 1
  for (; c + 2 < c1; c += 2) {
    seq_load<PG>(nxt, kpool, vpool, page0, s_pt, maxpages, c + 1, l, r16, q4, P);
    seq_step<HG, OBS, PG>(cur, c, n, app, tnew, knew, vnew, page0, s_pt, kpool, vpool, l, r16, q4, P, head, qb,
                          scale, s_lg, s_mc, nstride, oacc, m_run, l_run);
    seq_load<PG>(cur, kpool, vpool, page0, s_pt, maxpages, c + 2, l, r16, q4, P);
    seq_step<HG, OBS, PG>(nxt, c + 1, n, app, tnew, knew, vnew, page0, s_pt, kpool, vpool, l, r16, q4, P, head, qb,
                          scale, s_lg, s_mc, nstride, oacc, m_run, l_run);
  }
  if (c + 1 < c1) {
    seq_load<PG>(nxt, kpool, vpool, page0, s_pt, maxpages, c + 1, l, r16, q4, P);
    seq_step<HG, OBS, PG>(cur, c, n, app, tnew, knew, vnew, page0, s_pt, kpool, vpool, l, r16, q4, P, head, qb,
                          scale, s_lg, s_mc, nstride, oacc, m_run, l_run);
    seq_step<HG, OBS, PG>(nxt, c + 1, n, app, tnew, knew, vnew, page0, s_pt, kpool, vpool, l, r16, q4, P, head, qb,
                          scale, s_lg, s_mc, nstride, oacc, m_run, l_run);
  } else if (c < c1) {
    seq_step<HG, OBS, PG>(cur, c, n, app, tnew, knew, vnew, page0, s_pt, kpool, vpool, l, r16, q4, P, head, qb,
                          scale, s_lg, s_mc, nstride, oacc, m_run, l_run);
  }

  // ---- merge the waves --------------------------------------------------------
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (head) {
    if (q4 == 0) {
      wm[wave][r16] = m_run;
      wl[wave][r16] = l_run;
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
      *reinterpret_cast<float4*>(&o_m[(wave * HG + r16) * D + 16 * ct + 4 * q4]) =
          make_float4(oacc[ct][0], oacc[ct][1], oacc[ct][2], oacc[ct][3]);
  }
  __syncthreads();
  // per (wave, head) weight of the wave's output, exp(m_wave - M) / Z, and
  // per (chunk, head) scale of the chunk's probabilities, exp(m_chunk - M) /
  // Z, with the head's overall maximum M and normaliser Z (a wave or chunk
  // without slots has m = -inf and weighs 0)
  if (tid < NW * HG) {
    const int w = tid / HG, h = tid % HG;
    float M, Z;
    head_stats<NW, HG>(wm, wl, h, M, Z);
    sf[w][h] = wm[w][h] == -INFINITY ? 0.f : __expf(wm[w][h] - M) / Z;
  }
  if constexpr (OBS) {
    const int nc = (n + 31) / 32;
    for (int i = tid; i < nc * HG; i += NT) {
      float M, Z;
      head_stats<NW, HG>(wm, wl, i % HG, M, Z);
      const float mc = s_mc[i];
      s_mc[i] = mc == -INFINITY ? 0.f : __expf(mc - M) / Z;
    }
  }
  __syncthreads();
  // token mode: the outputs and masses are written through to memory (sc1)
  // rather than left dirty in the L2 when the launch ends (measured about
  // 1 us shorter per launch on the 32k workload than plain stores; the
  // block mode's many rounds of workgroups gain nothing from it)
  for (int idx = tid; idx < HG * D; idx += NT) {
    const int h = idx / D, cc = idx % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) o += sf[w][h] * o_m[(w * HG + h) * D + cc];
    float* dst = &out[(static_cast<int64_t>(l * Bsz + b) * Hq + kvh * HG + h) * D + cc];
    if constexpr (PG)
      *dst = o;
    else
      st_through(dst, o);
  }
  if constexpr (OBS && PG) {
    // the group's mass of every table entry
    float* gm = gmass + (static_cast<int64_t>(b * L + l) * Hkv + kvh) * maxpages;
    const int ne = min((n + 15) / 16, 2 * nchm);
    for (int e = tid; e < ne; e += NT) {
      const float* f = s_mc + (e >> 1) * HG;
      float m = 0.f;
#pragma unroll
      for (int h = 0; h < HG; ++h) m += s_lg[e * HG + h] * f[h];
      gm[e] = m;
    }
  } else if constexpr (OBS) {
    // probability pass: the group's mass of every slot
    float* gm = gmass + (static_cast<int64_t>(g) * L + l) * lstride;
    for (int t = tid; t < n; t += NT) {
      const float* f = s_mc + (t >> 5) * HG;
      float m = 0.f;
#pragma unroll
      for (int h = 0; h < HG; ++h) m += s_lg[h * nstride + t] * f[h];
      st_through(&gm[t], m);
    }
  }
}

// Grid (groups, layers); dynamic LDS: the probabilities (observation
// steps), the per-wave outputs and (block mode) the staged page table.
// Workgroups of 8 waves when the grid is about one round of the chip (one
// workgroup per CU); of 4 waves when it is several rounds (two per CU, so
// that one's start and epilogue overlap the other's stream): measured on
// the 16 x 8k workloads 2.3% faster with 4, on the 32k one (256 workgroups)
// the same within 0.2%.  The block mode's grids are always many rounds.
constexpr int kSeqNW = 8;
constexpr int kSeqRoundsNW = 4;
constexpr int kSeqBlkNW = 4;

static int64_t lds_bytes(int hg, int64_t n_max, bool obs, bool paged, int nw) {
  const int64_t nstride = (n_max + 31) / 32 * 32, nchm = nstride / 32;
  const int64_t probs = obs ? (paged ? hg * 2 * nchm : hg * nstride) + hg * nchm : 0;
  return (probs + static_cast<int64_t>(nw) * hg * 128 + (paged ? 2 * nchm + 2 : 0)) * 4;
}

// the largest the launch can take (8 waves in the token modes)
int64_t seq_attn_lds_bytes(int hg, int64_t n_max, bool obs, bool paged) {
  return lds_bytes(hg, n_max, obs, paged, paged ? kSeqBlkNW : kSeqNW);
}

static hipError_t launch_seq(kvev_ctx* c, const void* q, const void* k_new, const void* v_new, float* out,
                             int n_max, bool obs, bool paged) {
  const auto& cf = c->cfg;
  const int nstride = (n_max + 31) / 32 * 32;
  const bool rounds = static_cast<int64_t>(c->G) * cf.n_layers >= 512;  // at least two rounds of 256 CUs
  const int nw = paged ? kSeqBlkNW : (rounds ? kSeqRoundsNW : kSeqNW);
  const size_t shm = static_cast<size_t>(lds_bytes(c->HG, n_max, obs, paged, nw));
  dim3 grid(c->G, cf.n_layers);
  // block mode: the entry masses go to the per-block buffer
  float* gm = paged ? c->d.bpart : c->d.logits;
  return with_group(c->HG, [&](auto hg) -> hipError_t {
    constexpr int HG = decltype(hg)::value;
    auto launch = [&](auto kern) -> hipError_t {
      if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(shm)))
        return e;
      return timed_launch(c, "attn_whole", kern, grid, dim3(nw * kWave), shm,
                          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_new),
                          static_cast<const uint16_t*>(v_new), static_cast<uint16_t*>(c->d.kpool),
                          static_cast<uint16_t*>(c->d.vpool), static_cast<const int*>(c->d.count),
                          static_cast<const int*>(c->d.hole), out, gm, static_cast<int>(cf.n_layers), c->G,
                          static_cast<int>(cf.n_kv_heads), static_cast<int>(cf.n_q_heads), c->P, c->maxpages,
                          c->lstride, nstride, 1.0f / sqrtf(128.0f), n_max, static_cast<const int*>(c->d.ptab));
    };
    if (paged) return launch(attn_seq_kernel<kSeqBlkNW, HG, true, true>);
    if (rounds)
      return obs ? launch(attn_seq_kernel<kSeqRoundsNW, HG, true, false>)
                 : launch(attn_seq_kernel<kSeqRoundsNW, HG, false, false>);
    return obs ? launch(attn_seq_kernel<kSeqNW, HG, true, false>) : launch(attn_seq_kernel<kSeqNW, HG, false, false>);
  });
}

hipError_t launch_attention_seq(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                                float* out, int n_max, int obs) {
  return launch_seq(c, q, k_new, v_new, out, n_max, obs != 0, false);
}

hipError_t launch_attention_seq_blocks(kvev_ctx* c, const void* q, const void* k_new, const void* v_new,
                                       float* out, int n_max) {
  return launch_seq(c, q, k_new, v_new, out, n_max, true, true);
}

}  // namespace kvev
