// Two-tier window mode: per-layer routing of windows of W = 32 or 8 tokens
// between a full-precision tier, a recoverable INT2 tier and permanent
// eviction.
//
// Source: the technical review of "QEvict: Recoverable Quantized KV Eviction
// for Attention-Drift-Robust Long-Context Decoding", section 4: the
// accessible keys and values are the full-precision windows plus the
// reconstructions of the INT2 windows (section 4.1, (Attention)); each
// window's score accumulates its attention mass averaged over the layer's
// query heads, over the steps of a routing interval (section 4.2, Eq.1); at
// each routing event the candidates are ranked, the best K_f stay in full
// precision, the next K_q go to the INT2 tier and the rest are evicted for
// good (section 4.4, Eq.4-6); a window is quantized once, at its first
// demotion, keys per channel and values per token, and its codes are reused
// by every later demotion and promotion (section 4.4, Algorithm 1).  In the
// rotary mode keys are quantized before the rotary embedding and rotated
// again at their original positions when reconstructed (section 4.4,
// positional handling for promoted keys).
//
// Storage, per (layer l, KV head h), in two slot pools sized from the byte
// budget (section 4.1 (Budget), section 4.3 Eq.3): a window holds only the
// slots its tier needs, and the per-layer slot maps fslot / lslot name them.
//   kfp    [L][Hkv][SF][W][128] bf16  full-precision keys, token-major
//          (rotated in the rotary mode)
//   vfp    [L][Hkv][SF][128][W] bf16  values, channel-major (a channel's W
//          tokens are contiguous: the p.V operand of the matrix cores)
//   kpre   [L][Hkv][SF][W][128] bf16  rotary mode only: the keys as given,
//          read by a window's first quantization
//   ledger [L][Hkv][SQ][record]  INT2 records; for W = 32 (3,072 B):
//     [0, 1024)     key codes, 16 B per lane of a wave (see below)
//     [1024, 2048)  value codes, 16 B per lane
//     [2048, 2304)  key scale per channel, fp16 [128] (with key groups:
//                   per (32-channel group, token), [4][W])
//     [2304, 2560)  key zero point, laid out as the scales
//     [2560, 2816)  value scale per (32-channel group, token), fp16 [4][32]
//     [2816, 3072)  value zero point, fp16 [4][32]
//   and for W = 8 (1,152 B) the kRec8* offsets below.
// SF covers the pinned windows, the windows not yet routed and K_f routed
// ones (and the K_q INT2 windows where they are read through bf16
// reconstructions: 8-token windows, the rotary mode or key groups); SQ =
// K_f + K_q.  A window releases its full-precision slot when it leaves full
// precision and its record when it is evicted; a promotion takes a new slot
// and writes the reconstruction into it.  The prefill windows wait in
// staging buffers of the same layout (slot SF + w) until the first routing
// event places them.
//
// Code records (32-token windows).  The attention multiplies the 2-bit
// codes as int8 B operands of v_mfma_i32_16x16x64_i8; a 32-bit word holds
// the 16 codes of one lane's operand, element k at bits 8 (k % 4) + 2 (k / 4),
// so that (w >> 2d) & 0x03030303 is the operand's word d.
//   keys:   lane (r16, q4) = lane r16 + 16 q4 owns four words (n-tile j,
//           k-step ks) at word 4 lane + 2 j + ks: token 16 j + r16, channels
//           64 ks + 16 q4 .. +16
//   values: word (hf 16 + r16) 8 + ct holds channel 16 ct + r16, tokens
//           16 hf .. +16 (hf = 0, 1)
#include "kvev_internal.h"

namespace kvev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int D = kTierD;  // head dim
constexpr int HG = 4;      // query heads per KV head
constexpr int W = kTierWin;  // the fused INT2 path's window (32 tokens)
constexpr int kRecK = 0, kRecV = 1024, kRecSK = 2048, kRecZK = 2304, kRecSV = 2560, kRecZV = 2816;
constexpr int kQW = 4;  // INT2 windows per wave of the fused INT2 path
// 8-token record: key codes [8][128] and value codes [8][128] at 2 bits
// (element e at byte e / 4, bits 2 (e % 4)), key scale and zero [128], value
// scale and zero [4][8] (fp16)
constexpr int kRec8K = 0, kRec8V = 256, kRec8SK = 512, kRec8ZK = 768, kRec8SV = 1024, kRec8ZV = 1088;

// A store written through the L2 to memory (relaxed agent-scope atomic
// store: global_store ... sc1).  The attention's chunk partials and window
// masses use it: the merge and mass kernels read them next, and the launch
// measured about 2.7 us shorter than with plain stores on the 131k
// workload.
__device__ __forceinline__ void st_through(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bf16x8_t as_b8(const uint4& r) {
  bf16x8_t v;
  __builtin_memcpy(&v, &r, sizeof(v));
  return v;
}

__device__ __forceinline__ float h2f(uint32_t bits) {
  const uint16_t b = static_cast<uint16_t>(bits);
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return static_cast<float>(h);
}

__device__ __forceinline__ uint16_t f2h(float f) {
  const _Float16 h = static_cast<_Float16>(f);  // round to nearest even
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// 16 two-bit codes of a spread word as the 16 int8 elements of a matrix-core
// operand: byte j of word d is the code at bits 8j + 2d (element 4d + j).
__device__ __forceinline__ uint4 spread_codes(uint32_t w) {
  constexpr uint32_t m = 0x03030303u;
  return make_uint4(w & m, (w >> 2) & m, (w >> 4) & m, (w >> 6) & m);
}

// Bit position of element k (0..15) in a spread word.
__host__ __device__ constexpr int spread_bit(int k) { return 8 * (k & 3) + 2 * (k >> 2); }

// Fixed-point digits as int8 operand bytes.  A value t = v * 2^F with
// |t| < 2^21 is rounded to the integer x = rint(t) by one fused multiply-add,
// f = v * 2^F + 1.5 * 2^23, whose bits are 0x4B000000 + 2^22 + x: bytes 0
// and 1 of f are those of x and byte 2 is 64 + (x >> 16).  The operand takes
// bytes 0 and 1 offset by 128 (u ^ 0x80 is u - 128 as int8) and byte 2 as
// it is, so x = 65536 (b2 - 64) + 256 (b1' + 128) + (b0' + 128).
__device__ __forceinline__ void digits4(const uint32_t* x, uint32_t& d0, uint32_t& d1, uint32_t& d2) {
  const uint32_t t01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);  // x0.b0 x1.b0 x0.b1 x1.b1
  const uint32_t t23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  d0 = __builtin_amdgcn_perm(t23, t01, 0x05040100u) ^ 0x80808080u;
  d1 = __builtin_amdgcn_perm(t23, t01, 0x07060302u) ^ 0x80808080u;
  const uint32_t u01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);  // x0.b2 x1.b2 x0.b3 x1.b3
  const uint32_t u23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  d2 = __builtin_amdgcn_perm(u23, u01, 0x05040100u);
}

// The product of a digit A operand (rows 4 hd + 0..2 the digits of head hd,
// row 4 hd + 3 all ones) with codes, summed back into sum_k x_k code_k: the
// lane's four accumulator rows are (d0, d1, d2, sum of codes), and
// sum x code = R0 + 256 R1 + 65536 R2 + (128 + 32768 - 64 * 65536) S.
// Exact (modulo 2^32 on the way) while the true sum fits in int32.
__device__ __forceinline__ int digit_sum(const i32x4_t& r) {
  const uint32_t t = static_cast<uint32_t>(r[0]) + (static_cast<uint32_t>(r[1]) << 8) +
                     (static_cast<uint32_t>(r[2]) << 16) - 4161408u * static_cast<uint32_t>(r[3]);
  return static_cast<int>(t);
}

__device__ __forceinline__ i32x4_t mfma_i8(const uint4& a, const uint4& b, const i32x4_t& c) {
  const i32x4_t av = {static_cast<int>(a.x), static_cast<int>(a.y), static_cast<int>(a.z), static_cast<int>(a.w)};
  const i32x4_t bv = {static_cast<int>(b.x), static_cast<int>(b.y), static_cast<int>(b.z), static_cast<int>(b.w)};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
}

// Exponent F that puts the largest magnitude m of a set under 2^21:
// |v| * 2^F < 2^21 for every |v| <= m (0 when m is 0; at most 127).
__device__ __forceinline__ int fixed_exp(float m) {
  return m > 0.f ? min(21 - __builtin_amdgcn_frexp_expf(m), 127) : 0;
}

// The float bits of v * 2^F + 1.5 * 2^23 (rint(v * 2^F) in the low bits) for
// eight values; p2 = 2^F.
__device__ __forceinline__ void to_fixed(const float* v, float p2, uint32_t* x) {
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = __float_as_uint(fmaf(v[e], p2, 12582912.0f));
}

// DPP within the 16 lanes of a row: rotate by 4 / 8, or take lane 4k + g of
// each quad.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_row_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// A 16-byte load that streams past the caches (each byte is read once).
__device__ __forceinline__ uint4 ld_nt(const void* p) {
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v r = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
}

__device__ __forceinline__ uint32_t word_of(const uint4& r, int i) {
  return i == 0 ? r.x : (i == 1 ? r.y : (i == 2 ? r.z : r.w));
}

// Two fp32 values rounded to nearest-even bf16, packed (low half first).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

// A operand of 8 fp32 values split into bf16 high parts (rows 0..3) and
// low parts (rows 4..7); rows 8..15 are zero.  high + low carries 16
// significant bits of each value.
__device__ __forceinline__ bf16x8_t split_rows(const float* x, int r16) {
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t hi = pack_bf16(x[2 * p], x[2 * p + 1]);
    const uint32_t lo = pack_bf16(x[2 * p] - __uint_as_float(hi << 16),
                                  x[2 * p + 1] - __uint_as_float(hi & 0xffff0000u));
    w[p] = r16 < 4 ? hi : (r16 < 8 ? lo : 0u);
  }
  return as_b8(make_uint4(w[0], w[1], w[2], w[3]));
}

// Orders a wave's LDS stores and loads that exchange data between its lanes
// (the LDS executes a wave's operations in order; this keeps the compiler
// from moving them across each other).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Rotary embedding of channel c of a key or query: x its value, y the value
// of its partner channel c ^ 64, rc the (cos, sin) row of its position.  The
// products and the sum are separately rounded fp64 operations (no fused
// multiply-add), the result rounded to fp32.
__device__ __forceinline__ float rope_elem(float x, float y, int c, const double* __restrict__ rc) {
  const double cs = rc[2 * (c & 63)], sn = rc[2 * (c & 63) + 1];
  const double a = __dmul_rn(static_cast<double>(x), cs), b = __dmul_rn(static_cast<double>(y), sn);
  return static_cast<float>(c < 64 ? __dsub_rn(a, b) : __dadd_rn(a, b));
}

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float((b & 0xffffu) << 16); }

// Full-precision storage of slot s of (layer, KV head) lh: the pool below
// SF, the prefill staging (window s - SF) above.
__device__ __forceinline__ uint16_t* kfp_at(const TierArgs& A, int64_t lh, int s, int Wn) {
  return s < A.SF ? A.kfp + (lh * A.SF + s) * Wn * kTierD : A.kst + (lh * A.NWS + (s - A.SF)) * Wn * kTierD;
}
__device__ __forceinline__ uint16_t* vfp_at(const TierArgs& A, int64_t lh, int s, int Wn) {
  return s < A.SF ? A.vfp + (lh * A.SF + s) * Wn * kTierD : A.vst + (lh * A.NWS + (s - A.SF)) * Wn * kTierD;
}
__device__ __forceinline__ uint16_t* kpre_at(const TierArgs& A, int64_t lh, int s, int Wn) {
  return s < A.SF ? A.kpre + (lh * A.SF + s) * Wn * kTierD : A.kpst + (lh * A.NWS + (s - A.SF)) * Wn * kTierD;
}
__device__ __forceinline__ uint8_t* rec_at(const TierArgs& A, int64_t lh, int s, int bytes) {
  return A.ledger + (lh * A.SQ + s) * static_cast<int64_t>(bytes);
}
// list entry: slot << kTierWinBits | window
__device__ __forceinline__ int ent_win(int e) { return e & ((1 << kTierWinBits) - 1); }
__device__ __forceinline__ int ent_slot(int e) { return e >> kTierWinBits; }
__device__ __forceinline__ int make_ent(int slot, int w) { return (slot << kTierWinBits) | w; }

__device__ __forceinline__ f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace

// ---------------------------------------------------------------------------
// Prefill: windows [0, nwin) of every (layer, KV head) from k, v
// [L][Hkv][n][128] into the staging buffers; tokens past n are zero.  Block
// (w, h, l), 256 threads.  Also resets the window state of layer l (h == 0):
// window w holds staging slot SF + w.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tier_prefill_kernel(TierArgs A, const uint16_t* __restrict__ k,
                                                           const uint16_t* __restrict__ v, int n) {
  __shared__ uint16_t vt[W][D + 2];
  const int w = blockIdx.x, h = blockIdx.y, l = blockIdx.z, tid = threadIdx.x;
  const int Wn = A.W;  // tokens per window (8 or 32)
  const int64_t lh = static_cast<int64_t>(l) * A.Hkv + h;
  const int64_t src0 = lh * n;
  uint16_t* kd = kfp_at(A, lh, A.SF + w, Wn);
  uint16_t* vd = vfp_at(A, lh, A.SF + w, Wn);
  for (int i = tid; i < Wn * D; i += 256) {
    const int r = i / D, c = i % D;
    const int p = w * Wn + r;
    const bool in = p < n;
    const uint16_t kv = in ? k[(src0 + p) * D + c] : 0;
    if (A.rope) {  // rotary mode: keep the key as given, store it rotated at its position
      kpre_at(A, lh, A.SF + w, Wn)[i] = kv;
      const uint16_t kp = in ? k[(src0 + p) * D + (c ^ 64)] : 0;
      kd[i] = in ? static_cast<uint16_t>(bf16_rne(rope_elem(bf2f(kv), bf2f(kp), c, A.rcs + static_cast<int64_t>(p) * 128)))
                 : 0;
    } else {
      kd[i] = kv;
    }
    vt[r][c] = in ? v[(src0 + p) * D + c] : 0;
  }
  __syncthreads();
  for (int i = tid; i < Wn * D; i += 256) {
    const int c = i / Wn, r = i % Wn;
    vd[i] = vt[r][c];
  }
  if (h == 0 && tid == 0) {
    const int64_t lw = static_cast<int64_t>(l) * A.NW + w;
    A.fplist[lw] = make_ent(A.SF + w, w);
    A.fslot[lw] = A.SF + w;
    A.lslot[lw] = -1;
    A.tier[lw] = 0;
    A.hasled[lw] = 0;
    A.S[lw] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Rotary mode: (cos, sin) of position * frequency_i for positions
// [p0, p0 + n) and i < 64, in fp64.  One thread per (position, i).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tier_rope_table_kernel(TierArgs A, int64_t p0, int64_t n) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= n * 64) return;
  const int64_t p = p0 + idx / 64;
  const int i = static_cast<int>(idx % 64);
  double sn, cs;
  sincos(__dmul_rn(static_cast<double>(p), A.ifreq[i]), &sn, &cs);
  A.rcs[(p * 64 + i) * 2] = cs;
  A.rcs[(p * 64 + i) * 2 + 1] = sn;
}

// ---------------------------------------------------------------------------
// Append: the new token (position npos) into its window's storage.  When it
// opens a window, that window takes free slot kslot of its layer (the
// kslot-th window opened since the last routing event), starts full
// precision with score 0 and joins the full-precision list at index n_fp.
// Block (h, l), 128 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void tier_append_kernel(TierArgs A, const uint16_t* __restrict__ k_new,
                                                          const uint16_t* __restrict__ v_new, int npos,
                                                          int n_fp, int kslot) {
  const int h = blockIdx.x, l = blockIdx.y, c = threadIdx.x;
  const int Wn = A.W;
  const int64_t lh = static_cast<int64_t>(l) * A.Hkv + h;
  const int w = npos / Wn, r = npos % Wn;
  const int64_t lw = static_cast<int64_t>(l) * A.NW + w;
  const int slot = max(r == 0 ? A.ffree[static_cast<int64_t>(l) * A.SF + kslot] : A.fslot[lw], 0);
  const int64_t ki = static_cast<int64_t>(r) * D + c;
  if (A.rope) {
    kpre_at(A, lh, slot, Wn)[ki] = k_new[lh * D + c];
    kfp_at(A, lh, slot, Wn)[ki] = static_cast<uint16_t>(bf16_rne(
        rope_elem(bf2f(k_new[lh * D + c]), bf2f(k_new[lh * D + (c ^ 64)]), c, A.rcs + static_cast<int64_t>(npos) * 128)));
  } else {
    kfp_at(A, lh, slot, Wn)[ki] = k_new[lh * D + c];
  }
  vfp_at(A, lh, slot, Wn)[c * Wn + r] = v_new[lh * D + c];
  if (r == 0 && h == 0 && c == 0) {
    A.fplist[static_cast<int64_t>(l) * A.NW + n_fp] = make_ent(slot, w);
    A.fslot[lw] = slot;
    A.lslot[lw] = -1;
    A.tier[lw] = 0;
    A.hasled[lw] = 0;
    A.S[lw] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Attention over the accessible windows of (layer l, KV head h).  Block
// (chunk, h, l) of 4 waves; a wave takes 64 tokens of the full-precision
// list (2 windows of 32 or 8 of 8) or kQW = 4 windows of the INT2 list (the
// INT2 path: 16 windows a chunk).  Chunks [0, nch_f) cover the
// full-precision list, the rest the INT2 list; each list entry names the
// window and the slot its storage is read from.  Writes the chunk's (max,
// sum) and unnormalised output per head, and per window and head the sum of
// exp(s - chunk max) over the window's tokens (its attention mass before
// normalisation).
//   Full precision, bf16 matrix cores: q.K with A = the 4 query rows, B = K^T
//     (n-tiles of 16 tokens, k-steps of 32 channels); p.V with A = P (bf16
//     high / low rows), B = V (a k-step is 32 tokens).
//   INT2, int8 matrix cores: logit = sum_c (q_c s_c) code_c + sum_c q_c z_c
//     and out_c = sum_t (p_t s_tg) code_tc + sum_t p_t z_tg (g = c / 32),
//     the scaled operands as fixed-point digit rows, the codes as B.
// ---------------------------------------------------------------------------
// Three waves per SIMD: the register cap this sets (168) costs no spills.
// WT: tokens per window (32 or 8).  MAT: INT2 windows are read from their
// bf16 reconstruction in the full-precision pool (8-token windows, rotary
// mode, key groups), so every window takes the full-precision path; in
// rotary mode the queries are rotated at the new token's position npos - 1.
template <int WT, bool MAT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void tier_attn_kernel(
    TierArgs A, const uint16_t* __restrict__ q, int n_fp, int n_q, int nch_f, int npos, float scale) {
  constexpr int FW = 64 / WT;                    // full-precision-path windows per wave
  constexpr int NWIN = FW > kQW ? FW : kQW;
  static_assert(WT == 32 || (WT == 8 && MAT), "8-token windows are read through the full-precision path");
  __shared__ __align__(16) float p_lds[4][HG][32 * kQW];
  __shared__ __align__(16) float o_lds[4][HG][D];
  __shared__ float wstat[4][HG][2];
  __shared__ float e_lds[4][NWIN][HG];
  __shared__ uint4 opk[4][2 * 16 * 4];  // INT2 q.K digit operands, per wave
  __shared__ uint4 opv[4][4 * 16 * 4];  // INT2 p.V digit operands, per wave

  const int chunk = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r16 = lane & 15, q4 = lane >> 4;
  const bool isq = chunk >= nch_f;
  const bool fused = isq && !MAT;  // the fused INT2 path
  const int wpw = fused ? kQW : FW;  // windows per wave
  const int base = isq ? (chunk - nch_f) * 4 * wpw : chunk * 4 * FW;
  const int nlist = isq ? n_q : n_fp;
  const int64_t lh = static_cast<int64_t>(l) * A.Hkv + h;
  const int* list = (isq ? A.qlist : A.fplist) + static_cast<int64_t>(l) * A.NW;
  int win[NWIN], slot[NWIN];  // window and its storage slot (full precision, or its record)
  bool live[NWIN];
#pragma unroll
  for (int k = 0; k < NWIN; ++k) {
    const int idx = base + wpw * wave + k;
    live[k] = k < wpw && idx < nlist;
    const int e = live[k] ? list[idx] : 0;
    win[k] = ent_win(e);
    slot[k] = ent_slot(e);
  }

  // the lane's query row (head r16 & 3) on channels 32s + 8q4 .. +8
  uint4 qraw[4];
  {
    const uint16_t* qp = q + (static_cast<int64_t>(l) * A.Hq + h * HG + (r16 & 3)) * D + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) qraw[s] = *reinterpret_cast<const uint4*>(qp + 32 * s);
  }
  if constexpr (MAT) {
    if (A.rope) {  // channel 32s + 8q4 + e (s < 2) pairs with the same element of k-step s + 2
      const double* rc = A.rcs + static_cast<int64_t>(npos - 1) * 128;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t a = word_of(qraw[s], u), b = word_of(qraw[s + 2], u);
          uint32_t ra = 0, rb = 0;
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int c = 32 * s + 8 * q4 + 2 * u + half;
            const float x = bf2f(a >> (16 * half)), y = bf2f(b >> (16 * half));
            ra |= bf16_rne(rope_elem(x, y, c, rc)) << (16 * half);
            rb |= bf16_rne(rope_elem(y, x, c + 64, rc)) << (16 * half);
          }
          lo[u] = ra;
          hi[u] = rb;
        }
        qraw[s] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        qraw[s + 2] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      }
    }
  }

  if (!fused) {
    float sv[4][HG];  // logits of n-tile jj (lanes q4 == 0 hold them)
    f32x4_t oacc[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) oacc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // ---- windows read from full-precision storage ---------------------------
    // A wave reads 64 tokens: 2 windows of 32, or 8 of 8.  K tile jj is
    // tokens 16jj .. 16jj+15 of the wave (token r16 of the tile in window
    // slot (16jj + r16) / WT); p.V k-step k is tokens 32k .. 32k+31 (the
    // lane's 8 tokens 8q4 .. +8 in slot (32k + 8q4) / WT).
    bf16x8_t qa[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = as_b8(r16 < HG ? qraw[s] : make_uint4(0, 0, 0, 0));
    // Loads are unconditional: a window past the list reads window 0 of the
    // layer, and its logits are masked (-inf), so its values meet p = 0.
    uint4 kr[4][4], vr[2][8];
    int kpos[4];
    bool klive[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      int wk, sk, rk;
      if constexpr (WT == 32) {
        wk = win[jj >> 1];
        sk = slot[jj >> 1];
        klive[jj] = live[jj >> 1];
        rk = 16 * (jj & 1) + r16;
      } else {
        const bool up = r16 >= 8;
        wk = up ? win[2 * jj + 1] : win[2 * jj];
        sk = up ? slot[2 * jj + 1] : slot[2 * jj];
        klive[jj] = up ? live[2 * jj + 1] : live[2 * jj];
        rk = r16 & 7;
      }
      kpos[jj] = wk * WT + rk;
      const uint16_t* kb = kfp_at(A, lh, sk, WT) + rk * D + 8 * q4;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kr[jj][s] = *reinterpret_cast<const uint4*>(kb + 32 * s);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      int sv, r0;
      if constexpr (WT == 32) {
        sv = slot[k];
        r0 = 8 * q4;
      } else {
        const int a = 4 * k;
        sv = q4 == 0 ? slot[a] : (q4 == 1 ? slot[a + 1] : (q4 == 2 ? slot[a + 2] : slot[a + 3]));
        r0 = 0;
      }
      const uint16_t* vb = vfp_at(A, lh, sv, WT) + r16 * WT + r0;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        vr[k][ct] = *reinterpret_cast<const uint4*>(vb + 16 * ct * WT);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma(qa[s], as_b8(kr[jj][s]), acc);
      const bool valid = q4 == 0 && klive[jj] && kpos[jj] < npos;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) sv[jj][hh] = valid ? acc[hh] * scale : -INFINITY;
    }
    // softmax statistics of the wave, per-window masses, probabilities to LDS
    float mh[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      float m = fmaxf(fmaxf(sv[0][hh], sv[1][hh]), fmaxf(sv[2][hh], sv[3][hh]));
      mh[hh] = row16_max(m);
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      float tile[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float pv = mh[hh] == -INFINITY ? 0.f : __expf(sv[jj][hh] - mh[hh]);
        sv[jj][hh] = pv;
        tile[jj] = pv;
      }
      float tot = 0.f;
      if constexpr (WT == 32) {
        const float e0 = row16_sum(tile[0] + tile[1]), e1 = row16_sum(tile[2] + tile[3]);
        if (lane == 0) {
          e_lds[wave][0][hh] = e0;
          e_lds[wave][1][hh] = e1;
        }
        tot = e0 + e1;
      } else {
        // a tile holds two windows: lanes 0..7 and 8..15 of the row
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float e = tile[jj];
          e += __shfl_xor(e, 1, kWave);
          e += __shfl_xor(e, 2, kWave);
          e += __shfl_xor(e, 4, kWave);
          if (lane == 0) e_lds[wave][2 * jj][hh] = e;
          if (lane == 8) e_lds[wave][2 * jj + 1][hh] = e;
          tot += e + __shfl_xor(e, 8, kWave);
        }
      }
      if (lane == 0) {
        wstat[wave][hh][0] = mh[hh];
        wstat[wave][hh][1] = tot;
      }
    }
    if (q4 == 0) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) p_lds[wave][hh][16 * jj + r16] = sv[jj][hh];
    }
    __syncthreads();
    // p.V: one k-step per window, P in high / low rows
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&p_lds[wave][r16 & 3][32 * k + 8 * q4]);
      const float4 b = *reinterpret_cast<const float4*>(&p_lds[wave][r16 & 3][32 * k + 8 * q4 + 4]);
      const float pv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      const bf16x8_t pa = split_rows(pv, r16);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) oacc[ct] = mfma(pa, as_b8(vr[k][ct]), oacc[ct]);
    }
    // the wave's output: high rows (q4 == 0) + low rows (q4 == 1)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float o = oacc[ct][hh] + __shfl_xor(oacc[ct][hh], 16, kWave);
        if (q4 == 0) o_lds[wave][hh][16 * ct + r16] = o;
      }
    }
  } else if constexpr (!MAT) {
    // ---- INT2 windows: int8 matrix-core products -----------------------------
    // Each product runs on the codes as int8 B operands and on fixed-point
    // digits of the scaled operands as the A operand: rows 4 hd + 0..2 hold
    // the three digits of head hd, row 4 hd + 3 is all ones (the sum of the
    // codes, which undoes the digits' offset).  The scaled operands are
    // formed once per (head, channel) and (head, token, group) and staged in
    // LDS by the lanes that form them:
    //   q.K: lane (head hs = lane / 16, channels 8 cs .. +8, cs = lane % 16);
    //        exponent per (head, window) from the largest |q_c s_c|
    //   p.V: lane (head hs, tokens 8 ts .. +8, ts = lane / 4 % 4, 32-channel
    //        group gs = lane % 4), two windows (64 tokens) per k range;
    //        exponent per (head, group, window pair) from the largest p_t s_tg
    // A lane (r16, q4) of a product's result holds head q4 (= hs of the lane
    // that formed its operand): token or channel r16, accumulator rows
    // (d0, d1, d2, sum of codes).
    const int hs = lane >> 4, cs = lane & 15, ts = (lane >> 2) & 3, gs = lane & 3;
    uint4* ka = opk[wave];  // [k-step 2][row 16][k-group 4]
    uint4* va = opv[wave];  // [group 4][row 16][k-group 4]
    // Every record load is issued up front and unconditionally (a window
    // past the list reads window 0 of the layer, whose results are masked:
    // its logits are -inf, so its probabilities and p.V digits are 0).
    const uint8_t* recs[kQW];
#pragma unroll
    for (int k = 0; k < kQW; ++k) recs[k] = rec_at(A, lh, slot[k], kTierLedgerBytes);
    uint4 kc[kQW], ksr[kQW], kzr[kQW];
#pragma unroll
    for (int k = 0; k < kQW; ++k) {
      kc[k] = ld_nt(recs[k] + kRecK + 16 * lane);
      ksr[k] = *reinterpret_cast<const uint4*>(recs[k] + kRecSK + 16 * cs);
      kzr[k] = *reinterpret_cast<const uint4*>(recs[k] + kRecZK + 16 * cs);
    }
    float qx[8];
    Vec16<bf16_t>::widen(
        *reinterpret_cast<const uint4*>(q + (static_cast<int64_t>(l) * A.Hq + h * HG + hs) * D + 8 * cs), qx);
    // the ones rows: 32 entries of ka, 64 of va
    {
      const uint4 ones = make_uint4(0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u);
      const int ent = (4 * ((lane >> 2) & 3) + 3) * 4 + (lane & 3);
      if (lane < 32) ka[(lane >> 4) * 64 + ent] = ones;
      va[(lane >> 4) * 64 + ent] = ones;
    }
    float lgt[2 * kQW];  // logits of head q4, token r16 of n-tile jj
    // where the lane's 8 digit bytes of a k-step go: k-step cs / 8, k-group
    // (cs % 8) / 2, half cs % 2 of the 16-byte row entry
    uint2* kdst = reinterpret_cast<uint2*>(ka) + (((cs >> 3) * 16 + 4 * hs) * 4 + ((cs & 7) >> 1)) * 2 + (cs & 1);
#pragma unroll
    for (int k = 0; k < kQW; ++k) {
      float a[8];
      float bias = 0.f, amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float sc = h2f(word_of(ksr[k], e >> 1) >> (16 * (e & 1)));
        const float zp = h2f(word_of(kzr[k], e >> 1) >> (16 * (e & 1)));
        a[e] = qx[e] * sc;
        bias = fmaf(qx[e], zp, bias);
        amax = fmaxf(amax, fabsf(a[e]));
      }
      // per head: the exponent and sum_c q_c z_c (the 16 lanes of head hs)
      const int F = fixed_exp(row16_max(amax));
      bias = row16_sum(bias);
      uint32_t x[8];
      to_fixed(a, __builtin_amdgcn_ldexpf(1.0f, F), x);
      uint32_t dg[3][2];
      digits4(x, dg[0][0], dg[1][0], dg[2][0]);
      digits4(x + 4, dg[0][1], dg[1][1], dg[2][1]);
      wave_lds_order();
#pragma unroll
      for (int d = 0; d < 3; ++d) kdst[d * 4 * 2] = make_uint2(dg[d][0], dg[d][1]);
      wave_lds_order();
      const uint4 a0 = ka[(0 * 16 + r16) * 4 + q4], a1 = ka[(1 * 16 + r16) * 4 + q4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        i32x4_t acc = {0, 0, 0, 0};
        acc = mfma_i8(a0, spread_codes(word_of(kc[k], 2 * j)), acc);
        acc = mfma_i8(a1, spread_codes(word_of(kc[k], 2 * j + 1)), acc);
        const float lg = __builtin_amdgcn_ldexpf(static_cast<float>(digit_sum(acc)), -F) + bias;
        lgt[2 * k + j] = live[k] ? lg * scale : -INFINITY;
      }
    }
    // p.V records: scale and zero point of (group gs, tokens 8 ts .. +8),
    // stored [group][token], and the codes of the lane's B operands: window
    // 2 pr + q4 / 2, tokens 16 (q4 % 2) .. +16, channel 16 ct + r16
    uint4 vsr[kQW], vzr[kQW], vc[kQW / 2][2];
#pragma unroll
    for (int k = 0; k < kQW; ++k) {
      vsr[k] = *reinterpret_cast<const uint4*>(recs[k] + kRecSV + 2 * (32 * gs + 8 * ts));
      vzr[k] = *reinterpret_cast<const uint4*>(recs[k] + kRecZV + 2 * (32 * gs + 8 * ts));
    }
#pragma unroll
    for (int pr = 0; pr < kQW / 2; ++pr) {
      const uint8_t* rc = (q4 >> 1) ? recs[2 * pr + 1] : recs[2 * pr];
      const uint8_t* b = rc + kRecV + 32 * ((q4 & 1) * 16 + r16);
      vc[pr][0] = ld_nt(b);
      vc[pr][1] = ld_nt(b + 16);
    }
    // softmax statistics of head q4 over the wave's windows
    float m = lgt[0];
#pragma unroll
    for (int jj = 1; jj < 2 * kQW; ++jj) m = fmaxf(m, lgt[jj]);
    m = row16_max(m);
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < kQW; ++k) {
      const float p0 = m == -INFINITY ? 0.f : __expf(lgt[2 * k] - m);
      const float p1 = m == -INFINITY ? 0.f : __expf(lgt[2 * k + 1] - m);
      lgt[2 * k] = p0;
      lgt[2 * k + 1] = p1;
      const float e = row16_sum(p0 + p1);
      if (r16 == 0) e_lds[wave][k][q4] = e;
      tot += e;
    }
    if (r16 == 0) {
      wstat[wave][q4][0] = m;
      wstat[wave][q4][1] = tot;
    }
#pragma unroll
    for (int jj = 0; jj < 2 * kQW; ++jj) p_lds[wave][q4][16 * jj + r16] = lgt[jj];
    wave_lds_order();
    // p.V over window pairs
    float ov[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // head q4, channel 16 ct + r16
    float bzl = 0.f;  // sum_t p_t z_tg of (head hs, group gs) over the lane's tokens
#pragma unroll
    for (int pr = 0; pr < kQW / 2; ++pr) {
      float y[2][8];
      float ymax = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int k = 2 * pr + kk;
        const float4 pa4 = *reinterpret_cast<const float4*>(&p_lds[wave][hs][32 * k + 8 * ts]);
        const float4 pb4 = *reinterpret_cast<const float4*>(&p_lds[wave][hs][32 * k + 8 * ts + 4]);
        const float pv[8] = {pa4.x, pa4.y, pa4.z, pa4.w, pb4.x, pb4.y, pb4.z, pb4.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sc = h2f(word_of(vsr[k], e >> 1) >> (16 * (e & 1)));
          const float zp = h2f(word_of(vzr[k], e >> 1) >> (16 * (e & 1)));
          y[kk][e] = pv[e] * sc;
          bzl = fmaf(pv[e], zp, bzl);
          ymax = fmaxf(ymax, y[kk][e]);
        }
      }
      // exponent of (head hs, group gs): the lanes of its 4 token blocks
      // (lanes 4k + gs of the row)
      ymax = fmaxf(ymax, dpp_row<0x124>(ymax));
      ymax = fmaxf(ymax, dpp_row<0x128>(ymax));
      const int Fv = fixed_exp(ymax);
      const float p2 = __builtin_amdgcn_ldexpf(1.0f, Fv);
      uint32_t dg[2][3][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t x[8];
        to_fixed(y[kk], p2, x);
        digits4(x, dg[kk][0][0], dg[kk][1][0], dg[kk][2][0]);
        digits4(x + 4, dg[kk][0][1], dg[kk][1][1], dg[kk][2][1]);
      }
      // the exponent of (head q4, group g): lane g of any quad of row q4
      const int Fg[4] = {dpp_row_i<0x00>(Fv), dpp_row_i<0x55>(Fv), dpp_row_i<0xAA>(Fv), dpp_row_i<0xFF>(Fv)};
      wave_lds_order();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int d = 0; d < 3; ++d)
          reinterpret_cast<uint2*>(va)[((gs * 16 + 4 * hs + d) * 4 + 2 * kk + (ts >> 1)) * 2 + (ts & 1)] =
              make_uint2(dg[kk][d][0], dg[kk][d][1]);
      wave_lds_order();
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint4 ag = va[(g * 16 + r16) * 4 + q4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int ct = 2 * g + t;
          const i32x4_t acc = mfma_i8(ag, spread_codes(word_of(vc[pr][ct >> 2], ct & 3)), i32x4_t{0, 0, 0, 0});
          ov[ct] += __builtin_amdgcn_ldexpf(static_cast<float>(digit_sum(acc)), -Fg[g]);
        }
      }
    }
    // sum_t p_t z_tg of each (head, group): over the lanes' token blocks,
    // then lane g of a quad of row q4 holds group g
    bzl += dpp_row<0x124>(bzl);
    bzl += dpp_row<0x128>(bzl);
    const float bz[4] = {dpp_row<0x00>(bzl), dpp_row<0x55>(bzl), dpp_row<0xAA>(bzl), dpp_row<0xFF>(bzl)};
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) o_lds[wave][q4][16 * ct + r16] = ov[ct] + bz[ct >> 1];
  }
  __syncthreads();

  // merge the block's waves into one partial
  const int nch = gridDim.x;
  const int64_t pb = lh * A.maxch + chunk;
  for (int idx = tid; idx < HG * D; idx += 256) {
    const int hh = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wstat[w][hh][0]);
    float o = 0.f, Z = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = wstat[w][hh][0] == -INFINITY ? 0.f : __expf(wstat[w][hh][0] - M);
      o += f * o_lds[w][hh][c];
      Z += f * wstat[w][hh][1];
    }
    st_through(&A.part_o[pb * HG * D + idx], o);
    if (c == 0) {
      st_through(&A.part_ml[(pb * HG + hh) * 2 + 0], M);
      st_through(&A.part_ml[(pb * HG + hh) * 2 + 1], Z);
    }
  }
  if (tid < 4 * wpw * HG) {
    const int slot = tid / HG, hh = tid % HG;  // slot = wpw * wave + k
    const int wv = slot / wpw, k = slot % wpw;
    const int idx = base + slot;
    if (idx < nlist) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, wstat[w][hh][0]);
      const float f = wstat[wv][hh][0] == -INFINITY ? 0.f : __expf(wstat[wv][hh][0] - M);
      const int cidx = (isq ? n_fp : 0) + idx;
      st_through(&A.emass[(lh * A.NW + cidx) * HG + hh], e_lds[wv][k][hh] * f);
    }
  }
  (void)nch;
}

// ---------------------------------------------------------------------------
// Merge the chunks of query head hh of (layer l, KV head h): its output and
// global (max, sum).  Block (hh, h, l), 256 threads, dynamic LDS of 2 * nch
// floats.  The chunks' (max, sum) are staged in LDS; wave 0 reduces M and Z
// and turns each chunk's max m into its weight e^(m - M).  Output channel c
// is summed by threads c (even chunks) and c + 128 (odd chunks),
// kMergeLoads independent loads at a time, and the halves are added in LDS.
// ---------------------------------------------------------------------------
constexpr int kMergeLoads = 32;

__global__ __launch_bounds__(256) void tier_merge_kernel(TierArgs A, float* __restrict__ out, int nch) {
  extern __shared__ float mlds[];
  float* sm = mlds;        // [nch]: chunk max, then its weight
  float* sz = mlds + nch;  // [nch]: chunk sum
  __shared__ float s_Z, half[D];
  const int hh = blockIdx.x, h = blockIdx.y, l = blockIdx.z, tid = threadIdx.x, lane = tid % kWave;
  const int64_t lh = static_cast<int64_t>(l) * A.Hkv + h;
  const float* pml = A.part_ml + lh * A.maxch * HG * 2;
  for (int c = tid; c < nch; c += 256) {
    sm[c] = pml[(c * HG + hh) * 2];
    sz[c] = pml[(c * HG + hh) * 2 + 1];
  }
  __syncthreads();
  if (tid < kWave) {
    float M = -INFINITY;
    for (int c = lane; c < nch; c += kWave) M = fmaxf(M, sm[c]);
    M = wave_max(M);
    float Z = 0.f;
    for (int c = lane; c < nch; c += kWave) {
      const float m = sm[c];
      const float f = m == -INFINITY ? 0.f : __expf(m - M);
      sm[c] = f;
      Z += f * sz[c];
    }
    Z = wave_sum(Z);
    if (lane == 0) {
      s_Z = Z;
      A.ml[(lh * HG + hh) * 2] = M;
      A.ml[(lh * HG + hh) * 2 + 1] = Z;
    }
  }
  __syncthreads();
  const int ch = tid % D, par = tid / D;  // channel, chunk parity
  const float* po = A.part_o + (lh * A.maxch * HG + hh) * D + ch;
  float o = 0.f;
  for (int c0 = par; c0 < nch; c0 += 2 * kMergeLoads) {
    float v[kMergeLoads];
#pragma unroll
    for (int k = 0; k < kMergeLoads; ++k) {
      const int c = c0 + 2 * k;
      v[k] = c < nch ? po[static_cast<int64_t>(c) * HG * D] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < kMergeLoads; ++k)
      if (c0 + 2 * k < nch) o = fmaf(sm[c0 + 2 * k], v[k], o);
  }
  if (par == 1) half[ch] = o;
  __syncthreads();
  if (par == 0) out[(static_cast<int64_t>(l) * A.Hq + h * HG + hh) * D + ch] = (o + half[ch]) / s_Z;
}

// ---------------------------------------------------------------------------
// Window mass of every accessible window of layer l, added to its score:
// (1/Hq) sum over KV heads and their query heads of the window's
// probability mass.  Block (x, l), 256 threads, one window per thread.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tier_mass_kernel(TierArgs A, int n_fp, int n_q, int nch_f, int cw_f,
                                                        int cw_q) {
  const int l = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= n_fp + n_q) return;
  const bool isq = idx >= n_fp;
  const int chunk = isq ? nch_f + (idx - n_fp) / cw_q : idx / cw_f;  // cw_*: windows per chunk
  const int w = ent_win(isq ? A.qlist[static_cast<int64_t>(l) * A.NW + idx - n_fp]
                            : A.fplist[static_cast<int64_t>(l) * A.NW + idx]);
  float acc = 0.f;
  // the KV heads in batches of 8, every load of a batch issued before use
  for (int h0 = 0; h0 < A.Hkv; h0 += 8) {
    float mb[8][HG], M[8][HG], Z[8][HG], em[8][HG];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int h = min(h0 + k, A.Hkv - 1);
      const int64_t lh = static_cast<int64_t>(l) * A.Hkv + h;
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        mb[k][hh] = A.part_ml[((lh * A.maxch + chunk) * HG + hh) * 2];
        M[k][hh] = A.ml[(lh * HG + hh) * 2];
        Z[k][hh] = A.ml[(lh * HG + hh) * 2 + 1];
        em[k][hh] = A.emass[(lh * A.NW + idx) * HG + hh];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        const float f = mb[k][hh] == -INFINITY ? 0.f : __expf(mb[k][hh] - M[k][hh]) / Z[k][hh];
        if (h0 + k < A.Hkv) acc += em[k][hh] * f;
      }
  }
  A.S[static_cast<int64_t>(l) * A.NW + w] += acc / static_cast<float>(A.Hq);
}

// ---------------------------------------------------------------------------
// Routing event of layer l0 + blockIdx.x (one block of 1024 threads per
// layer).  Candidates are the aged windows (w >= np, W(w+1) <= recent_lo)
// not yet evicted; each is ranked by (score, window) descending; rank < k_f
// stays / becomes full precision, rank < k_f + k_q INT2, the rest evicted.
// With `forced` the tiers of every window are taken from it instead (state
// import).  Then the storage follows the tiers:
//   * a window keeps its full-precision slot while it stays full precision
//     (with bf16 reconstructions: also while INT2); a prefill window moves
//     from the staging buffers into a slot of the pool (adopt job); a
//     promoted window takes a new slot (promote job); a demoted or evicted
//     window releases its slot;
//   * a first demotion takes a record slot (quantize job, which also writes
//     the bf16 reconstruction where INT2 windows are read through it); an
//     evicted window releases its record.
// New slots are given in window order: first the lowest slots free before
// the event, then the lowest ones it released.  The transitions run in two
// launches: phase 1 the quantize jobs (which read released slots) and the
// jobs into slots free before the event, phase 2 the jobs into released
// slots.  The lists are rebuilt in window order with each entry's slot.
// Errors (flag bits): the list sizes differ from the host's (exp_fp,
// exp_q): 32; an evicted window would be kept (its storage is gone): 64; a
// pool is exhausted: 128.
// ---------------------------------------------------------------------------
constexpr int kRouteNT = 1024;
constexpr int kSlotWords = kTierMaxWin / 32;  // bitmap words of a slot pool

// Stable rank of the calling thread's first item among the items of the
// block (thread tid owning a consecutive run of cnt items): an exclusive
// block-wide prefix sum.  `ws` holds kRouteNT / 64 ints of scratch; returns
// the total in `tot`.
__device__ __forceinline__ int block_excl_scan(int cnt, int* ws, int& tot) {
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  int x = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == kWave - 1) ws[wv] = x;
  __syncthreads();
  int off = x - cnt;
  tot = 0;
  for (int u = 0; u < kRouteNT / kWave; ++u) {
    if (u < wv) off += ws[u];
    tot += ws[u];
  }
  return off;
}

// The r-th set bit (0-based) of a bitmap of nw words whose exclusive prefix
// popcounts are pre[]; -1 when there are not that many.
__device__ __forceinline__ int nth_bit(const uint32_t* bits, const int* pre, int nw, int total, int r) {
  if (r >= total) return -1;
  int lo = 0, hi = nw - 1;  // the last word with pre <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  uint32_t b = bits[lo];
  for (int k = r - pre[lo]; k > 0; --k) b &= b - 1;
  return 32 * lo + __builtin_ctz(b);
}

__global__ __launch_bounds__(kRouteNT) void tier_route_kernel(TierArgs A, int nw, int np, int recent_lo,
                                                              int k_f, int k_q, int exp_fp, int exp_q,
                                                              const uint8_t* __restrict__ forced, int l0) {
  __shared__ unsigned long long keys[kTierMaxWin];  // the ranking; then the two slot arrays
  __shared__ uint8_t tl[kTierMaxWin];               // tier after the event
  __shared__ uint8_t hl[kTierMaxWin];               // record held after the event
  __shared__ uint8_t act[kTierMaxWin];              // bit 0 new full-precision slot, bit 1 new record, bits 2.. job
  __shared__ uint32_t freeF[kSlotWords], freeQ[kSlotWords], freshF[kSlotWords];
  __shared__ int preF[kSlotWords], preQ[kSlotWords], preN[kSlotWords];
  __shared__ int ncand, njobs, wsum[kRouteNT / kWave], tots[4];
  __shared__ int hist[2][256], rsel[2], nsel[2];  // the two threshold searches
  __shared__ unsigned long long psel[2];
  __shared__ int dsum[6][kRouteNT / kWave];
  const int l = l0 + blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int64_t lw0 = static_cast<int64_t>(l) * A.NW;
  if (tid == 0) {
    ncand = 0;
    njobs = 0;
  }
  for (int w = tid; w < nw; w += kRouteNT) {
    tl[w] = A.tier[lw0 + w];
    act[w] = tl[w];  // the tier before the event, until the storage pass
    hl[w] = A.hasled[lw0 + w];
  }
  __syncthreads();
  auto aged = [&](int w) { return w >= np && (w + 1) * A.W <= recent_lo; };
  if (!forced) {
    for (int w = tid; w < nw; w += kRouteNT) {
      if (aged(w) && tl[w] != 2) {
        const int i = atomicAdd(&ncand, 1);
        keys[i] = (static_cast<unsigned long long>(float_key(A.S[lw0 + w])) << 32) | static_cast<unsigned>(w);
      }
    }
    __syncthreads();
    const int nc = ncand;
    // F: the k_f largest keys, Q: the next k_q, E: the rest.  The keys are
    // distinct (window ids), so the two thresholds are the keys of rank
    // k_f - 1 and k_f + k_q - 1 (from the top), found together by 8-bit
    // radix passes from the top byte: each pass counts the keys that share
    // the prefix found so far by their next byte, and one wave per
    // threshold takes the byte whose bucket holds the rank.
    const int nsel0 = k_f, nsel1 = k_f + k_q;
    const bool act0 = nsel0 > 0 && nsel0 < nc, act1 = nsel1 > 0 && nsel1 < nc;
    if (tid == 0) {
      psel[0] = psel[1] = 0ull;
      rsel[0] = nsel0 - 1;
      rsel[1] = nsel1 - 1;
      nsel[0] = act0 ? nc : 1;  // keys sharing the prefix found so far
      nsel[1] = act1 ? nc : 1;
    }
    int pass = 0;
    for (; pass < 8; ++pass) {
      const int sh = 56 - 8 * pass;
      for (int i = tid; i < 512; i += kRouteNT) (&hist[0][0])[i] = 0;
      __syncthreads();
      const unsigned long long hm = pass == 0 ? 0ull : (~0ull << (sh + 8));
      const unsigned long long p0 = psel[0] & hm, p1 = psel[1] & hm;
      for (int i = tid; i < nc; i += kRouteNT) {
        const unsigned long long key = keys[i];
        const int b = static_cast<int>((key >> sh) & 255u);
        if (act0 && (key & hm) == p0) atomicAdd(&hist[0][b], 1);
        if (act1 && (key & hm) == p1) atomicAdd(&hist[1][b], 1);
      }
      __syncthreads();
      if (wv < 2 && (wv == 0 ? act0 : act1)) {
        const int sx = wv;
        int c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) c[u] = hist[sx][4 * lane + u];
        const int tot = c[0] + c[1] + c[2] + c[3];
        int x = tot;  // keys in buckets >= 4 lane (a suffix sum over the lanes)
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int y = __shfl_down(x, o, kWave);
          if (lane + o < kWave) x += y;
        }
        const int r = rsel[sx];
        int acc = x - tot;  // keys in buckets above the lane's four
        if (acc <= r && r < x) {
          for (int u = 3; u >= 0; --u) {
            if (r < acc + c[u]) {
              psel[sx] |= static_cast<unsigned long long>(4 * lane + u) << sh;
              rsel[sx] = r - acc;
              nsel[sx] = c[u];
              break;
            }
            acc += c[u];
          }
        }
      }
      __syncthreads();
      // once each threshold's prefix is held by its key alone (distinct
      // scores settle within the first bytes), that key is the threshold
      if (nsel[0] == 1 && nsel[1] == 1) break;  // block-uniform (LDS after a barrier)
    }
    if (pass < 7) {
      const unsigned long long hm = ~0ull << (56 - 8 * pass);
      const unsigned long long p0 = psel[0], p1 = psel[1];
      __syncthreads();  // every thread has read psel before it is replaced
      for (int i = tid; i < nc; i += kRouteNT) {
        const unsigned long long key = keys[i];
        if (act0 && (key & hm) == p0) psel[0] = key;
        if (act1 && (key & hm) == p1) psel[1] = key;
      }
      __syncthreads();
    }
    const unsigned long long t0 = psel[0], t1 = psel[1];
    for (int i = tid; i < nc; i += kRouteNT) {
      const unsigned long long key = keys[i];
      const int w = static_cast<int>(key & 0xffffffffu);
      const bool inF = nsel0 >= nc ? true : (nsel0 <= 0 ? false : key >= t0);
      const bool inR = nsel1 >= nc ? true : (nsel1 <= 0 ? false : key >= t1);
      tl[w] = inF ? 0 : (inR ? 1 : 2);
    }
  } else {
    for (int w = tid; w < nw; w += kRouteNT) tl[w] = forced[lw0 + w];
  }
  __syncthreads();
  // ---- storage of the new tiers --------------------------------------------
  int* fs = reinterpret_cast<int*>(keys);  // [nw] full-precision slot
  int* qs = fs + kTierMaxWin;              // [nw] record slot
  for (int i = tid; i < kSlotWords; i += kRouteNT) {
    freeF[i] = 0xffffffffu;
    freeQ[i] = 0xffffffffu;
    freshF[i] = 0xffffffffu;  // slots no window held before the event
  }
  __syncthreads();
  for (int w = tid; w < nw; w += kRouteNT) {
    const int f = A.fslot[lw0 + w];
    fs[w] = f;
    qs[w] = A.lslot[lw0 + w];
    if (f >= 0 && f < A.SF) atomicAnd(&freshF[f >> 5], ~(1u << (f & 31)));
  }
  __syncthreads();
  int err = 0;
  for (int w = tid; w < nw; w += kRouteNT) {
    const int o = act[w];
    int t = tl[w];
    if (o == 2 && t != 2) {  // an evicted window's storage is gone
      err |= 64;
      t = 2;
      tl[w] = 2;
    }
    const bool h0 = hl[w] != 0;
    const int f = fs[w], q = qs[w];
    const bool needF = t == 0 || (A.mat && t == 1);
    const bool quant = t == 1 && !h0;  // first demotion
    const bool needQ = t != 2 && (h0 || quant);
    const bool keepF = needF && f >= 0 && f < A.SF;
    const bool keepQ = needQ && q >= 0;
    uint8_t a = 0;
    if (needF && !keepF) a |= 1;
    if (needQ && !keepQ) a |= 2;
    if (quant) a |= 1 << 2;                                    // quantize (from slot f)
    else if (!A.mat && o == 1 && t == 0) a |= 2 << 2;         // promote (record q into a new slot)
    else if (needF && f >= A.SF) a |= 3 << 2;                 // adopt (staging into a new slot)
    act[w] = a;
    hl[w] = needQ ? 1 : 0;
    if (keepF) atomicAnd(&freeF[f >> 5], ~(1u << (f & 31)));
    if (keepQ) atomicAnd(&freeQ[q >> 5], ~(1u << (q & 31)));
    if (!keepF) fs[w] = -1;  // a new slot is given below when act bit 0 is set
    if (!keepQ) qs[w] = -1;
  }
  if (err) atomicOr(A.errflag, err);
  __syncthreads();
  // free slots: prefix popcounts of the bitmaps (slots past the pool are not free)
  const int nwf = (A.SF + 31) / 32, nwq = (A.SQ + 31) / 32;
  // free full-precision slots: fresh ones (free before the event) in freshF,
  // the ones released by it in freeF; new slots come from the fresh ones
  // first, so that their jobs need not wait for the reads of released slots
  for (int i = tid; i < kSlotWords; i += kRouteNT) {
    const int bf = A.SF - 32 * i, bq = A.SQ - 32 * i;
    const uint32_t mf = bf >= 32 ? 0xffffffffu : (bf <= 0 ? 0u : (1u << bf) - 1u);
    const uint32_t fr = freeF[i] & mf;
    freshF[i] &= fr;
    freeF[i] = fr & ~freshF[i];
    freeQ[i] &= bq >= 32 ? 0xffffffffu : (bq <= 0 ? 0u : (1u << bq) - 1u);
  }
  __syncthreads();
  if (tid < kWave) {  // one wave scans the three bitmaps
    int cf = 0, cq = 0, cn = 0;
    for (int i0 = 0; i0 < kSlotWords; i0 += kWave) {
      const int i = i0 + lane;
      int xf = __popc(freeF[i]), xq = __popc(freeQ[i]), xn = __popc(freshF[i]);
      const int yf0 = xf, yq0 = xq, yn0 = xn;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int yf = __shfl_up(xf, o, kWave), yq = __shfl_up(xq, o, kWave), yn = __shfl_up(xn, o, kWave);
        if (lane >= o) {
          xf += yf;
          xq += yq;
          xn += yn;
        }
      }
      preF[i] = cf + xf - yf0;
      preQ[i] = cq + xq - yq0;
      preN[i] = cn + xn - yn0;
      cf += __shfl(xf, kWave - 1, kWave);
      cq += __shfl(xq, kWave - 1, kWave);
      cn += __shfl(xn, kWave - 1, kWave);
    }
    if (lane == 0) {
      tots[0] = cf;
      tots[1] = cq;
      tots[2] = cn;
    }
  }
  __syncthreads();
  // requests in window order: thread tid owns windows [tid * E, tid * E + E)
  const int E = (nw + kRouteNT - 1) / kRouteNT;
  int rf = 0, rq = 0;
  for (int e = 0; e < E; ++e) {
    const int w = tid * E + e;
    if (w < nw) {
      rf += act[w] & 1;
      rq += (act[w] >> 1) & 1;
    }
  }
  int totF, totQ;
  int offF = block_excl_scan(rf, wsum, totF);
  int offQ = block_excl_scan(rq, wsum, totQ);
  int err2 = 0;
  for (int e = 0; e < E; ++e) {
    const int w = tid * E + e;
    if (w >= nw) continue;
    const uint8_t a = act[w];
    const int kind = a >> 2;
    const int fold = kind ? A.fslot[lw0 + w] : -1;  // the slot before the event (a job's source)
    int fnew = fs[w], qnew = qs[w];
    bool fresh = true;  // the job writes no slot released by this event
    if (a & 1) {
      const int r = offF++;
      if (r < tots[2]) {
        fnew = nth_bit(freshF, preN, nwf, tots[2], r);
      } else {
        fnew = nth_bit(freeF, preF, nwf, tots[0], r - tots[2]);
        fresh = false;
      }
      if (fnew < 0) err2 |= 128;
    }
    if (a & 2) {
      qnew = nth_bit(freeQ, preQ, nwq, tots[1], offQ++);
      if (qnew < 0) err2 |= 128;
    }
    if (kind && !(err2 & 128)) {
      // (window << 3 | phase 2 << 2 | kind, source full-precision slot,
      // full-precision slot after the event, record slot); a promote or
      // adopt job into a released slot waits for phase 2
      const int late = (kind != 1 && !fresh) ? 1 : 0;
      A.jobs[lw0 + atomicAdd(&njobs, 1)] = make_int4((w << 3) | (late << 2) | kind, fold, fnew, qnew);
    }
    fs[w] = fnew;
    qs[w] = qnew;
  }
  if (err2) atomicOr(A.errflag, err2);
  __syncthreads();
  // stable compaction of the two lists (entries carry the slot the
  // attention reads: the full-precision one, or the record for INT2 windows
  // read from their codes)
  int cF = 0, cQ = 0;
  for (int e = 0; e < E; ++e) {
    const int w = tid * E + e;
    if (w < nw) {
      cF += tl[w] == 0;
      cQ += tl[w] == 1;
    }
  }
  int totLF, totLQ;
  int oF = block_excl_scan(cF, wsum, totLF);
  int oQ = block_excl_scan(cQ, wsum, totLQ);
  for (int e = 0; e < E; ++e) {
    const int w = tid * E + e;
    if (w < nw) {
      // (a slot that could not be given (flag 128) reads as slot 0: in
      // bounds, and the step fails at the next check)
      if (tl[w] == 0) A.fplist[lw0 + oF++] = make_ent(max(fs[w], 0), w);
      else if (tl[w] == 1) A.qlist[lw0 + oQ++] = make_ent(max(A.mat ? fs[w] : qs[w], 0), w);
    }
  }
  // the free full-precision slots after the event, ascending (new windows
  // take them in order until the next event)
  __syncthreads();
  for (int i = tid; i < kSlotWords; i += kRouteNT) freeF[i] |= freshF[i];
  __syncthreads();
  for (int w = tid; w < nw; w += kRouteNT) {
    const int f = fs[w];
    if (f >= 0 && f < A.SF) atomicAnd(&freeF[f >> 5], ~(1u << (f & 31)));
  }
  __syncthreads();
  {
    int c = 0;
    const int EW = (kSlotWords + kRouteNT - 1) / kRouteNT;
    for (int e = 0; e < EW; ++e) {
      const int i = tid * EW + e;
      if (i < nwf) c += __popc(freeF[i]);
    }
    int tf;
    int off = block_excl_scan(c, wsum, tf);
    for (int e = 0; e < EW; ++e) {
      const int i = tid * EW + e;
      if (i >= nwf) continue;
      uint32_t b = freeF[i];
      while (b) {
        A.ffree[static_cast<int64_t>(l) * A.SF + off++] = 32 * i + __builtin_ctz(b);
        b &= b - 1;
      }
    }
  }
  // routing diagnostics over this event's candidates (aged, not evicted
  // before it): the stamps of the previous event give the overlaps, the run
  // counters the sustained absences and revivals
  const bool diag = A.rd_cnt != nullptr && forced == nullptr;
  const int ev = A.rd_event;
  int dF = 0, dFo = 0, dR = 0, dRo = 0, dS = 0, dV = 0;
  for (int w = tid; w < nw; w += kRouteNT) {
    const int64_t i = lw0 + w;
    if (diag && aged(w) && A.tier[i] != 2) {
      const bool inF = tl[w] == 0, inR = tl[w] != 2;
      if (inF) {
        ++dF;
        dFo += (ev > 1 && A.rd_fstamp[i] == ev - 1) ? 1 : 0;  // stamps start at 0
        A.rd_fstamp[i] = ev;
      }
      if (inR) {
        ++dR;
        dRo += (ev > 1 && A.rd_rstamp[i] == ev - 1) ? 1 : 0;
        A.rd_rstamp[i] = ev;
      }
      int run = A.rd_run[i];
      if (inF) {
        dV += run >= A.rd_gap ? 1 : 0;
        run = 0;
      } else {
        ++run;
        dS += run == A.rd_gap ? 1 : 0;
      }
      A.rd_run[i] = run;
    }
    A.tier[i] = tl[w];
    A.hasled[i] = hl[w];
    A.fslot[i] = fs[w];
    A.lslot[i] = qs[w];
  }
  if (diag) {
    int v[6] = {dF, dFo, dR, dRo, dS, dV};
#pragma unroll
    for (int j = 0; j < 6; ++j) {
      v[j] = wave_sum_int(v[j]);
      if (lane == 0) dsum[j][wv] = v[j];
    }
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        int t = 0;
        for (int u = 0; u < kRouteNT / kWave; ++u) t += dsum[j][u];
        v[j] = t;
      }
      int* cn = A.rd_cnt + l * 6;
      double* ac = A.rd_acc + l * 6;
      const int fp = cn[1], rp = cn[4];  // the previous event's sizes
      const bool pair = ev > 1;
      cn[0] = pair ? fp : 0;
      cn[1] = v[0];
      cn[2] = v[1];
      cn[3] = pair ? rp : 0;
      cn[4] = v[2];
      cn[5] = v[3];
      ac[0] += 1.0;
      if (pair) {
        const int uf = fp + v[0] - v[1], ur = rp + v[2] - v[3];
        ac[1] += 1.0;
        ac[2] += uf > 0 ? 1.0 - static_cast<double>(v[1]) / uf : 0.0;
        ac[3] += ur > 0 ? 1.0 - static_cast<double>(v[3]) / ur : 0.0;
      }
      ac[4] += v[4];
      ac[5] += v[5];
    }
  }
  if (tid == 0) {
    A.njobs[l] = njobs;
    if (totLF != exp_fp || totLQ != exp_q) atomicOr(A.errflag, 32);
  }
}

// ---------------------------------------------------------------------------
// Tier transitions of layer l: quantize a window's full-precision values
// into its ledger record (first demotion) or write its reconstruction,
// rounded to bf16, into its full-precision storage (promotion).  Block
// (x, l), 256 threads, takes the layer's (job, KV head) pairs x, x + gridDim.x,
// ...: a step with few transitions launches few blocks per layer, and the
// first routing event still spreads its many jobs over all of them.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void int2_group(const float* x, int n, int stride, float& sc, float& zp,
                                           uint16_t& s16, uint16_t& z16) {
  float lo = x[0], hi = x[0];
  for (int i = 1; i < n; ++i) {
    lo = fminf(lo, x[i * stride]);
    hi = fmaxf(hi, x[i * stride]);
  }
  const float span = __fsub_rn(hi, lo);
  s16 = f2h(__fdiv_rn(span, 3.0f));
  z16 = f2h(lo);
  sc = h2f(s16);
  zp = h2f(z16);
}

__device__ __forceinline__ uint8_t int2_code(float x, float sc, float zp) {
  if (sc == 0.f) return 0;
  const float t = __fdiv_rn(__fsub_rn(x, zp), sc);
  const float r = __builtin_rintf(t);  // ties to even
  return static_cast<uint8_t>(fminf(fmaxf(r, 0.f), 3.f));
}

constexpr int kXferMaxLayers = 64;  // the library's layer bound

__global__ __launch_bounds__(256) void tier_xfer_kernel(TierArgs A, int phase, int l0, int nl) {
  __shared__ float xk[W][D + 1];
  __shared__ float xv[W][D + 1];
  __shared__ uint8_t ck[W][D];
  __shared__ uint8_t cv[W][D];
  __shared__ uint32_t recl[kTierLedgerBytes / 4];
  __shared__ float ksc[D], kzp[D], vsc[W][4], vzp[W][4];  // the window's parameters as fp32
  __shared__ int jpre[kXferMaxLayers + 1];  // (job, KV head) pairs of the layers before
  const int tid = threadIdx.x;
  const int Wn = A.W;  // tokens per window (8 or 32)
  if (tid < kWave) {  // exclusive prefix of the layers' pair counts
    int c = tid < nl ? A.njobs[l0 + tid] * A.Hkv : 0;
    const int c0 = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(c, o, kWave);
      if (tid >= o) c += y;
    }
    jpre[tid] = c - c0;
    if (tid == kWave - 1) jpre[kWave] = c;
  }
  __syncthreads();
  const int total = jpre[nl];
  // the (layer, job, KV head) triples of every layer, strided over the
  // blocks; phase 1 runs the quantize jobs and the promote / adopt jobs into
  // slots that were free before the event, phase 2 those into slots the
  // event released (after phase 1 has read them)
  for (int p = blockIdx.x; p < total; p += gridDim.x) {
    int lo = 0, hi = nl - 1;  // the last layer whose pairs start at or before p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (jpre[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    const int l = l0 + lo, pq = p - jpre[lo];
    const int j = pq / A.Hkv, h = pq % A.Hkv;
    const int64_t lh = static_cast<int64_t>(l) * A.Hkv + h;
    const int4 job = A.jobs[static_cast<int64_t>(l) * A.NW + j];
    const int w = job.x >> 3, kind = job.x & 3, late = (job.x >> 2) & 1;
    if ((late ? 2 : 1) != phase) continue;  // block-uniform
    // every slot the job uses was given (the routing flags it otherwise)
    const bool ok = kind == 1 ? (job.y >= 0 && job.w >= 0 && (!A.mat || job.z >= 0))
                              : (kind == 2 ? (job.z >= 0 && job.w >= 0) : (job.y >= A.SF && job.z >= 0));
    if (!ok) continue;
    // source storage (quantize, adopt), the window's storage after the
    // event (promote, adopt, the bf16 reconstruction of a quantize) and its
    // record
    const uint16_t* ksrc = job.y >= 0 ? kfp_at(A, lh, job.y, Wn) : nullptr;
    const uint16_t* vsrc = job.y >= 0 ? vfp_at(A, lh, job.y, Wn) : nullptr;
    uint16_t* kd = job.z >= 0 ? kfp_at(A, lh, job.z, Wn) : nullptr;
    uint16_t* vd = job.z >= 0 ? vfp_at(A, lh, job.z, Wn) : nullptr;
    // keys are quantized before the rotation in rotary mode
    const uint16_t* ks = A.rope && job.y >= 0 ? kpre_at(A, lh, job.y, Wn) : ksrc;
    uint8_t* rec = job.w >= 0 ? rec_at(A, lh, job.w, A.recb) : nullptr;
    uint16_t* rec16 = reinterpret_cast<uint16_t*>(rec);
    uint32_t* rec32 = reinterpret_cast<uint32_t*>(rec);
    if (kind == 3) {
      // adopt: a prefill window from the staging buffers into its slot
      for (int i0 = 8 * tid; i0 < Wn * D; i0 += 8 * 256) {
        const uint4 kx = *reinterpret_cast<const uint4*>(ksrc + i0);
        const uint4 vx = *reinterpret_cast<const uint4*>(vsrc + i0);
        uint4 px = make_uint4(0, 0, 0, 0);
        if (A.rope) px = *reinterpret_cast<const uint4*>(ks + i0);
        *reinterpret_cast<uint4*>(kd + i0) = kx;
        *reinterpret_cast<uint4*>(vd + i0) = vx;
        if (A.rope) *reinterpret_cast<uint4*>(kpre_at(A, lh, job.z, Wn) + i0) = px;
      }
    } else if (kind == 1) {
      // stage the window in LDS as fp32: 8 consecutive elements of K
      // (token-major) and of V (channel-major) per 16-byte load, all loads
      // of the thread issued before the first store
      uint4 kr[2], vr[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i0 = 8 * (tid + 256 * u);
        const bool in = i0 < Wn * D;
        kr[u] = in ? *reinterpret_cast<const uint4*>(ks + i0) : make_uint4(0, 0, 0, 0);
        vr[u] = in ? *reinterpret_cast<const uint4*>(vsrc + i0) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i0 = 8 * (tid + 256 * u);
        if (i0 >= Wn * D) continue;
        const uint32_t kw[4] = {kr[u].x, kr[u].y, kr[u].z, kr[u].w};
        const uint32_t vw[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t kb = (kw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
          const uint32_t vb = (vw[e >> 1] >> (16 * (e & 1))) & 0xffffu;
          xk[(i0 + e) / D][(i0 + e) % D] = __uint_as_float(kb << 16);
          xv[(i0 + e) % Wn][(i0 + e) / Wn] = __uint_as_float(vb << 16);
        }
      }
      __syncthreads();
      if (tid < D && !A.kgroups) {  // keys: one channel over the window's tokens
        const int c = tid;
        float sc, zp;
        uint16_t s16, z16;
        int2_group(&xk[0][c], Wn, D + 1, sc, zp, s16, z16);
        rec16[(Wn == 8 ? kRec8SK : kRecSK) / 2 + c] = s16;
        rec16[(Wn == 8 ? kRec8ZK : kRecZK) / 2 + c] = z16;
        ksc[c] = sc;
        kzp[c] = zp;
        for (int r = 0; r < Wn; ++r) ck[r][c] = int2_code(xk[r][c], sc, zp);
      } else if (tid < D) {
        // keys grouped like the values: one token's 32-channel group,
        // parameters stored [group][token] and kept as ksc[token * 4 + group]
        if (tid / 4 < Wn) {
          const int r = tid / 4, g = tid % 4;
          float sc, zp;
          uint16_t s16, z16;
          int2_group(&xk[r][32 * g], 32, 1, sc, zp, s16, z16);
          rec16[(Wn == 8 ? kRec8SK / 2 + 8 * g : kRecSK / 2 + 32 * g) + r] = s16;
          rec16[(Wn == 8 ? kRec8ZK / 2 + 8 * g : kRecZK / 2 + 32 * g) + r] = z16;
          ksc[4 * r + g] = sc;
          kzp[4 * r + g] = zp;
          for (int c = 32 * g; c < 32 * g + 32; ++c) ck[r][c] = int2_code(xk[r][c], sc, zp);
        }
      } else if ((tid - D) / 4 < Wn) {  // values: one token's 32-channel group
        const int r = (tid - D) / 4, g = (tid - D) % 4;
        float sc, zp;
        uint16_t s16, z16;
        int2_group(&xv[r][32 * g], 32, 1, sc, zp, s16, z16);
        rec16[(Wn == 8 ? kRec8SV / 2 + 8 * g : kRecSV / 2 + 32 * g) + r] = s16;
        rec16[(Wn == 8 ? kRec8ZV / 2 + 8 * g : kRecZV / 2 + 32 * g) + r] = z16;
        vsc[r][g] = sc;
        vzp[r][g] = zp;
        for (int c = 32 * g; c < 32 * g + 32; ++c) cv[r][c] = int2_code(xv[r][c], sc, zp);
      }
      __syncthreads();
      if (Wn == 8) {
        // 8-token record: four codes a byte, element order (token, channel)
        const int e = 4 * tid;  // 256 threads cover the 1,024 elements
        uint32_t kb = 0, vb = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          kb |= static_cast<uint32_t>(ck[(e + u) / D][(e + u) % D]) << (2 * u);
          vb |= static_cast<uint32_t>(cv[(e + u) / D][(e + u) % D]) << (2 * u);
        }
        rec[kRec8K + tid] = static_cast<uint8_t>(kb);
        rec[kRec8V + tid] = static_cast<uint8_t>(vb);
      } else {
        // keys: thread = (lane ln, n-tile j, k-step ks) of the attention's
        // int8 product, 16 channels 64 ks + 16 q4 .. +16 of token 16 j + r16;
        // values: thread = (half hf, r16, tile ct), 16 tokens 16 hf .. +16 of
        // channel 16 ct + r16 (element k of a word at bits spread_bit(k))
        const int ln = tid >> 2, jt = (tid >> 1) & 1, kx = tid & 1, r16 = ln & 15, q4 = ln >> 4;
        const int hf = tid >> 7, vr16 = (tid >> 3) & 15, ct = tid & 7;
        uint32_t kw = 0, vw = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          kw |= static_cast<uint32_t>(ck[16 * jt + r16][64 * kx + 16 * q4 + e]) << spread_bit(e);
          vw |= static_cast<uint32_t>(cv[16 * hf + e][16 * ct + vr16]) << spread_bit(e);
        }
        rec32[kRecK / 4 + 4 * ln + 2 * jt + kx] = kw;
        rec32[kRecV / 4 + (hf * 16 + vr16) * 8 + ct] = vw;
      }
      if (A.mat) {
        // the reconstruction, rounded to bf16, replaces the full-precision
        // storage: code * scale + zero (separate fp32 multiply and add),
        // keys rotated at their original positions in rotary mode
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i0 = 8 * (tid + 256 * u);
          if (i0 >= Wn * D) continue;
          uint32_t ko[4] = {0, 0, 0, 0}, vo[4] = {0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = i0 + e;
            const int r = i / D, c = i % D;  // key element (token r, channel c)
            const int pk = A.kgroups ? 4 * r + (c >> 5) : c;  // the key element's parameters
            float kx = __fadd_rn(__fmul_rn(static_cast<float>(ck[r][c]), ksc[pk]), kzp[pk]);
            if (A.rope) {
              const int cp = c ^ 64, pp = A.kgroups ? 4 * r + (cp >> 5) : cp;
              const float ky = __fadd_rn(__fmul_rn(static_cast<float>(ck[r][cp]), ksc[pp]), kzp[pp]);
              kx = rope_elem(kx, ky, c, A.rcs + static_cast<int64_t>(w * Wn + r) * 128);
            }
            const int vc = i / Wn, vr_ = i % Wn;  // value element (channel vc, token vr_)
            const float vx = __fadd_rn(__fmul_rn(static_cast<float>(cv[vr_][vc]), vsc[vr_][vc >> 5]), vzp[vr_][vc >> 5]);
            ko[e >> 1] |= bf16_rne(kx) << (16 * (e & 1));
            vo[e >> 1] |= bf16_rne(vx) << (16 * (e & 1));
          }
          *reinterpret_cast<uint4*>(kd + i0) = make_uint4(ko[0], ko[1], ko[2], ko[3]);
          *reinterpret_cast<uint4*>(vd + i0) = make_uint4(vo[0], vo[1], vo[2], vo[3]);
        }
      }
      __syncthreads();
    } else if (kind == 2 && !A.mat) {
      // (with bf16 reconstruction the storage already holds what a
      // promotion would write)
      // the record into LDS (3,072 B, three words per thread), then 8
      // consecutive elements of K (one token) and of V (one channel) per
      // thread and 16-byte store
      uint32_t rw[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) rw[u] = rec32[tid + 256 * u];
#pragma unroll
      for (int u = 0; u < 3; ++u) recl[tid + 256 * u] = rw[u];
      __syncthreads();
      const uint16_t* rl16 = reinterpret_cast<const uint16_t*>(recl);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i0 = 8 * (tid + 256 * u);
        uint32_t ko[4], vo[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t kb, vb;
          {  // key element (token r, channel c)
            const int i = i0 + e, r = i / D, c = i % D;
            const int ln = ((c >> 4) & 3) * 16 + (r & 15);
            const uint32_t code = (recl[kRecK / 4 + 4 * ln + 2 * (r >> 4) + (c >> 6)] >> spread_bit(c & 15)) & 3u;
            const float sc = h2f(rl16[kRecSK / 2 + c]), zp = h2f(rl16[kRecZK / 2 + c]);
            kb = bf16_rne(__fadd_rn(__fmul_rn(static_cast<float>(code), sc), zp));
          }
          {  // value element (channel c, token r): channel-major index
            const int i = i0 + e, c = i / W, r = i % W;
            const uint32_t code = (recl[kRecV / 4 + ((r >> 4) * 16 + (c & 15)) * 8 + (c >> 4)] >> spread_bit(r & 15)) & 3u;
            const int g = c >> 5;
            const float sc = h2f(rl16[kRecSV / 2 + 32 * g + r]), zp = h2f(rl16[kRecZV / 2 + 32 * g + r]);
            vb = bf16_rne(__fadd_rn(__fmul_rn(static_cast<float>(code), sc), zp));
          }
          if (e & 1) {
            ko[e >> 1] |= kb << 16;
            vo[e >> 1] |= vb << 16;
          } else {
            ko[e >> 1] = kb;
            vo[e >> 1] = vb;
          }
        }
        *reinterpret_cast<uint4*>(kd + i0) = make_uint4(ko[0], ko[1], ko[2], ko[3]);
        *reinterpret_cast<uint4*>(vd + i0) = make_uint4(vo[0], vo[1], vo[2], vo[3]);
      }
      __syncthreads();  // recl is reused by the block's next job
    }
  }
}

// ---------------------------------------------------------------------------
// Export of the full-precision storage of (layer l, KV head h), windows
// [0, nwin), token-major: k_out, v_out [nwin * W][128]; a window that holds
// no full-precision storage exports zeros.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tier_export_kernel(TierArgs A, int l, int h, uint16_t* __restrict__ k_out,
                                                          uint16_t* __restrict__ v_out) {
  const int w = blockIdx.x, tid = threadIdx.x;
  const int64_t lh = static_cast<int64_t>(l) * A.Hkv + h;
  const int Wn = A.W;
  const int s = A.fslot[static_cast<int64_t>(l) * A.NW + w];
  const uint16_t* ks = s >= 0 ? kfp_at(A, lh, s, Wn) : nullptr;
  const uint16_t* vs = s >= 0 ? vfp_at(A, lh, s, Wn) : nullptr;
  for (int i = tid; i < Wn * D; i += 256) {
    const int r = i / D, c = i % D;
    k_out[static_cast<int64_t>(w) * Wn * D + i] = s >= 0 ? ks[i] : 0;
    v_out[static_cast<int64_t>(w) * Wn * D + i] = s >= 0 ? vs[c * Wn + r] : 0;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static TierArgs tier_args(kvev_ctx* c) {
  TierArgs a;
  a.kfp = c->td.kfp;
  a.vfp = c->td.vfp;
  a.ledger = c->td.ledger;
  a.tier = c->td.tier;
  a.hasled = c->td.hasled;
  a.S = c->td.S;
  a.fplist = c->td.fplist;
  a.qlist = c->td.qlist;
  a.jobs = c->td.jobs;
  a.njobs = c->td.njobs;
  a.part_ml = c->d.part_ml;
  a.part_o = c->d.part_o;
  a.ml = c->d.ml;
  a.emass = c->td.emass;
  a.errflag = c->d.errflag;
  a.rd_fstamp = c->td.rd_fstamp;
  a.rd_rstamp = c->td.rd_rstamp;
  a.rd_run = c->td.rd_run;
  a.rd_cnt = c->td.rd_cnt;
  a.rd_acc = c->td.rd_acc;
  a.rd_gap = c->cfg.revival_gap;
  a.rd_event = c->tw.events + 1;
  a.L = c->cfg.n_layers;
  a.Hkv = c->cfg.n_kv_heads;
  a.Hq = c->cfg.n_q_heads;
  a.NW = c->tw.NW;
  a.maxch = c->tw.maxch;
  a.W = c->tw.W;
  a.rope = c->tw.rope ? 1 : 0;
  a.mat = c->tw.mat ? 1 : 0;
  a.recb = tier_rec_bytes(c->tw.W);
  a.kpre = c->td.kpre;
  a.rcs = c->td.rcs;
  a.ifreq = c->td.ifreq;
  a.kst = c->td.kst;
  a.vst = c->td.vst;
  a.kpst = c->td.kpst;
  a.fslot = c->td.fslot;
  a.lslot = c->td.lslot;
  a.ffree = c->td.ffree;
  a.SF = c->tw.SF;
  a.SQ = c->tw.SQ;
  a.NWS = c->tw.NWS;
  a.kgroups = c->tw.kgroups ? 1 : 0;
  return a;
}

// windows per attention chunk: (full-precision list, INT2 list)
static void tier_chunk_windows(const kvev_ctx* c, int& cw_f, int& cw_q) {
  cw_f = 4 * (64 / c->tw.W);
  cw_q = c->tw.mat ? cw_f : 4 * kQW;
}

hipError_t launch_tier_rope_table(kvev_ctx* c, int64_t p0, int64_t n) {
  const int64_t threads = n * 64;
  // timed as "rope" on decode steps (one new position), untimed at prefill
  return timed_launch(c, n == 1 ? "rope" : nullptr, tier_rope_table_kernel,
                      dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, tier_args(c), p0, n);
}

hipError_t launch_tier_prefill(kvev_ctx* c, const void* k, const void* v, int64_t n) {
  const int nwin = static_cast<int>((n + c->tw.W - 1) / c->tw.W);
  dim3 grid(nwin, c->cfg.n_kv_heads, c->cfg.n_layers);
  tier_prefill_kernel<<<grid, 256, 0, c->stream>>>(tier_args(c), static_cast<const uint16_t*>(k),
                                                   static_cast<const uint16_t*>(v), static_cast<int>(n));
  return hipGetLastError();
}

hipError_t launch_tier_append(kvev_ctx* c, const void* k_new, const void* v_new, int kslot) {
  dim3 grid(c->cfg.n_kv_heads, c->cfg.n_layers);
  return timed_launch(c, "append", tier_append_kernel, grid, dim3(D), 0, tier_args(c),
                      static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                      static_cast<int>(c->tw.npos), c->tw.n_fp, kslot);
}

hipError_t launch_tier_attention(kvev_ctx* c, const void* q) {
  int cw_f, cw_q;
  tier_chunk_windows(c, cw_f, cw_q);
  const int nch_f = (c->tw.n_fp + cw_f - 1) / cw_f, nch_q = (c->tw.n_q + cw_q - 1) / cw_q;
  const int npos = static_cast<int>(c->tw.npos);
  TierArgs a = tier_args(c);
  dim3 grid(nch_f + nch_q, c->cfg.n_kv_heads, c->cfg.n_layers);
  const auto* qq = static_cast<const uint16_t*>(q);
  const float scale = 1.0f / sqrtf(static_cast<float>(D));
  auto kern = c->tw.W == 8 ? tier_attn_kernel<8, true>
                            : (c->tw.mat ? tier_attn_kernel<32, true> : tier_attn_kernel<32, false>);
  return timed_launch(c, "attn", kern, grid, dim3(256), 0, a, qq, c->tw.n_fp, c->tw.n_q, nch_f, npos, scale);
}

hipError_t launch_tier_merge(kvev_ctx* c, float* out) {
  int cw_f, cw_q;
  tier_chunk_windows(c, cw_f, cw_q);
  const int nch_f = (c->tw.n_fp + cw_f - 1) / cw_f, nch_q = (c->tw.n_q + cw_q - 1) / cw_q;
  TierArgs a = tier_args(c);
  hipError_t e;
  dim3 gm(HG, c->cfg.n_kv_heads, c->cfg.n_layers);
  const size_t shm = sizeof(float) * 2 * static_cast<size_t>(nch_f + nch_q);
  e = timed_launch(c, "merge", tier_merge_kernel, gm, dim3(256), shm, a, out, nch_f + nch_q);
  if (e != hipSuccess) return e;
  const int ntot = c->tw.n_fp + c->tw.n_q;
  dim3 gs((ntot + 255) / 256, c->cfg.n_layers);
  return timed_launch(c, "mass", tier_mass_kernel, gs, dim3(256), 0, a, c->tw.n_fp, c->tw.n_q, nch_f, cw_f, cw_q);
}

hipError_t launch_tier_route(kvev_ctx* c, int nw, int np, int recent_lo, int exp_fp, int exp_q,
                             const uint8_t* forced_dev, int layer) {
  TierArgs a = tier_args(c);
  const int l0 = layer < 0 ? 0 : layer, nl = layer < 0 ? c->cfg.n_layers : 1;
  hipError_t e = timed_launch(c, "route", tier_route_kernel, dim3(nl), dim3(kRouteNT), 0, a, nw, np, recent_lo,
                              static_cast<int>(c->cfg.fp_windows), static_cast<int>(c->cfg.int2_windows), exp_fp,
                              exp_q, forced_dev, l0);
  if (e != hipSuccess) return e;
  // one residency round of blocks over every layer's jobs
  e = timed_launch(c, "xfer", tier_xfer_kernel, dim3(kTierXferBlocks), dim3(256), 0, a, 1, l0,
                   nl);  // quantize, jobs into fresh slots
  if (e != hipSuccess) return e;
  return timed_launch(c, "xfer", tier_xfer_kernel, dim3(kTierXferBlocks), dim3(256), 0, a, 2, l0,
                      nl);  // jobs into released slots
}

hipError_t launch_tier_export(kvev_ctx* c, int l, int h, void* k_out, void* v_out, int nwin) {
  tier_export_kernel<<<nwin, 256, 0, c->stream>>>(tier_args(c), l, h, static_cast<uint16_t*>(k_out),
                                                  static_cast<uint16_t*>(v_out));
  return hipGetLastError();
}

}  // namespace kvev
