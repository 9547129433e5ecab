"""Seeded synthetic workloads (inputs only; none of the method's arithmetic).

Every tensor is a pure function of (workload seed, tensor kind, layer,
sequence, head, step) through a counter-based 32-bit integer hash, so any
slice can be regenerated alone, on the CPU or on the GPU, with identical
bits: the hash runs in torch int64 arithmetic (exact on both devices), a
standard-normal value is read from a fixed inverse-CDF table, and the few
floating-point operations applied afterwards (x8 outlier scaling, adding the
mean-query offset, bf16 rounding) are single IEEE operations.

Workload recipe (shapes and structure of the pages' settings: Llama-3.1-8B
GQA attention, 8k-131k contexts, 5-25% budgets):

* K, V, Q entries ~ N(0, 1) (65536-level inverse-CDF quantiles).
* Outlier channels: 4 of the 128 channels are scaled x8, drawn
  independently for K and for Q per (layer, sequence, KV head); the Q set is
  shared by the KV head's query group.  ``outlier_shared_qk`` takes the
  other reading of the 32k workload's wording: the same 4 channels in Q and
  K (logits then grow about five times wider and one token takes nearly all
  of a group's mass).
* Mean query direction u: a unit vector with +-1/8 on 64 hashed channels.
  Queries add mu*u with mu = |c|/4, |c| = sqrt(124 + 4*64) the expected row
  norm.  Heavy keys: 64 positions per (layer, sequence, KV head, epoch) in
  [4, L0) are replaced by |c| (0.6 u + 0.8 w), w a unit vector with +-1/8 on
  the other 64 channels (cosine 0.6 with u).  Epoch e of a multi-epoch run
  uses its own u_e; all epochs' heavy keys are planted at prefill.
* New keys / values appended at decode steps have no heavy rows.
* Block-granular workloads: the heavy positions of an epoch are shared by
  every layer and KV head of a sequence (``heavy_shared``), so they mark
  whole blocks; region labels are contiguous spans in the order system,
  plan, user, tool, scratch with the configured fractions (cut points
  floor(cumulative fraction * L0)); the block budget is the configured
  fraction of the prefill's blocks, rounded half up.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

_M32 = 0xFFFFFFFF
_TABLE_CACHE = {}

# tensor-kind ids of the hash streams
_K, _V, _Q, _KN, _VN = 1, 2, 3, 4, 5
_META_KOUT, _META_QOUT, _META_U, _META_HEAVY, _META_LEN = 11, 12, 13, 14, 15


def _mix32_int(x: int) -> int:
    x &= _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    return (x >> 16) ^ x


def stream_key(*fields: int) -> int:
    """32-bit key of one stream, chained through the hash field by field."""
    k = 0x9E3779B9
    for f in fields:
        k = _mix32_int(k ^ (int(f) & _M32))
        k = _mix32_int(k + 0x7F4A7C15)
    return k


def stream_keys(*fields) -> np.ndarray:
    """stream_key over broadcast integer arrays of fields: the same 32-bit
    chain evaluated elementwise in int64 (identical values)."""
    arrs = np.broadcast_arrays(*[np.asarray(f, dtype=np.int64) for f in fields])
    k = np.full(arrs[0].shape, 0x9E3779B9, dtype=np.int64)
    for f in arrs:
        k = _mix32_np(k ^ (f & _M32))
        k = _mix32_np(k + 0x7F4A7C15)
    return k


def _mix32_np(x):
    x = x & _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    return (x >> 16) ^ x


def _mix32_t(x):
    x = x & _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    return (x >> 16) ^ x


def _normal_table(device):
    import torch
    key = str(device)
    if key not in _TABLE_CACHE:
        from scipy.special import ndtri
        vals = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0).astype(np.float32)
        _TABLE_CACHE[key] = torch.from_numpy(vals).to(device)
    return _TABLE_CACHE[key]


def normal_stream(key: int, shape, device="cpu"):
    """float32 tensor of N(0,1) quantiles, element i from hash(hash(i) ^ key)."""
    import torch
    n = int(np.prod(shape))
    idx = torch.arange(n, dtype=torch.int64, device=device)
    h = _mix32_t(_mix32_t(idx) ^ key)
    return _normal_table(device)[h >> 16].reshape(shape)


def _rank_channels(key: int, n: int) -> np.ndarray:
    """A key-dependent permutation of range(n) (sorting hashed ids)."""
    h = _mix32_np(_mix32_np(np.arange(n, dtype=np.int64)) ^ key)
    return np.lexsort((np.arange(n), h))


def _rank_channels_many(keys, n: int) -> np.ndarray:
    """_rank_channels for every key of an integer array: [..., n]."""
    keys = np.asarray(keys, dtype=np.int64)
    h = _mix32_np(_mix32_np(np.arange(n, dtype=np.int64)) ^ keys[..., None])
    ids = np.broadcast_to(np.arange(n, dtype=np.int64), h.shape)
    return np.lexsort((ids, h), axis=-1)


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload and its eviction settings."""
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                      # "f32" or "bf16"
    prefill_lens: tuple             # per sequence
    steps: int
    seed: int
    alpha_new: float = 0.05
    budget: int = 0                 # per selection group (tokens or blocks)
    n_sink: int = 0
    n_recent: int = 0
    policy: str = "ema"             # ema | cumulative | lrfu_block | tiered_int2
    refresh_interval: int = 1
    score_free: bool = False
    structured: bool = True         # outliers, mean query direction, heavy keys
    n_heavy: int = 64
    n_epochs: int = 1
    epoch_steps: int = 0            # 0: one epoch for the whole run
    beta: float = 0.001
    page_tokens: int = 16
    region_fracs: tuple = ()
    region_half_lives: tuple = ()
    pinned_regions: tuple = ()
    window_tokens: int = 32
    fp_windows: int = 0
    int2_windows: int = 0
    heavy_shared: bool = False      # heavy positions per (sequence, epoch) only
    budget_frac: float = 0.0        # block budget as a fraction of prefill blocks
    decode_region: int = 4
    scorer: str = "attention"       # attention | vnorm | entropy | vnorm+entropy
    granularity: str = "kv_head"    # kv_head | sequence
    route_interval: int = 1         # tiered mode: routing events every route_interval steps
    diag_topk: int = 0              # token modes: rank-trace diagnostics over the top-k (0: off)
    offload_blocks: int = 0         # block mode: host-offload pool slots (0: off)
    revival_gap: int = 0            # tiered mode: routing diagnostics, sustained-absence length (0: off)
    attn_path: int = 0              # token and block modes: attention kernel (0 auto, 1 split, 2 whole-cache)
    evict_interval: int = 1         # token modes: select only every evict_interval steps
    rope_theta: float = 0.0         # tiered mode: keys and queries arrive before the rotary embedding
    int2_key_groups: int = 0        # tiered mode: 1 = keys quantized per token and 32-channel group
    outlier_shared_qk: bool = False  # the same outlier channels in Q and K
    new_token_init: int = 0         # token modes: 1 = the new token starts at the mean on observation steps too
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def batch(self):
        return len(self.prefill_lens)

    @property
    def group_size(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def torch_dtype(self):
        import torch
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def scaled(self, **kw):
        return replace(self, extra={}, **kw)

    # -- per-(layer, sequence, KV head) structure --------------------------
    def _structure(self, layer, seq, kvh):
        d = self.head_dim
        kout = _rank_channels(stream_key(self.seed, _META_KOUT, layer, seq, kvh), d)[:4]
        qmeta = _META_KOUT if self.outlier_shared_qk else _META_QOUT
        qout = _rank_channels(stream_key(self.seed, qmeta, layer, seq, kvh), d)[:4]
        ck = np.ones(d, np.float32)
        ck[kout] = 8.0
        cq = np.ones(d, np.float32)
        cq[qout] = 8.0
        return ck, cq

    def _directions(self, layer, seq, kvh, epoch):
        d = self.head_dim
        perm = _rank_channels(stream_key(self.seed, _META_U, layer, seq, kvh, epoch), d)
        signs = np.where(_mix32_np(np.arange(d, dtype=np.int64) ^ stream_key(
            self.seed, _META_U + 100, layer, seq, kvh, epoch)) & 1, 1.0, -1.0)
        u = np.zeros(d, np.float32)
        w = np.zeros(d, np.float32)
        half = d // 2
        u[perm[:half]] = (signs[perm[:half]] / math.sqrt(half)).astype(np.float32)
        w[perm[half:]] = (signs[perm[half:]] / math.sqrt(half)).astype(np.float32)
        return u, w

    def _structure_many(self, layers, seqs, heads):
        """(ck, cq) of _structure for broadcast index arrays: [..., d]."""
        d = self.head_dim
        out = []
        for meta in (_META_KOUT, _META_KOUT if self.outlier_shared_qk else _META_QOUT):
            top = _rank_channels_many(stream_keys(self.seed, meta, layers, seqs, heads), d)[..., :4]
            c = np.ones(top.shape[:-1] + (d,), np.float32)
            np.put_along_axis(c, top, np.float32(8.0), axis=-1)
            out.append(c)
        return out[0], out[1]

    def _u_many(self, layers, seqs, heads, epoch):
        """The u of _directions for broadcast index arrays: [..., d]."""
        d = self.head_dim
        half = d // 2
        perm = _rank_channels_many(stream_keys(self.seed, _META_U, layers, seqs, heads, epoch), d)
        sk = stream_keys(self.seed, _META_U + 100, layers, seqs, heads, epoch)
        signs = np.where(_mix32_np(np.arange(d, dtype=np.int64) ^ sk[..., None]) & 1, 1.0, -1.0)
        vals = (np.take_along_axis(signs, perm[..., :half], axis=-1) / math.sqrt(half)).astype(np.float32)
        u = np.zeros(perm.shape, np.float32)
        np.put_along_axis(u, perm[..., :half], vals, axis=-1)
        return u

    def _norm_c(self):
        return math.sqrt((self.head_dim - 4) + 4 * 64.0)

    def heavy_positions(self, layer, seq, kvh, epoch):
        L0 = self.prefill_lens[seq]
        lo = 4
        if L0 - lo < self.n_heavy:
            return np.zeros(0, np.int64)
        if self.heavy_shared:
            ck = (seq, epoch)
        else:
            ck = (layer, seq, kvh, epoch)
        cache = self.extra.setdefault("_heavy", {})
        if ck not in cache:
            key = stream_key(self.seed, _META_HEAVY, *ck)
            # distinct positions: sort hashed candidate ids and take the first n
            cand = np.arange(lo, L0, dtype=np.int64)
            h = _mix32_np(_mix32_np(cand) ^ key)
            cache[ck] = np.sort(cand[np.lexsort((cand, h))[: self.n_heavy]])
        return cache[ck]

    def _heavy_rows(self, layer, seq, kvh):
        """(positions, rows [n, d]) of every epoch's heavy keys for one
        (layer, sequence, KV head); a position heavy in several epochs takes
        the latest epoch's row."""
        nc = self._norm_c()
        owner = {}
        for e in range(self.n_epochs):
            for p in self.heavy_positions(layer, seq, kvh, e).tolist():
                owner[p] = e
        if not owner:
            return np.zeros(0, np.int64), np.zeros((0, self.head_dim), np.float32)
        pos = np.array(sorted(owner), dtype=np.int64)
        rows = {}
        for e in sorted(set(owner.values())):
            u, w = self._directions(layer, seq, kvh, e)
            rows[e] = (np.float32(nc * 0.6) * u + np.float32(nc * 0.8) * w).astype(np.float32)
        return pos, np.stack([rows[owner[p]] for p in pos.tolist()])

    def _heavy_rows_at(self, layer, seq, kvh, pos):
        """(indices into pos, rows) of the requested positions that hold a
        heavy key, each with the latest owning epoch's row: the rows of
        _heavy_rows restricted to pos, with directions computed only for
        the epochs that own one of them."""
        pos = np.asarray(pos, dtype=np.int64)
        owner = np.full(len(pos), -1, dtype=np.int64)
        for e in range(self.n_epochs):
            owner[np.isin(pos, self.heavy_positions(layer, seq, kvh, e))] = e
        hit = np.flatnonzero(owner >= 0)
        rows = np.zeros((len(hit), self.head_dim), np.float32)
        nc = self._norm_c()
        for e in np.unique(owner[hit]).tolist():
            u, w = self._directions(layer, seq, kvh, e)
            rows[owner[hit] == e] = (np.float32(nc * 0.6) * u + np.float32(nc * 0.8) * w).astype(np.float32)
        return hit, rows

    def region_labels(self, seq):
        """uint8 region id of every prefill position (contiguous spans)."""
        L0 = self.prefill_lens[seq]
        from fractions import Fraction
        lab = np.zeros(L0, np.uint8)
        cum = Fraction(0)
        for r, f in enumerate(self.region_fracs):
            lo = math.floor(cum * L0)
            cum += Fraction(str(f))
            hi = L0 if r == len(self.region_fracs) - 1 else math.floor(cum * L0)
            lab[lo:hi] = r
        return lab

    def block_budget(self, seq):
        nb = -(-self.prefill_lens[seq] // self.page_tokens)
        return max(1, int(math.floor(self.budget_frac * nb + 0.5)))

    def heavy_blocks(self, seq, epoch):
        """Blocks holding epoch ``epoch``'s heavy keys (shared positions)."""
        pos = self.heavy_positions(0, seq, 0, epoch)
        return sorted(set((pos // self.page_tokens).tolist()))

    def epoch_of(self, t):
        if self.epoch_steps <= 0:
            return 0
        return min((t - 1) // self.epoch_steps, self.n_epochs - 1)

    # -- tensors -------------------------------------------------------------
    def _round(self, x):
        import torch
        return x if self.dtype == "f32" else x.to(torch.bfloat16)

    def prefill_kv(self, seq, device="cpu", layers=None, heads=None):
        """(K, V) of one sequence: [len(layers), len(heads), L0, d]."""
        import torch
        layers = range(self.n_layers) if layers is None else layers
        heads = range(self.n_kv_heads) if heads is None else heads
        L0, d = self.prefill_lens[seq], self.head_dim
        Ks, Vs = [], []
        for l in layers:
            kh, vh = [], []
            for h in heads:
                k = normal_stream(stream_key(self.seed, _K, l, seq, h), (L0, d), device)
                v = normal_stream(stream_key(self.seed, _V, l, seq, h), (L0, d), device)
                if self.structured:
                    ck, _ = self._structure(l, seq, h)
                    k = k * torch.from_numpy(ck).to(device)
                    pos, rows = self._heavy_rows(l, seq, h)
                    if len(pos):
                        k[torch.from_numpy(pos).to(device)] = torch.from_numpy(rows).to(device)
                kh.append(self._round(k))
                vh.append(self._round(v))
            Ks.append(torch.stack(kh))
            Vs.append(torch.stack(vh))
        return torch.stack(Ks), torch.stack(Vs)

    def prefill_rows(self, seq, positions, device="cpu"):
        """(K, V) of chosen prefill positions: [L, Hkv, len(positions), d],
        bit-identical to the same rows of ``prefill_kv``."""
        import torch
        pos = np.asarray(positions, dtype=np.int64)
        d = self.head_dim
        idx = torch.from_numpy(pos[:, None] * d + np.arange(d)[None, :]).to(device)
        table = _normal_table(device)
        Ks, Vs = [], []
        for l in range(self.n_layers):
            kh, vh = [], []
            for h in range(self.n_kv_heads):
                hk = _mix32_t(_mix32_t(idx) ^ stream_key(self.seed, _K, l, seq, h))
                hv = _mix32_t(_mix32_t(idx) ^ stream_key(self.seed, _V, l, seq, h))
                k = table[hk >> 16]
                v = table[hv >> 16]
                if self.structured:
                    ck, _ = self._structure(l, seq, h)
                    k = k * torch.from_numpy(ck).to(device)
                    hit, rows = self._heavy_rows_at(l, seq, h, pos)
                    if len(hit):
                        k[torch.from_numpy(hit).to(device)] = torch.from_numpy(rows).to(device)
                kh.append(self._round(k))
                vh.append(self._round(v))
            Ks.append(torch.stack(kh))
            Vs.append(torch.stack(vh))
        return torch.stack(Ks), torch.stack(Vs)

    def _step_structure(self, seqs, epoch):
        """Stacked (ck, cq, mu*u) arrays [L, len(seqs), Hkv, d] (cached)."""
        cache = self.extra.setdefault("_step_structure", {})
        key = (tuple(seqs), epoch)
        if key not in cache:
            L, Hkv, d = self.n_layers, self.n_kv_heads, self.head_dim
            ck = np.ones((L, len(seqs), Hkv, d), np.float32)
            cq = np.ones((L, len(seqs), Hkv, d), np.float32)
            mu_u = np.zeros((L, len(seqs), Hkv, d), np.float32)
            if self.structured:
                mu = np.float32(self._norm_c() / 4.0)
                lg = np.arange(L, dtype=np.int64)[:, None, None]
                bg = np.asarray(seqs, dtype=np.int64)[None, :, None]
                hg = np.arange(Hkv, dtype=np.int64)[None, None, :]
                ck, cq = self._structure_many(lg, bg, hg)
                mu_u = (mu * self._u_many(lg, bg, hg, epoch)).astype(np.float32)
            cache[key] = (ck, cq, mu_u)
        return cache[key]

    def step_inputs(self, t, device="cpu", seqs=None):
        """(q [L,b,Hq,d], k_new [L,b,Hkv,d], v_new [L,b,Hkv,d]) for step t >= 1."""
        import torch
        seqs = list(range(self.batch)) if seqs is None else list(seqs)
        L, d, Hkv, Hg = self.n_layers, self.head_dim, self.n_kv_heads, self.group_size
        nb = len(seqs)

        lg = np.arange(L, dtype=np.int64)[:, None, None]
        bg = np.asarray(seqs, dtype=np.int64)[None, :, None]
        hg = np.arange(Hkv, dtype=np.int64)[None, None, :]

        def keys(kind):
            return torch.from_numpy(stream_keys(self.seed, kind, lg, bg, hg, t)).to(device)

        table = _normal_table(device)
        idx_kv = _mix32_t(torch.arange(d, dtype=torch.int64, device=device))
        idx_q = _mix32_t(torch.arange(Hg * d, dtype=torch.int64, device=device))
        k = table[_mix32_t(idx_kv ^ keys(_KN)[..., None]) >> 16]            # [L,b,Hkv,d]
        v = table[_mix32_t(idx_kv ^ keys(_VN)[..., None]) >> 16]
        z = table[_mix32_t(idx_q ^ keys(_Q)[..., None]) >> 16].reshape(L, nb, Hkv, Hg, d)
        if self.structured:
            ck, cq, mu_u = (torch.from_numpy(a).to(device)
                            for a in self._step_structure(seqs, self.epoch_of(t)))
            k = k * ck
            z = z * cq[:, :, :, None, :]
            z = z + mu_u[:, :, :, None, :]
        q = z.reshape(L, nb, Hkv * Hg, d)
        return self._round(q), self._round(k), self._round(v)


def _lengths(seed, n, lo, hi):
    key = stream_key(seed, _META_LEN)
    h = _mix32_np(_mix32_np(np.arange(n, dtype=np.int64)) ^ key)
    return tuple(int(lo + (x % (hi - lo + 1))) for x in h)


def workload(name: str) -> Workload:
    """The configured workloads, by short name: the five of the method's
    configurations plus variants of the 32k one (pooled granularity, the
    scorer variants, the Qwen2.5-7B group shape)."""
    if name == "tiny":
        return Workload("tiny_inertiakv_1L_8q2kv_d64_f32", 1, 8, 2, 64, "f32", (512,), 64,
                        seed=1001, alpha_new=0.05, budget=128, structured=False)
    if name == "llama8b_32k":
        return Workload("llama8b_32k_10pct", 32, 32, 8, 128, "bf16", (32768,), 256,
                        seed=1002, alpha_new=0.05, budget=3277, n_sink=4, n_recent=32)
    if name == "llama8b_32k_pooled":
        # one utility and one retained set per sequence ("What Matters ...", section 3.1 Eq.1)
        return Workload("llama8b_32k_10pct_pooled", 32, 32, 8, 128, "bf16", (32768,), 256,
                        seed=1002, alpha_new=0.05, budget=3277, n_sink=4, n_recent=32,
                        granularity="sequence")
    if name == "llama8b_32k_vnorm_entropy":
        return Workload("llama8b_32k_10pct_vnorm_entropy", 32, 32, 8, 128, "bf16", (32768,), 256,
                        seed=1002, alpha_new=0.05, budget=3277, n_sink=4, n_recent=32,
                        scorer="vnorm+entropy")
    if name == "qwen7b_32k":
        # Qwen2.5-7B attention shape: 28 layers, 28 query and 4 KV heads (groups of 7)
        return Workload("qwen2.5_7b_32k_10pct", 28, 28, 4, 128, "bf16", (32768,), 256,
                        seed=1006, alpha_new=0.05, budget=3277, n_sink=4, n_recent=32)
    if name == "lazy16x8k":
        return Workload("batch16_8k_25pct_lazy8", 32, 32, 8, 128, "bf16", (8192,) * 16, 512,
                        seed=1003, alpha_new=0.05, budget=2048, refresh_interval=8)
    if name == "lazy16x8k_evict8":
        # the batched lazy workload's wording taken literally: scores recomputed and the cache
        # evicted every 8 steps (it grows to the budget + 7 in between)
        return replace(workload("lazy16x8k"), name="batch16_8k_25pct_lazy8_evict8", evict_interval=8)
    if name == "scorefree16x8k":
        return Workload("batch16_8k_25pct_scorefree", 32, 32, 8, 128, "bf16", (8192,) * 16, 512,
                        seed=1003, alpha_new=0.05, budget=2048, score_free=True, n_recent=32)
    if name == "lrfu64":
        return Workload("lrfu_64seq_4k16k_blocks20pct", 32, 32, 8, 128, "bf16",
                        _lengths(1004, 64, 4096, 16384), 1024, seed=1004, alpha_new=0.05,
                        policy="lrfu_block", beta=0.001, n_epochs=32, epoch_steps=32,
                        n_heavy=16, heavy_shared=True, budget_frac=0.2,
                        region_fracs=(0.1, 0.1, 0.2, 0.4, 0.2),
                        region_half_lives=(170.0, 100.0, 60.0, 30.0, 15.0), pinned_regions=(0,))
    if name == "qevict131k":
        return Workload("qevict_131k_fp5_int2_20", 32, 32, 8, 128, "bf16", (131072,), 128,
                        seed=1005, policy="tiered_int2", n_sink=5, n_recent=32, n_epochs=4,
                        epoch_steps=32, window_tokens=32, fp_windows=205, int2_windows=819)
    if name == "llama8b_32k_diag":
        # rank-trace diagnostics at k = the budget ("What Matters ...", appendix I)
        return replace(workload("llama8b_32k"), name="llama8b_32k_10pct_diag", diag_topk=3277)
    if name == "lrfu64_offload":
        # evicted blocks kept in a pinned host pool of 1,024 blocks ("MemDecay" section III-E)
        return replace(workload("lrfu64"), name="lrfu_64seq_4k16k_blocks20pct_offload1024",
                       offload_blocks=1024)
    if name == "qevict131k_omega8":
        # the review's routing interval: one routing event every 8 steps (section 4.2 Eq.1)
        return replace(workload("qevict131k"), name="qevict_131k_fp5_int2_20_omega8", route_interval=8)
    if name == "qevict65k_w8_rope":
        # the review's own defaults: 8-token windows, routing every 8 steps, keys quantized before
        # the rotary embedding and rotated again on promotion (section 4.4), tier capacities from
        # the byte budget with q = 0.70 (section 4.3 Eq.3): B_hist = 10% of the prefill's
        # full-precision bytes, M_f = 8 tokens x 4,096 B and M_q = 8 KV heads x the 1,152-byte
        # record, per window and layer
        n = 65536
        m_f, m_q = 8 * 4096, 8 * 1152
        b_hist = 0.1 * (n // 8) * m_f
        return Workload("qevict_65k_w8_rope", 32, 32, 8, 128, "bf16", (n,), 128, seed=1006,
                        policy="tiered_int2", n_sink=5, n_recent=32, n_epochs=4, epoch_steps=32,
                        window_tokens=8, fp_windows=int(0.3 * b_hist // m_f),
                        int2_windows=int(0.7 * b_hist // m_q), route_interval=8, rope_theta=500000.0)
    if name == "qevict131k_allfp":
        # calibration: every routed window full precision (the tier split of the attention)
        return replace(workload("qevict131k"), name="qevict_131k_allfp", fp_windows=1024, int2_windows=0)
    if name == "qevict131k_allint2":
        # calibration: every routed window INT2
        return replace(workload("qevict131k"), name="qevict_131k_allint2", fp_windows=0, int2_windows=1024)
    raise KeyError(name)


WORKLOADS = ("tiny", "llama8b_32k", "lazy16x8k", "scorefree16x8k", "lrfu64", "qevict131k",
             "llama8b_32k_pooled", "llama8b_32k_vnorm_entropy", "qwen7b_32k", "qevict131k_omega8",
             "llama8b_32k_diag", "lrfu64_offload", "lazy16x8k_evict8", "qevict131k_allfp", "qevict131k_allint2",
             "qevict65k_w8_rope")
