"""ctypes binding of libkvev.so: argument marshalling only.

Every step of the eviction path runs in the library's HIP kernels; this
module checks tensor shapes, dtypes and devices on the host (so the C side
never reads out of bounds), passes raw pointers and turns status codes into
exceptions.  PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvev.so")

OK, EINVAL, ENOMEM, EHIP, ESTATE, ERANGE = 0, -1, -2, -3, -4, -5
ATTN_AUTO, ATTN_SPLIT, ATTN_WHOLE = 0, 1, 2
NEW_TOKEN_ZERO, NEW_TOKEN_MEAN = 0, 1
F32, BF16 = 0, 1
EMA, CUMULATIVE, LRFU_BLOCK, TIERED_INT2 = 0, 1, 2, 3
SCORE_VNORM, SCORE_ENTROPY = 1, 2
PER_KV_HEAD, PER_SEQUENCE = 0, 1
MAX_REGIONS = 8
_SCORER_BITS = {"attention": 0, "vnorm": SCORE_VNORM, "entropy": SCORE_ENTROPY,
                "vnorm+entropy": SCORE_VNORM | SCORE_ENTROPY}
_GRANULARITY = {"kv_head": PER_KV_HEAD, "sequence": PER_SEQUENCE}
_STATUS = {EINVAL: "EINVAL", ENOMEM: "ENOMEM", EHIP: "EHIP", ESTATE: "ESTATE", ERANGE: "ERANGE"}


class KvevError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"kvev {_STATUS.get(status, status)}: {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("max_tokens", ctypes.c_int64), ("page_tokens", ctypes.c_int32),
        ("policy", ctypes.c_int32), ("alpha_new", ctypes.c_float),
        ("refresh_interval", ctypes.c_int32), ("score_free", ctypes.c_int32),
        ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
        ("budget", ctypes.c_int64),
        ("beta", ctypes.c_float), ("region_half_life", ctypes.c_float * 8),
        ("pinned_region_mask", ctypes.c_uint32), ("decode_region", ctypes.c_int32),
        ("access_tau_mult", ctypes.c_float),
        ("window_tokens", ctypes.c_int32), ("fp_windows", ctypes.c_int32),
        ("int2_windows", ctypes.c_int32),
        ("scorer", ctypes.c_int32), ("granularity", ctypes.c_int32),
        ("route_interval", ctypes.c_int32),
        ("diag_topk", ctypes.c_int32),
        ("offload_blocks", ctypes.c_int32),
        ("revival_gap", ctypes.c_int32),
        ("prefetch_blocks", ctypes.c_int32),
        ("offload_min_score", ctypes.c_float),
        ("attn_path", ctypes.c_int32),
        ("evict_interval", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
        ("int2_key_groups", ctypes.c_int32),
        ("new_token_init", ctypes.c_int32),
    ]


class RouteDiag(ctypes.Structure):
    """kvev_route_diag: one layer's routing diagnostics."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "f_prev", "f_new", "f_overlap", "r_prev", "r_new", "r_overlap")] + [
        ("events", ctypes.c_int64), ("pairs", ctypes.c_int64), ("sustained", ctypes.c_int64),
        ("revived", ctypes.c_int64), ("sum_f_churn", ctypes.c_double), ("sum_r_churn", ctypes.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class DiagGroup(ctypes.Structure):
    """kvev_diag_group: one (sequence, KV head) group's rank-trace statistics."""
    _fields_ = [(name, ctypes.c_int32) for name in (
        "n", "k", "raw_overlap", "raw_prev", "util_overlap", "util_prev", "raw_util_overlap",
        "raw_top_evicted", "evicted", "retained", "retained_overlap", "retained_prev")] + [
        ("steps", ctypes.c_int64), ("pairs", ctypes.c_int64),
        ("sum_raw_churn", ctypes.c_double), ("sum_util_churn", ctypes.c_double),
        ("sum_raw_util_jaccard", ctypes.c_double), ("sum_raw_top_evicted", ctypes.c_double),
        ("sum_selection_churn", ctypes.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None

_SIGS = {
    "kvev_config_init": (None, [ctypes.POINTER(Config)]),
    "kvev_create": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]),
    "kvev_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "kvev_prefill": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_void_p]),
    "kvev_decode_step": (ctypes.c_int, [ctypes.c_void_p] * 5),
    "kvev_evict": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64]),
    "kvev_step": (ctypes.c_int, [ctypes.c_void_p] * 5 + [ctypes.c_int64]),
    "kvev_scores": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "kvev_retained": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "kvev_export_kv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "kvev_import_group": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "kvev_set_budget": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64]),
    "kvev_readmit": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]),
    "kvev_readmit_offloaded": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p]),
    "kvev_prefetch_offloaded": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p]),
    "kvev_offload_state": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.POINTER(ctypes.c_int64)]),
    "kvev_block_state": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "kvev_import_blocks": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_void_p]),
    "kvev_tier_state": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "kvev_tier_export": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]),
    "kvev_tier_ledger": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                         + [ctypes.c_void_p] * 6),
    "kvev_tier_import": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "kvev_tier_capacities": (ctypes.c_int, [ctypes.c_double] * 4 + [ctypes.POINTER(ctypes.c_int32)] * 2),
    "kvev_tier_footprint": (ctypes.c_int, [ctypes.c_void_p] + [ctypes.POINTER(ctypes.c_int64)] * 3
                            + [ctypes.POINTER(ctypes.c_int32)] * 2),
    "kvev_diag_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(DiagGroup), ctypes.c_int32]),
    "kvev_diag_trace": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.POINTER(ctypes.c_int64)]),
    "kvev_diag_fmm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]),
    "kvev_diag_fmm_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)]),
    "kvev_calibrate_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p]),
    "kvev_tier_diag": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(RouteDiag)]),
    "kvev_sync": (ctypes.c_int, [ctypes.c_void_p]),
    "kvev_step_index": (ctypes.c_int64, [ctypes.c_void_p]),
    "kvev_profile_enable": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "kvev_profile_reset": (ctypes.c_int, [ctypes.c_void_p]),
    "kvev_profile_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_int64)]),
    "kvev_last_error": (ctypes.c_char_p, [ctypes.c_void_p]),
}


def lib():
    """Load libkvev.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run decode_kv_cache_gqa_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def config_init():
    c = Config()
    lib().kvev_config_init(ctypes.byref(c))
    return c


def make_config(**kw):
    c = config_init()
    for k, v in kw.items():
        if not hasattr(c, k):
            raise KeyError(k)
        setattr(c, k, v)
    return c


def _ptr(t, dtype=None, shape=None, name="tensor", device=True):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


class Context:
    """One library context (cache, scores, page tables) on the current device."""

    def __init__(self, cfg: Config, stream=None):
        import torch
        self.cfg = cfg
        self._h = ctypes.c_void_p()
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        st = lib().kvev_create(ctypes.byref(cfg), ctypes.c_void_p(self.stream.cuda_stream),
                               ctypes.byref(self._h))
        if st != OK:
            raise KvevError(st, lib().kvev_last_error(None).decode())
        self.dtype = torch.float32 if cfg.dtype == F32 else torch.bfloat16

    # -- helpers ---------------------------------------------------------------
    def _check(self, st):
        if st != OK:
            raise KvevError(st, lib().kvev_last_error(self._h).decode())

    def close(self):
        if self._h:
            lib().kvev_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def step_index(self):
        return lib().kvev_step_index(self._h)

    # -- C ABI ---------------------------------------------------------------
    def prefill(self, seq, k, v, region_labels=None):
        c = self.cfg
        n = k.shape[2]
        shape = (c.n_layers, c.n_kv_heads, n, c.head_dim)
        lab = None
        if region_labels is not None:
            lab = np.ascontiguousarray(region_labels, dtype=np.uint8)
            if lab.shape != (n,):
                raise ValueError(f"region_labels has shape {lab.shape}, expected ({n},)")
        self._check(lib().kvev_prefill(self._h, seq, _ptr(k, self.dtype, shape, "k"),
                                       _ptr(v, self.dtype, shape, "v"), n,
                                       None if lab is None else lab.ctypes.data_as(ctypes.c_void_p)))

    def decode_step(self, q, k_new, v_new, out):
        import torch
        c = self.cfg
        qs = (c.n_layers, c.batch, c.n_q_heads, c.head_dim)
        ks = (c.n_layers, c.batch, c.n_kv_heads, c.head_dim)
        self._check(lib().kvev_decode_step(
            self._h, _ptr(q, self.dtype, qs, "q"), _ptr(k_new, self.dtype, ks, "k_new"),
            _ptr(v_new, self.dtype, ks, "v_new"), _ptr(out, torch.float32, qs, "out")))

    def step(self, q, k_new, v_new, out, budget=0):
        """decode_step + evict(budget) in one call (fused launches)."""
        import torch
        c = self.cfg
        qs = (c.n_layers, c.batch, c.n_q_heads, c.head_dim)
        ks = (c.n_layers, c.batch, c.n_kv_heads, c.head_dim)
        self._check(lib().kvev_step(
            self._h, _ptr(q, self.dtype, qs, "q"), _ptr(k_new, self.dtype, ks, "k_new"),
            _ptr(v_new, self.dtype, ks, "v_new"), _ptr(out, torch.float32, qs, "out"), int(budget)))

    def evict(self, budget=0):
        self._check(lib().kvev_evict(self._h, int(budget)))

    def scores(self, seq, kv_head):
        n = ctypes.c_int64()
        buf = np.zeros(self.cfg.max_tokens, np.float32)
        self._check(lib().kvev_scores(self._h, seq, kv_head, buf.ctypes.data_as(ctypes.c_void_p),
                                      buf.size, ctypes.byref(n)))
        return buf[: n.value].copy()

    def retained(self, seq, kv_head):
        n = ctypes.c_int64()
        buf = np.zeros(self.cfg.max_tokens, np.int32)
        self._check(lib().kvev_retained(self._h, seq, kv_head, buf.ctypes.data_as(ctypes.c_void_p),
                                        buf.size, ctypes.byref(n)))
        return buf[: n.value].copy()

    def export_kv(self, seq, kv_head):
        import torch
        c = self.cfg
        cap = c.max_tokens
        k = torch.empty((c.n_layers, cap, c.head_dim), dtype=self.dtype, device="cuda")
        v = torch.empty_like(k)
        n = ctypes.c_int64()
        self._check(lib().kvev_export_kv(self._h, seq, kv_head, _ptr(k), _ptr(v), cap, ctypes.byref(n)))
        self.sync()
        return k[:, : n.value].clone(), v[:, : n.value].clone()

    def import_group(self, seq, kv_head, positions, scores, k, v):
        c = self.cfg
        positions = np.ascontiguousarray(positions, dtype=np.int32)
        scores = np.ascontiguousarray(scores, dtype=np.float32)
        n = positions.shape[0]
        if scores.shape[0] != n:
            raise ValueError("positions and scores differ in length")
        shape = (c.n_layers, n, c.head_dim)
        self._check(lib().kvev_import_group(
            self._h, seq, kv_head, n, positions.ctypes.data_as(ctypes.c_void_p),
            scores.ctypes.data_as(ctypes.c_void_p), _ptr(k, self.dtype, shape, "k"),
            _ptr(v, self.dtype, shape, "v")))

    # -- block-granular mode ----------------------------------------------------
    def set_budget(self, seq, budget):
        self._check(lib().kvev_set_budget(self._h, seq, int(budget)))

    def readmit(self, seq, block_ids, k, v):
        """k, v: [L, Hkv, 16 * len(block_ids), d] holding the blocks' tokens."""
        c = self.cfg
        ids = np.ascontiguousarray(block_ids, dtype=np.int64)
        shape = (c.n_layers, c.n_kv_heads, 16 * ids.shape[0], c.head_dim)
        self._check(lib().kvev_readmit(self._h, seq, ids.shape[0], ids.ctypes.data_as(ctypes.c_void_p),
                                       _ptr(k, self.dtype, shape, "k"), _ptr(v, self.dtype, shape, "v")))

    def readmit_offloaded(self, seq, block_ids):
        """Re-admit evicted blocks of `seq` from the host-offload pool."""
        ids = np.ascontiguousarray(block_ids, dtype=np.int64)
        self._check(lib().kvev_readmit_offloaded(self._h, seq, ids.size, ids.ctypes.data_as(ctypes.c_void_p)))

    def prefetch_offloaded(self, seq, block_ids):
        """Start copying evicted blocks of `seq` from the host pool into device staging."""
        ids = np.ascontiguousarray(block_ids, dtype=np.int64)
        self._check(lib().kvev_prefetch_offloaded(self._h, seq, ids.size, ids.ctypes.data_as(ctypes.c_void_p)))

    def offload_state(self, seq):
        """Pool slot of every block `seq` has had (-1: not in the pool)."""
        n = ctypes.c_int64()
        buf = np.zeros(self.cfg.max_tokens // 16 + 2, np.int32)
        self._check(lib().kvev_offload_state(self._h, seq, buf.ctypes.data_as(ctypes.c_void_p), buf.size,
                                             ctypes.byref(n)))
        return buf[: n.value].copy()

    def block_state(self, seq):
        """(score float32, tref int32, resident bool) over every block seen."""
        cap = (self.cfg.max_tokens + 15) // 16
        sc = np.zeros(cap, np.float32)
        tr = np.zeros(cap, np.int32)
        rs = np.zeros(cap, np.uint8)
        n = ctypes.c_int64()
        self._check(lib().kvev_block_state(self._h, seq, sc.ctypes.data_as(ctypes.c_void_p),
                                           tr.ctypes.data_as(ctypes.c_void_p),
                                           rs.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(n)))
        m = n.value
        return sc[:m].copy(), tr[:m].copy(), rs[:m].astype(bool)

    def import_blocks(self, seq, score, tref, resident, k, v):
        c = self.cfg
        score = np.ascontiguousarray(score, dtype=np.float32)
        tref = np.ascontiguousarray(tref, dtype=np.int32)
        res = np.ascontiguousarray(resident, dtype=np.uint8)
        nb = score.shape[0]
        if tref.shape[0] != nb or res.shape[0] != nb:
            raise ValueError("score, tref and resident differ in length")
        n_tok = k.shape[2]
        shape = (c.n_layers, c.n_kv_heads, n_tok, c.head_dim)
        self._check(lib().kvev_import_blocks(
            self._h, seq, nb, score.ctypes.data_as(ctypes.c_void_p), tref.ctypes.data_as(ctypes.c_void_p),
            res.ctypes.data_as(ctypes.c_void_p), n_tok, _ptr(k, self.dtype, shape, "k"),
            _ptr(v, self.dtype, shape, "v")))

    # -- two-tier window mode -----------------------------------------------------
    def tier_state(self, layer):
        """(score float32, tier uint8 (0 FP, 1 INT2, 2 evicted), ledger bool) by window."""
        W = self.cfg.window_tokens
        cap = (self.cfg.max_tokens + W - 1) // W
        sc = np.zeros(cap, np.float32)
        tr = np.zeros(cap, np.uint8)
        lg = np.zeros(cap, np.uint8)
        n = ctypes.c_int64()
        self._check(lib().kvev_tier_state(self._h, layer, sc.ctypes.data_as(ctypes.c_void_p),
                                          tr.ctypes.data_as(ctypes.c_void_p),
                                          lg.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(n)))
        m = n.value
        return sc[:m].copy(), tr[:m].copy(), lg[:m].astype(bool)

    def tier_export(self, layer, kv_head):
        """Full-precision storage of (layer, KV head) by position: k, v [W * windows, d]."""
        import torch
        c = self.cfg
        W = c.window_tokens
        cap = ((c.max_tokens + W - 1) // W) * W
        k = torch.empty((cap, c.head_dim), dtype=self.dtype, device="cuda")
        v = torch.empty_like(k)
        n = ctypes.c_int64()
        self._check(lib().kvev_tier_export(self._h, layer, kv_head, _ptr(k), _ptr(v), cap, ctypes.byref(n)))
        self.sync()
        return k[: n.value].clone(), v[: n.value].clone()

    def tier_ledger(self, layer, kv_head, window):
        """INT2 record: (k_codes [W,128], k_scale [128], k_zero [128], v_codes [W,128],
        v_scale [W,4], v_zero [W,4]); parameters as float16.  With key groups
        the key parameters are [W,4] like the values'."""
        W = self.cfg.window_tokens
        kc = np.zeros((W, self.cfg.head_dim), np.uint8)
        vc = np.zeros_like(kc)
        kshape = (W, 4) if self.cfg.int2_key_groups else (128,)
        ks = np.zeros(128, np.uint16)  # the C call writes at most 128 parameters
        kz = np.zeros(128, np.uint16)
        vs = np.zeros((W, 4), np.uint16)
        vz = np.zeros((W, 4), np.uint16)
        args = [a.ctypes.data_as(ctypes.c_void_p) for a in (kc, ks, kz, vc, vs, vz)]
        self._check(lib().kvev_tier_ledger(self._h, layer, kv_head, window, *args))
        n = int(np.prod(kshape))
        ks, kz = ks[:n].reshape(kshape), kz[:n].reshape(kshape)
        return kc, ks.view(np.float16), kz.view(np.float16), vc, vs.view(np.float16), vz.view(np.float16)

    def tier_footprint(self):
        """Device bytes held for windows: dict with fp_pool, record_pool,
        staging (bytes) and fp_slots, record_slots (per layer and KV head)."""
        a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        f, r = ctypes.c_int32(), ctypes.c_int32()
        self._check(lib().kvev_tier_footprint(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                              ctypes.byref(f), ctypes.byref(r)))
        return {"fp_pool": a.value, "record_pool": b.value, "staging": c.value,
                "fp_slots": f.value, "record_slots": r.value}

    def tier_import(self, layer, score, tier):
        score = np.ascontiguousarray(score, dtype=np.float32)
        tier = np.ascontiguousarray(tier, dtype=np.uint8)
        if score.shape != tier.shape:
            raise ValueError("score and tier differ in length")
        self._check(lib().kvev_tier_import(self._h, layer, score.shape[0], score.ctypes.data_as(ctypes.c_void_p),
                                           tier.ctypes.data_as(ctypes.c_void_p)))

    def diag_read(self):
        """Rank-trace statistics of every group (g = seq * n_kv_heads + kv_head)."""
        G = self.cfg.batch * self.cfg.n_kv_heads
        arr = (DiagGroup * G)()
        self._check(lib().kvev_diag_read(self._h, arr, G))
        return [a.as_dict() for a in arr]

    def diag_trace(self, seq, kv_head):
        """The last step's (positions, raw, util) of group (seq, kv_head), slot order."""
        n = ctypes.c_int64()
        cap = self.cfg.max_tokens
        pos = np.zeros(cap, np.int32)
        raw = np.zeros(cap, np.float32)
        util = np.zeros(cap, np.float32)
        self._check(lib().kvev_diag_trace(
            self._h, seq, kv_head, pos.ctypes.data_as(ctypes.c_void_p), raw.ctypes.data_as(ctypes.c_void_p),
            util.ctypes.data_as(ctypes.c_void_p), cap, ctypes.byref(n)))
        m = n.value
        return pos[:m].copy(), raw[:m].copy(), util[:m].copy()

    def tier_diag(self, layer):
        """Routing diagnostics of `layer` (tiered mode, revival_gap > 0)."""
        d = RouteDiag()
        self._check(lib().kvev_tier_diag(self._h, layer, ctypes.byref(d)))
        return d.as_dict()

    def sync(self):
        self._check(lib().kvev_sync(self._h))

    def profile(self, enable=True):
        self._check(lib().kvev_profile_enable(self._h, 1 if enable else 0))

    def profile_reset(self):
        self._check(lib().kvev_profile_reset(self._h))

    def profile_read(self, kernel):
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        self._check(lib().kvev_profile_read(self._h, kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value


def diag_fmm(full, compressed):
    """Future missed mass of `compressed` against the never-evicting `full`
    context, per group (the library's kvev_diag_fmm)."""
    G = compressed.cfg.batch * compressed.cfg.n_kv_heads
    out = (ctypes.c_double * G)()
    compressed._check(lib().kvev_diag_fmm(full._h, compressed._h, out))
    return np.array(list(out), dtype=np.float64)


def diag_fmm_noalloc(full, compressed):
    """As diag_fmm, through the library's allocation-free entry point
    kvev_diag_fmm_noalloc (its staging buffer is a fixed device array)."""
    G = compressed.cfg.batch * compressed.cfg.n_kv_heads
    out = (ctypes.c_double * G)()
    compressed._check(lib().kvev_diag_fmm_noalloc(full._h, compressed._h, out))
    return np.array(list(out), dtype=np.float64)


def calibrate_read(buf, nontemporal, blocks, sink, stream=None):
    """kvev_calibrate_read: one streaming read of the device tensor `buf`
    (16-byte aligned, a multiple of 16 bytes) on `stream` (default: torch's
    current stream); `sink` is a device uint32/int32 tensor of >= blocks
    words."""
    import torch
    if not (buf.is_cuda and sink.is_cuda):
        raise ValueError("device tensors required")
    if sink.numel() * sink.element_size() < 4 * blocks:
        raise ValueError("sink too small")
    s = torch.cuda.current_stream() if stream is None else stream
    st = lib().kvev_calibrate_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                   1 if nontemporal else 0, blocks, ctypes.c_void_p(sink.data_ptr()),
                                   ctypes.c_void_p(s.cuda_stream))
    if st != 0:
        raise RuntimeError(f"kvev_calibrate_read failed with status {st}")


def tier_capacities(b_hist, q, m_f, m_q):
    """(K_f, K_q) of the two-tier mode from a byte budget (the library's
    kvev_tier_capacities; host arithmetic)."""
    kf, kq = ctypes.c_int32(), ctypes.c_int32()
    st = lib().kvev_tier_capacities(float(b_hist), float(q), float(m_f), float(m_q), ctypes.byref(kf),
                                    ctypes.byref(kq))
    if st != OK:
        raise KvevError(st, "invalid tier capacity arguments")
    return kf.value, kq.value


def context_for(w, max_steps=None, budget=None, stream=None, diag_topk=None, offload_blocks=None,
                revival_gap=None, prefetch_blocks=0, offload_min_score=0.0, attn_path=None):
    """A context configured for a synth.Workload (diag_topk: rank-trace
    diagnostics, default the workload's)."""
    steps = w.steps if max_steps is None else max_steps
    if w.policy == "lrfu_block":
        cfg = make_config(
            n_layers=w.n_layers, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
            head_dim=w.head_dim, batch=w.batch, dtype=F32 if w.dtype == "f32" else BF16,
            max_tokens=max(w.prefill_lens) + steps + 1, page_tokens=16, policy=LRFU_BLOCK,
            alpha_new=w.alpha_new, budget=max(w.block_budget(b) for b in range(w.batch))
            if budget is None else budget, beta=w.beta,
            pinned_region_mask=sum(1 << r for r in w.pinned_regions), decode_region=w.decode_region,
            access_tau_mult=2.0, offload_blocks=w.offload_blocks if offload_blocks is None else offload_blocks,
            prefetch_blocks=prefetch_blocks, offload_min_score=offload_min_score,
            attn_path=w.attn_path if attn_path is None else attn_path)
        for r, hl in enumerate(w.region_half_lives):
            cfg.region_half_life[r] = hl
        return Context(cfg, stream=stream)
    if w.policy == "tiered_int2":
        cfg = make_config(
            n_layers=w.n_layers, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
            head_dim=w.head_dim, batch=w.batch, dtype=F32 if w.dtype == "f32" else BF16,
            max_tokens=max(w.prefill_lens) + steps + 1, page_tokens=16, policy=TIERED_INT2,
            n_sink=w.n_sink, n_recent=w.n_recent, budget=1, window_tokens=w.window_tokens,
            fp_windows=w.fp_windows, int2_windows=w.int2_windows, route_interval=w.route_interval,
            revival_gap=w.revival_gap if revival_gap is None else revival_gap, rope_theta=w.rope_theta,
            int2_key_groups=w.int2_key_groups)
        return Context(cfg, stream=stream)
    cfg = make_config(
        n_layers=w.n_layers, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
        head_dim=w.head_dim, batch=w.batch, dtype=F32 if w.dtype == "f32" else BF16,
        max_tokens=max(w.prefill_lens) + steps + 1, page_tokens=16,
        policy=CUMULATIVE if w.policy == "cumulative" else EMA, alpha_new=w.alpha_new,
        refresh_interval=w.refresh_interval, score_free=1 if w.score_free else 0,
        n_sink=w.n_sink, n_recent=w.n_recent, budget=w.budget if budget is None else budget,
        scorer=_SCORER_BITS[w.scorer], granularity=_GRANULARITY[w.granularity],
        diag_topk=w.diag_topk if diag_topk is None else diag_topk,
        attn_path=w.attn_path if attn_path is None else attn_path, evict_interval=w.evict_interval,
        new_token_init=w.new_token_init)
    return Context(cfg, stream=stream)
