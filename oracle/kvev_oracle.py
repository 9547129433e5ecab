"""Plain, slow CPU oracle for one decode step of attention-scored KV eviction.

TEST INFRASTRUCTURE.  This module defines what the GPU library must compute.
Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import it; the GPU library never does, and this module imports nothing from
the library.  Floating point is fp64 except the INT2 quantizer, whose integer
codes are decided in IEEE fp32 exactly as the GPU decides them.

Sources (cited by short tag, with section / equation on that page):

* [InertiaKV]  "What Matters for Aggressive Decoding-Time KV Eviction?
  Temporal Aggregation and Ranking Preservation" (arXiv 2609.03515).
* [MemDecay]   "MemDecay: Region-Aware KV Cache Eviction for Efficient LLM
  Agent Inference" (arXiv 2607.10582).
* [QEvict]     "QEvict: Recoverable Quantized KV Eviction for
  Attention-Drift-Robust Long-Context Decoding", technical review.
* [LRFU-fig]   "Attention-Aware Block Eviction" figure page of the KV-cache
  docs (chapter 7, EMA eviction).

Conventions.  ``alpha_new`` is the weight on the new observation,
``score <- alpha_new*new + (1-alpha_new)*score`` ([LRFU-fig], table and
formula).  [InertiaKV] §3.1 Eq.4 puts its alpha on the old state; the two are
related by ``alpha_new = 1 - alpha_InertiaKV``.

Where the pages leave a step open, the reading taken is stated at the
function that implements it (and collected in the design notes).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "ema_update", "cumulative_update", "ema_half_life", "recency_decay",
    "lrfu_priority", "layer_fold", "layer_fold_weights", "decode_attention",
    "group_mass", "select_keep", "hole_fill_moves", "apply_moves",
    "tier_capacities", "route_tiers", "int2_quantize", "int2_dequantize",
    "TokenModeOracle", "region_decay_rates", "block_survival", "block_priority",
    "select_blocks", "BlockLRFUOracle", "bf16_round", "TieredOracle",
    "vnorm_weights", "normalized_entropy", "scored_mass", "SCORERS",
    "PooledTokenOracle", "jaccard", "top_k_positions", "RankTraceDiagnostics",
    "future_missed_mass", "HostOffloadPool", "RoutingDiagnostics", "rope",
]


# ---------------------------------------------------------------------------
# Score aggregation primitives
# ---------------------------------------------------------------------------

def ema_update(score, new, alpha_new):
    """EMA step ``score <- alpha_new*new + (1-alpha_new)*score``.

    [LRFU-fig] smoothing formula and worked table; [InertiaKV] §3.1 Eq.4
    (with its alpha equal to ``1 - alpha_new``); [MemDecay] §III-C Eq.2
    (with rho equal to ``1 - alpha_new``).  Written with plain operators so
    it also runs on ``decimal.Decimal`` inputs.
    """
    return alpha_new * new + (1 - alpha_new) * score


def cumulative_update(score, new):
    """Non-decaying accumulator ``m_t = m_{t-1} + s_t``.

    [InertiaKV] §3.1 Eq.3; [QEvict] §4.2 Eq.1 (per window, per layer).
    """
    return score + new


def ema_half_life(alpha_new):
    """Steps for the EMA weight of an observation to halve: ln0.5/ln(1-a).

    [LRFU-fig]: at alpha 0.05 the page gives ln0.5/ln0.95 = 13.5 steps.
    """
    return math.log(0.5) / math.log(1.0 - alpha_new)


def recency_decay(idle, beta):
    """``1 - exp(-beta*idle)``: the idle-time factor of [LRFU-fig]."""
    return 1.0 - np.exp(-beta * np.asarray(idle, dtype=np.float64))


def lrfu_priority(score, idle, beta):
    """Eviction priority ``(1 - score) * (1 - exp(-beta*idle))``.

    [LRFU-fig]: the block with the HIGHER priority is evicted (block B in the
    page's example).
    """
    return (1.0 - np.asarray(score, dtype=np.float64)) * recency_decay(idle, beta)


def region_decay_rates(half_lives):
    """Decay rate per region from its half-life, ``lambda = ln2 / t_half``.

    [MemDecay] §IV-B Eq.7 (``t_half = ln2 / lambda``).
    """
    return np.array([math.log(2.0) / h for h in half_lives], dtype=np.float64)


def layer_fold(m, G_layers, alpha_new, policy="ema"):
    """Fold per-layer group mass into the shared state, layer by layer.

    [InertiaKV] App. E "Layer scoring": each eligible layer immediately
    updates the shared state, ``m_{t,l} = a m_{t,l-1} + (1-a) s_{t,l}`` with
    ``m_{t,0} = m_{t-1,K}``.  Reading: all layers are eligible, in ascending
    order.  ``policy="cumulative"`` applies [InertiaKV] Eq.3 per layer.
    """
    m = np.array(m, dtype=np.float64, copy=True)
    for G in G_layers:
        if policy == "ema":
            m = ema_update(m, np.asarray(G, dtype=np.float64), alpha_new)
        elif policy == "cumulative":
            m = cumulative_update(m, np.asarray(G, dtype=np.float64))
        else:
            raise ValueError(policy)
    return m


def layer_fold_weights(alpha_new, n_layers):
    """Closed-form weights of the layer-sequential EMA.

    [InertiaKV] App. E: the prior state has weight ``alpha^K`` and layer l
    (1-based) has weight ``(1-alpha) alpha^{K-l}`` (alpha on the old state).
    Returned as (prior_weight, [w_0 .. w_{L-1}]) with 0-based layers.
    """
    keep = 1.0 - alpha_new
    prior = keep ** n_layers
    w = [alpha_new * keep ** (n_layers - 1 - l) for l in range(n_layers)]
    return prior, w


# ---------------------------------------------------------------------------
# Attention with exposed probabilities
# ---------------------------------------------------------------------------

def decode_attention(q, K, V):
    """Scaled dot-product decode attention that also returns probabilities.

    [QEvict] §4.1 (Attention): ``a = softmax(q K^T / sqrt(d))``, ``o = a V``.
    ``q``: [H, d] (the query heads of one KV head's group), ``K``, ``V``:
    [n, d].  Returns ``(out [H, d], p [H, n], logits [H, n])`` in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d = q.shape[-1]
    s = (q @ K.T) / math.sqrt(d)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ V, p, s


def group_mass(p):
    """Per-token attention mass summed over a KV head's query group.

    [InertiaKV] §3.1 Eq.1 pools over heads; App. E: for GQA each KV head's
    attention is shared across its query-head group before pooling.
    Reading: one score per (sequence, KV head) token, equal to the SUM of the
    group's probabilities (the mean times the group size; a uniform positive
    scale, invisible to ranking per [InertiaKV] Corollary 2).
    """
    return np.asarray(p, dtype=np.float64).sum(axis=0)


def vnorm_weights(V):
    """Mean-normalised l2 norms of the value states of the cached tokens.

    [InertiaKV] §5.1 and App. E: VNorm multiplies each head's
    attention on token i by ||v_i|| divided by the mean of ||v_j|| over the
    tokens the head attends to.  ``V``: [n, d] of one KV head at one layer.
    Reading: when every value row is zero the weights are 1 (the scorer
    falls back to plain attention) instead of 0/0.
    """
    V = np.asarray(V, dtype=np.float64)
    norms = np.sqrt((V * V).sum(axis=1))
    mean = norms.mean()
    if mean == 0.0:
        return np.ones_like(norms)
    return norms / mean


def normalized_entropy(p):
    """Shannon entropy of each head's attention row, divided by ln(n).

    [InertiaKV] §5.1 and App. E: entropy weighting multiplies a layer's
    contribution by the normalised entropy of its attention distribution.
    ``p``: [H, n].  Returns [H] in [0, 1]; 0 log 0 = 0.  Reading: with a
    single token (ln 1 = 0) the weight is 1.
    """
    p = np.asarray(p, dtype=np.float64)
    n = p.shape[1]
    if n < 2:
        return np.ones(p.shape[0])
    t = np.zeros_like(p)
    nz = p > 0
    t[nz] = -p[nz] * np.log(p[nz])
    return t.sum(axis=1) / math.log(n)


SCORERS = ("attention", "vnorm", "entropy", "vnorm+entropy")


def scored_mass(p, V, scorer="attention"):
    """Per-token observation of one layer for a state fed by the heads ``p``.

    ``p``: [H, n] probabilities of the heads pooled into the state (one KV
    head's query group), ``V``: [n, d] that KV head's value states.

    * "attention": the group sum of probabilities (``group_mass``);
    * "vnorm": each head's probability times ``vnorm_weights(V)`` before the
      group sum;
    * "entropy": the group sum times one per-layer scalar, the mean over the
      pooled heads of ``normalized_entropy`` (reading: the page names one
      scalar per layer and does not say how heads combine; the mean keeps it
      in [0, 1]);
    * "vnorm+entropy": both factors.
    Both modifications act on the step's observation, before the temporal
    fold ([InertiaKV] §5.1).
    """
    if scorer not in SCORERS:
        raise ValueError(scorer)
    p = np.asarray(p, dtype=np.float64)
    if "vnorm" in scorer:
        G = (p * vnorm_weights(V)[None, :]).sum(axis=0)
    else:
        G = group_mass(p)
    if "entropy" in scorer:
        G = G * normalized_entropy(p).mean()
    return G


# ---------------------------------------------------------------------------
# Selection and compaction
# ---------------------------------------------------------------------------

def select_keep(scores, positions, budget, n_sink=0, n_recent=0):
    """Keep mask: protected tokens plus the top-(budget - |protected|) rest.

    [InertiaKV] §3.1: whenever the cache exceeds B, evict the tokens with the
    lowest utility.  [MemDecay] §III-A Eq.1: with a forced set F, keeping the
    highest-scoring tokens after forcing F is optimal.

    Readings: the protected set is the sinks (positions < n_sink) and the
    n_recent largest positions present (the new token included).  Ranking
    key is (score, position), larger is kept, so on an exact score tie the
    more recent token stays.  No eviction when ``len(scores) <= budget``.
    """
    scores = np.asarray(scores, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    n = scores.shape[0]
    keep = np.ones(n, dtype=bool)
    if n <= budget:
        return keep
    newest = positions.max()
    prot = (positions < n_sink) | (positions > newest - n_recent)
    room = budget - int(prot.sum())
    if room < 0:
        raise ValueError("protected tokens exceed the budget")
    cand = np.flatnonzero(~prot)
    # ascending by (score, position); the last `room` are kept
    order = cand[np.lexsort((positions[cand], scores[cand]))]
    keep[:] = prot
    if room > 0:
        keep[order[len(order) - room:]] = True
    return keep


def hole_fill_moves(keep, budget):
    """Compaction plan that packs the survivors into slots [0, budget).

    Reading (the pages fix no layout): holes are the unkept slots below the
    budget, ascending; movers are the kept slots at or above it, ascending;
    mover j fills hole j.  Returns a list of (src_slot, dst_slot).
    """
    keep = np.asarray(keep, dtype=bool)
    n = keep.shape[0]
    if n <= budget:
        return []
    holes = [s for s in range(budget) if not keep[s]]
    movers = [s for s in range(budget, n) if keep[s]]
    if len(holes) != len(movers):
        raise ValueError("keep mask does not hold exactly `budget` slots")
    return list(zip(movers, holes))


def apply_moves(arr, moves, axis=0):
    """Copy slot ``src`` onto slot ``dst`` for every move, along ``axis``."""
    arr = np.moveaxis(arr, axis, 0)
    for src, dst in moves:
        arr[dst] = arr[src]
    return np.moveaxis(arr, 0, axis)


# ---------------------------------------------------------------------------
# Tiered (full precision / INT2 / evicted) routing primitives
# ---------------------------------------------------------------------------

def tier_capacities(b_hist, q, m_f, m_q):
    """Tier sizes ``K_f = floor((1-q)B_hist/M_f)``, ``K_q = floor(q B_hist/M_q)``.

    [QEvict] §4.3 Eq.3.
    """
    return int(math.floor((1.0 - q) * b_hist / m_f)), int(math.floor(q * b_hist / m_q))


def route_tiers(scores, candidates, k_f, k_q):
    """One routing event: F = top K_f, Q = next K_q, E = the rest.

    [QEvict] §4.4 Eq.5 and Algorithm 1 (sort candidates by cumulative score,
    fill the full-precision tier, then the quantized tier).  Reading: equal
    scores rank the higher window index first.  Returns three sorted lists.
    """
    cand = np.asarray(sorted(candidates), dtype=np.int64)
    s = np.asarray(scores, dtype=np.float64)[cand]
    order = cand[np.lexsort((cand, s))][::-1]          # descending
    F = sorted(order[:k_f].tolist())
    Q = sorted(order[k_f:k_f + k_q].tolist())
    E = sorted(order[k_f + k_q:].tolist())
    return F, Q, E


def _int2_params(x32, axis):
    """Asymmetric min-max parameters of each group, stored as fp16.

    Reading of [QEvict] §4.4, Algorithm 1 (asymmetric, KIVI-style): zero = min,
    scale = (max - min) / 3, both rounded to fp16 (round to nearest even);
    the subtraction and division are single IEEE fp32 operations.  The
    groups run along ``axis`` of the fp32 array ``x32``.
    """
    lo = x32.min(axis=axis, keepdims=True).astype(np.float32)
    hi = x32.max(axis=axis, keepdims=True).astype(np.float32)
    span = (hi - lo).astype(np.float32)
    scale = (span / np.float32(3.0)).astype(np.float32).astype(np.float16)
    zero = lo.astype(np.float16)
    return scale, zero


def _int2_codes(x32, scale16, zero16):
    """Codes ``clamp(rint((x - zero)/scale), 0, 3)`` in IEEE fp32; a group
    whose scale is 0 (all values equal) takes code 0."""
    s = np.broadcast_to(scale16.astype(np.float32), x32.shape)
    z = zero16.astype(np.float32)
    t = (x32 - z).astype(np.float32)                          # fp32 subtract
    flat = s == np.float32(0.0)
    t = (t / np.where(flat, np.float32(1.0), s)).astype(np.float32)  # fp32 divide
    codes = np.clip(np.rint(t), 0, 3).astype(np.uint8)         # ties to even
    codes[flat] = 0
    return codes


def int2_quantize(x, axis_groups):
    """Quantize a [tokens, channels] fp32 tile to 2-bit codes.

    ``axis_groups="channel"``: one (scale, zero) per channel over all tokens
    of the tile (keys, [QEvict] §4.4 Algorithm 1: keys per channel).
    ``axis_groups="token32"``: one (scale, zero) per token per 32-channel
    group (values, "per-token-value"; the 32-channel grouping is the
    workload's stated group size).
    Returns (codes uint8 [T, C], scales fp16, zeros fp16): scales and zeros
    are [C] in channel mode and [T, C/32] in token32 mode.
    """
    x = np.asarray(x, dtype=np.float32)
    T, C = x.shape
    if axis_groups == "channel":
        s, z = _int2_params(x, axis=0)                 # [1, C]
        codes = _int2_codes(x, s, z)
        return codes, s[0], z[0]
    if axis_groups == "token32":
        ng = C // 32
        xg = x.reshape(T, ng, 32)
        s, z = _int2_params(xg, axis=2)                # [T, ng, 1]
        codes = _int2_codes(xg, s, z).reshape(T, C)
        return codes, s[..., 0], z[..., 0]
    raise ValueError(axis_groups)


def int2_dequantize(codes, scales, zeros, axis_groups):
    """``x_hat = code*scale + zero`` as a separate fp32 multiply and add."""
    codes = np.asarray(codes).astype(np.float32)
    T, C = codes.shape
    if axis_groups == "channel":
        s = np.asarray(scales, dtype=np.float32)[None, :]
        z = np.asarray(zeros, dtype=np.float32)[None, :]
    elif axis_groups == "token32":
        s = np.repeat(np.asarray(scales, dtype=np.float32), 32, axis=1)
        z = np.repeat(np.asarray(zeros, dtype=np.float32), 32, axis=1)
    else:
        raise ValueError(axis_groups)
    prod = (codes * s).astype(np.float32)
    return (prod + z).astype(np.float32)


def rope(x, positions, theta):
    """Rotary position embedding of the rows of ``x`` [n, d] at their
    absolute ``positions`` [n], in fp64.

    [QEvict] §4.4, "Positional handling for promoted keys": keys are
    quantized before the rotation, with their original absolute positions,
    and the rotation is applied again at those positions when a window is
    promoted.  Reading (the pages give no formula): the rotary embedding of
    the named Llama shape, which turns channel pair (i, i + d/2) by the
    angle ``position * theta**(-2i/d)``, i < d/2.
    """
    x = np.asarray(x, dtype=np.float64)
    n, d = x.shape
    h = d // 2
    freq = float(theta) ** (-2.0 * np.arange(h, dtype=np.float64) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * freq[None, :]
    c, sn = np.cos(ang), np.sin(ang)
    a, b = x[:, :h], x[:, h:]
    return np.concatenate([a * c - b * sn, b * c + a * sn], axis=1)


# ---------------------------------------------------------------------------
# Token-granular eviction step (InertiaKV, InertiaKV-Lazy, Score-Free)
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# Rank-trace diagnostics
# ---------------------------------------------------------------------------

def jaccard(a, b):
    """Jaccard index |a & b| / |a | b| of two sets of positions.

    [InertiaKV] App. I (raw / EMA Jaccard overlap, churn as its complement)
    and [QEvict] §3 (selection churn, the Jaccard distance).  Reading: two
    empty sets have index 1.
    """
    a, b = set(a), set(b)
    u = len(a | b)
    return 1.0 if u == 0 else len(a & b) / u


def top_k_positions(values, positions, k):
    """The positions of the k largest (value, position) keys.

    [InertiaKV] App. I traces top-k token sets by score.  Reading: the order
    is the selection's (``select_keep``): on equal values the larger
    (more recent) position ranks higher; k larger than the token count takes
    every token.
    """
    values = np.asarray(values, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    k = min(int(k), values.shape[0])
    if k <= 0:
        return set()
    order = np.lexsort((positions, values))  # ascending by (value, position)
    return set(positions[order[values.shape[0] - k:]].tolist())


class RankTraceDiagnostics:
    """Per-step rank-trace statistics of one selection group.

    [InertiaKV] App. I, Table 13: raw top-k churn, EMA (utility) top-k churn,
    the raw / EMA Jaccard overlap and the share of the raw top-k that is
    evicted; [QEvict] §3: selection churn, the Jaccard distance between the
    retained sets of consecutive selections.  Churn is one minus the Jaccard
    index against the previous observed step.

    Feed ``observe`` once per step, after the fold and before the eviction
    takes effect, with the step's tokens (positions), their raw observation
    and their utility, and the positions kept after the eviction.

    Readings: the raw score of a step is its observation summed over the
    layers (one raw value per token; the sum ranks like the mean); k is the
    caller's (App. I measures at k = the budget); the evicted set of a step
    is the step's tokens that are not kept.
    """

    COUNTS = ("n", "k", "raw_overlap", "raw_prev", "util_overlap", "util_prev",
              "raw_util_overlap", "raw_top_evicted", "evicted", "retained",
              "retained_overlap", "retained_prev")

    def __init__(self, k):
        self.k = int(k)
        self.prev = None  # (R, E, S) of the previous step
        self.step = 0
        self.evicted_at = {}  # position -> step that evicted it
        self.sums = {"steps": 0, "pairs": 0, "sum_raw_churn": 0.0, "sum_util_churn": 0.0,
                     "sum_raw_util_jaccard": 0.0, "sum_raw_top_evicted": 0.0,
                     "sum_selection_churn": 0.0}

    def observe(self, positions, raw, util, kept_positions):
        positions = np.asarray(positions, dtype=np.int64)
        self.step += 1
        R = top_k_positions(raw, positions, self.k)
        E = top_k_positions(util, positions, self.k)
        S = set(np.asarray(kept_positions, dtype=np.int64).tolist())
        Ev = set(positions.tolist()) - S
        for p in Ev:
            self.evicted_at[p] = self.step
        k = len(R)
        c = {"n": int(positions.shape[0]), "k": k, "raw_util_overlap": len(R & E),
             "raw_top_evicted": len(R & Ev), "evicted": len(Ev), "retained": len(S)}
        sm = self.sums
        sm["steps"] += 1
        sm["sum_raw_util_jaccard"] += jaccard(R, E)
        sm["sum_raw_top_evicted"] += len(R & Ev) / k
        if self.prev is None:
            c.update(raw_overlap=0, raw_prev=0, util_overlap=0, util_prev=0, retained_overlap=0,
                     retained_prev=0)
        else:
            Rp, Ep, Sp = self.prev
            c.update(raw_overlap=len(R & Rp), raw_prev=len(Rp), util_overlap=len(E & Ep),
                     util_prev=len(Ep), retained_overlap=len(S & Sp), retained_prev=len(Sp))
            sm["pairs"] += 1
            sm["sum_raw_churn"] += 1.0 - jaccard(R, Rp)
            sm["sum_util_churn"] += 1.0 - jaccard(E, Ep)
            sm["sum_selection_churn"] += 1.0 - jaccard(S, Sp)
        self.prev = (R, E, S)
        return c

    def evicted_before(self, step):
        """Positions evicted at a step earlier than ``step`` (1-based)."""
        return {p for p, e in self.evicted_at.items() if e < step}


def future_missed_mass(full_positions, full_raw, evicted):
    """Share of a full cache's attention mass on evicted positions.

    [QEvict] §3 (Future Missed Mass): the uncompressed model's attention
    distribution over its whole cache at a step, and the fraction of it that
    lands on tokens the compressed policy has already discarded.  Reading:
    the distribution of a (sequence, KV head) group is its observation
    summed over the layers and the group's query heads (a uniform scale of
    L * group size, which the ratio removes); ``evicted`` holds the
    positions discarded at earlier steps.
    """
    w = np.asarray(full_raw, dtype=np.float64)
    mask = np.isin(np.asarray(full_positions, dtype=np.int64), np.fromiter(evicted, dtype=np.int64))
    tot = w.sum()
    return float(w[mask].sum() / tot) if tot > 0 else 0.0


@dataclass
class _Group:
    """State of one (sequence, KV head) selection group, in slot order."""
    K: np.ndarray          # [L, cap, d] float64 (exact widenings of the inputs)
    V: np.ndarray          # [L, cap, d]
    pos: np.ndarray        # [cap] int64
    m: np.ndarray          # [cap] float64 utility
    n: int = 0


@dataclass
class TokenModeOracle:
    """Per-(sequence, KV head) utility, selection and compaction.

    One object holds any subset of a batch's sequences (sequences are
    independent), so large batches can be checked on a sample.

    * ``policy``: "ema" ([InertiaKV] Eq.4, layer-sequential per App. E) or
      "cumulative" ([InertiaKV] Eq.3).
    * ``refresh_interval`` r: scores are observed at t in R_r =
      {t >= 1 : (t-1) mod r == 0} ([InertiaKV] §3.2 Eq.6); r = 1 is full
      refresh.
    * ``score_free``: observe only at t = 1, then freeze ([InertiaKV] §3.2
      "Score-Free decoding").
    * New tokens: on a non-refresh step the new token starts at the mean of
      the existing utilities ([InertiaKV] App. E); on a refresh step it
      starts at 0, like the prefill tokens (m_0 = 0, App. E), and is then
      folded with its own attention mass (reading: the page states only the
      non-refresh rule).  ``new_token_init`` = "mean" applies the stated
      rule on refresh steps too: the mean, then the fold.
    * Eviction happens once per step after all layers, whenever the group
      holds more than ``budget`` tokens, including non-refresh steps with
      the stale utility ([InertiaKV] App. E "Eviction on non-refresh steps").
      ``evict_interval`` e > 1 takes the batched workload's wording "recompute
      scores and evict every 8 steps" literally: the caller selects only on
      the steps ``is_evict_step`` names, t in {1, 1 + e, 1 + 2e, ...}, and
      the cache grows by one token per step in between.
    * ``scorer``: the observation folded per layer, see ``scored_mass``.
    """
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    budget: int
    alpha_new: float
    policy: str = "ema"
    refresh_interval: int = 1
    score_free: bool = False
    n_sink: int = 0
    n_recent: int = 0
    capacity: int = 0
    scorer: str = "attention"
    evict_interval: int = 1
    new_token_init: str = "zero"
    groups: dict = field(default_factory=dict)
    prefill_len: dict = field(default_factory=dict)
    last_G: dict = field(default_factory=dict)

    @property
    def group_size(self):
        return self.n_q_heads // self.n_kv_heads

    def prefill(self, seq, K, V, heads=None):
        """Store a sequence's prefill cache, positions 0..n-1, utility 0.

        ``K``, ``V``: [L, len(heads), n, d] (``heads`` defaults to every KV
        head; holding a subset checks a sample of independent groups).
        [InertiaKV] App. E: m_0(i) = 0 for every prefill position;
        compression acts only during decoding.
        """
        K = np.asarray(K, dtype=np.float32)
        V = np.asarray(V, dtype=np.float32)
        L, nh, n, d = K.shape
        heads = list(range(nh)) if heads is None else list(heads)
        cap = max(self.capacity, n + 1)
        for j, h in enumerate(heads):
            g = _Group(K=np.zeros((L, cap, d), np.float64),
                       V=np.zeros((L, cap, d), np.float64),
                       pos=np.zeros(cap, np.int64), m=np.zeros(cap, np.float64))
            g.K[:, :n] = K[:, j]
            g.V[:, :n] = V[:, j]
            g.pos[:n] = np.arange(n)
            g.n = n
            self.groups[(seq, h)] = g
        self.prefill_len[seq] = n

    def is_refresh(self, t):
        if self.score_free:
            return t == 1
        return (t - 1) % self.refresh_interval == 0

    def _starts_at_mean(self, refresh):
        if self.new_token_init not in ("zero", "mean"):
            raise ValueError(self.new_token_init)
        return not refresh or self.new_token_init == "mean"

    def is_evict_step(self, t):
        """Whether step t selects (every step unless evict_interval > 1)."""
        return (t - 1) % max(self.evict_interval, 1) == 0

    def _grow(self, g):
        if g.n < g.K.shape[1]:
            return
        extra = max(64, g.K.shape[1] // 4)
        pad = lambda a, fill=0: np.concatenate(
            [a, np.full((a.shape[0], extra) + a.shape[2:], fill, a.dtype)], axis=1)
        g.K, g.V = pad(g.K), pad(g.V)
        g.pos = np.concatenate([g.pos, np.zeros(extra, np.int64)])
        g.m = np.concatenate([g.m, np.zeros(extra, np.float64)])

    def held_heads(self, seq):
        return sorted(h for (s, h) in self.groups if s == seq)

    def decode_step(self, t, q, k_new, v_new, seqs):
        """Append, attend every layer, fold (on refresh steps).

        ``q``: [L, len(seqs), Hq, d]; ``k_new``, ``v_new``: [L, len(seqs),
        Hkv, d]; ``seqs`` lists the sequence ids in that batch order.
        Returns ``out`` [L, len(seqs), Hq, d] in fp64 (zero for the query
        heads of KV heads this oracle does not hold).
        """
        q = np.asarray(q, dtype=np.float32)
        k_new = np.asarray(k_new, dtype=np.float32)
        v_new = np.asarray(v_new, dtype=np.float32)
        refresh = self.is_refresh(t)
        Hg = self.group_size
        for bi, seq in enumerate(seqs):
            for h in self.held_heads(seq):
                g = self.groups[(seq, h)]
                init = float(g.m[:g.n].mean()) if self._starts_at_mean(refresh) else 0.0
                self._grow(g)
                g.K[:, g.n] = k_new[:, bi, h]
                g.V[:, g.n] = v_new[:, bi, h]
                g.pos[g.n] = self.prefill_len[seq] + t - 1
                g.m[g.n] = init
                g.n += 1
        out = np.zeros((self.n_layers, len(seqs), self.n_q_heads, self.head_dim))
        self.last_G = {}
        for l in range(self.n_layers):
            for bi, seq in enumerate(seqs):
                for h in self.held_heads(seq):
                    g = self.groups[(seq, h)]
                    o, p, _ = decode_attention(q[l, bi, h * Hg:(h + 1) * Hg],
                                               g.K[l, :g.n], g.V[l, :g.n])
                    out[l, bi, h * Hg:(h + 1) * Hg] = o
                    if refresh:
                        G = scored_mass(p, g.V[l, :g.n], self.scorer)
                        self.last_G[(l, seq, h)] = G
                        g.m[:g.n] = layer_fold(g.m[:g.n], [G], self.alpha_new,
                                               self.policy)
        return out

    def evict(self, budget=None):
        """Select and compact every group that exceeds the budget."""
        B = self.budget if budget is None else budget
        for g in self.groups.values():
            if g.n <= B:
                continue
            keep = select_keep(g.m[:g.n], g.pos[:g.n], B, self.n_sink, self.n_recent)
            moves = hole_fill_moves(keep, B)
            for src, dst in moves:
                g.K[:, dst] = g.K[:, src]
                g.V[:, dst] = g.V[:, src]
                g.pos[dst] = g.pos[src]
                g.m[dst] = g.m[src]
            g.n = B

    # -- views used by tests ------------------------------------------------
    def step_observation(self, seq, h):
        """After an observation step's ``decode_step`` and before ``evict``:
        the group's (positions, raw, utility) in slot order, raw being the
        step's observation summed over the layers (``RankTraceDiagnostics``)."""
        g = self.groups[(seq, h)]
        raw = np.zeros(g.n, dtype=np.float64)
        for l in range(self.n_layers):
            raw += self.last_G[(l, seq, h)]
        return g.pos[:g.n].copy(), raw, g.m[:g.n].copy()

    def scores(self, seq, h):
        g = self.groups[(seq, h)]
        return g.m[:g.n].copy()

    def positions(self, seq, h):
        g = self.groups[(seq, h)]
        return g.pos[:g.n].copy()


class _SeqState:
    """State of one sequence in the pooled mode, in slot order."""

    def __init__(self, L, Hkv, cap, d):
        self.K = np.zeros((L, Hkv, cap, d), np.float64)
        self.V = np.zeros((L, Hkv, cap, d), np.float64)
        self.pos = np.zeros(cap, np.int64)
        self.m = np.zeros(cap, np.float64)
        self.n = 0


@dataclass
class PooledTokenOracle:
    """One utility per (sequence, position), pooled over every query head.

    [InertiaKV] §3.1 Eq.1: the step's score of token i is the mean over all
    H attention heads of their probability on i; App. E: for GQA each KV
    head's attention serves its query-head group before the pooling.  One
    retained set per sequence: every KV head at every layer holds the same
    positions, in the same slots, so selection and compaction act on all of
    them together.  Aggregation, refresh cadence, new-token rule, protection
    and eviction are those of ``TokenModeOracle`` (``new_token_init`` too).

    Scorers ([InertiaKV] §5.1, App. E): "vnorm" weights each head's
    probabilities by the VNorm weights of its own KV head's values before the
    mean; "entropy" multiplies the layer's pooled score by the mean over all
    H heads of their normalised entropy.
    """
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    budget: int
    alpha_new: float
    policy: str = "ema"
    refresh_interval: int = 1
    score_free: bool = False
    n_sink: int = 0
    n_recent: int = 0
    capacity: int = 0
    scorer: str = "attention"
    new_token_init: str = "zero"
    seqs: dict = field(default_factory=dict)
    prefill_len: dict = field(default_factory=dict)
    last_G: dict = field(default_factory=dict)

    @property
    def group_size(self):
        return self.n_q_heads // self.n_kv_heads

    def prefill(self, seq, K, V):
        """``K``, ``V``: [L, Hkv, n, d]; positions 0..n-1, utility 0."""
        K = np.asarray(K, dtype=np.float32)
        V = np.asarray(V, dtype=np.float32)
        L, Hkv, n, d = K.shape
        st = _SeqState(L, Hkv, max(self.capacity, n + 1), d)
        st.K[:, :, :n] = K
        st.V[:, :, :n] = V
        st.pos[:n] = np.arange(n)
        st.n = n
        self.seqs[seq] = st
        self.prefill_len[seq] = n

    def is_refresh(self, t):
        if self.score_free:
            return t == 1
        return (t - 1) % self.refresh_interval == 0

    _starts_at_mean = TokenModeOracle._starts_at_mean

    def _grow(self, st):
        if st.n < st.K.shape[2]:
            return
        extra = max(64, st.K.shape[2] // 4)
        pad = lambda a: np.concatenate(
            [a, np.zeros(a.shape[:2] + (extra,) + a.shape[3:], a.dtype)], axis=2)
        st.K, st.V = pad(st.K), pad(st.V)
        st.pos = np.concatenate([st.pos, np.zeros(extra, np.int64)])
        st.m = np.concatenate([st.m, np.zeros(extra, np.float64)])

    def decode_step(self, t, q, k_new, v_new, seqs):
        """Same arguments and result as ``TokenModeOracle.decode_step``."""
        if self.scorer not in SCORERS:
            raise ValueError(self.scorer)
        q = np.asarray(q, dtype=np.float32)
        k_new = np.asarray(k_new, dtype=np.float32)
        v_new = np.asarray(v_new, dtype=np.float32)
        refresh = self.is_refresh(t)
        Hg, H = self.group_size, self.n_q_heads
        for bi, seq in enumerate(seqs):
            st = self.seqs[seq]
            init = float(st.m[:st.n].mean()) if self._starts_at_mean(refresh) else 0.0
            self._grow(st)
            st.K[:, :, st.n] = k_new[:, bi]
            st.V[:, :, st.n] = v_new[:, bi]
            st.pos[st.n] = self.prefill_len[seq] + t - 1
            st.m[st.n] = init
            st.n += 1
        out = np.zeros((self.n_layers, len(seqs), H, self.head_dim))
        self.last_G = {}
        for l in range(self.n_layers):
            for bi, seq in enumerate(seqs):
                st = self.seqs[seq]
                n = st.n
                pooled = np.zeros(n)
                ent = []
                for h in range(self.n_kv_heads):
                    Vh = st.V[l, h, :n]
                    o, p, _ = decode_attention(q[l, bi, h * Hg:(h + 1) * Hg], st.K[l, h, :n], Vh)
                    out[l, bi, h * Hg:(h + 1) * Hg] = o
                    if "vnorm" in self.scorer:
                        pooled += (p * vnorm_weights(Vh)[None, :]).sum(axis=0)
                    else:
                        pooled += p.sum(axis=0)
                    ent.extend(normalized_entropy(p).tolist())
                G = pooled / H
                if "entropy" in self.scorer:
                    G = G * float(np.mean(ent))
                if refresh:
                    self.last_G[(l, seq)] = G
                    st.m[:n] = layer_fold(st.m[:n], [G], self.alpha_new, self.policy)
        return out

    def evict(self, budget=None):
        """Select and compact every sequence that exceeds the budget; the
        moves apply to every KV head and layer."""
        B = self.budget if budget is None else budget
        for st in self.seqs.values():
            if st.n <= B:
                continue
            keep = select_keep(st.m[:st.n], st.pos[:st.n], B, self.n_sink, self.n_recent)
            for src, dst in hole_fill_moves(keep, B):
                st.K[:, :, dst] = st.K[:, :, src]
                st.V[:, :, dst] = st.V[:, :, src]
                st.pos[dst] = st.pos[src]
                st.m[dst] = st.m[src]
            st.n = B

    def scores(self, seq):
        st = self.seqs[seq]
        return st.m[:st.n].copy()

    def positions(self, seq):
        st = self.seqs[seq]
        return st.pos[:st.n].copy()


# ---------------------------------------------------------------------------
# Block-granular LRFU eviction with region decay and re-admission
# ---------------------------------------------------------------------------

def block_survival(labels, idle, beta, rates):
    """Mean idle-time survival of a block's tokens.

    ``(1/|b|) sum_i exp(-(beta + lambda_{r(i)}) * idle)``: the recency factor
    ``exp(-beta*idle)`` of [LRFU-fig] times the region decay
    ``exp(-lambda_r*idle)`` of [MemDecay] §III-C Eq.4, averaged over the
    block's tokens as [MemDecay] §III-D Eq.5 averages a page's scores.
    ``labels``: region id of each token of the block; ``rates``: lambda per
    region.  With every lambda at 0 this is ``exp(-beta*idle)``.
    """
    lam = np.asarray(rates, dtype=np.float64)[np.asarray(labels, dtype=np.int64)]
    return float(np.mean(np.exp(-(beta + lam) * float(idle))))


def block_priority(score, labels, idle, beta, rates):
    """Eviction priority ``(1 - score) * (1 - survival)`` of one block.

    [LRFU-fig] priority ``(1 - score)(1 - exp(-beta*idle))``, with the
    survival term extended by the block's region decay (reading: the decay
    of [MemDecay] multiplies the recency term; with no region decay this is
    exactly the figure's formula).  The HIGHER priority is evicted.
    """
    return (1.0 - float(score)) * (1.0 - block_survival(labels, idle, beta, rates))


def select_blocks(ids, prio, pinned, budget):
    """Blocks kept: the pinned ones plus the lowest-priority rest.

    [MemDecay] §III-A Eq.1 with the pinned set forced, §III-D: non-pinned
    pages go in ascending score order; here the score to keep is low
    priority.  Reading: equal priorities keep the higher block id (the more
    recent block).  Returns the sorted list of kept ids.
    """
    ids = np.asarray(ids, dtype=np.int64)
    prio = np.asarray(prio, dtype=np.float64)
    pinned = np.asarray(pinned, dtype=bool)
    if len(ids) <= budget:
        return sorted(ids.tolist())
    room = budget - int(pinned.sum())
    if room < 0:
        raise ValueError("pinned blocks exceed the budget")
    cand = np.flatnonzero(~pinned)
    # kept first: ascending priority, then descending id
    order = cand[np.lexsort((-ids[cand], prio[cand]))]
    kept = ids[pinned].tolist() + ids[order[:room]].tolist()
    return sorted(kept)


@dataclass
class _BlockSeq:
    """One sequence of the block-granular mode, indexed by position."""
    K: np.ndarray            # [L, Hkv, cap, d] float64 (exact widenings of the inputs)
    V: np.ndarray
    labels: list             # region id of every position so far
    npos: int                # positions 0 .. npos-1 exist
    budget: int              # blocks
    score: dict = field(default_factory=dict)   # block id -> fp64 score
    tref: dict = field(default_factory=dict)    # block id -> last access step
    resident: set = field(default_factory=set)  # block ids in the cache
    last_mass: dict = field(default_factory=dict)
    last_nres: int = 0       # resident tokens during the last step


@dataclass
class BlockLRFUOracle:
    """Per-(sequence, block) LRFU state, region decay, pinning, re-admission.

    Follows [LRFU-fig] (block unit of 16 tokens over every head and layer;
    EMA score; priority; an evicted block's score persists and is restored
    on re-admission) and [MemDecay] §III (region labels, pinned system
    region, the decay clock of Eq.3 with a threshold scaled to the uniform
    level, per-page eviction until the budget holds).

    Readings:

    * Block mass at step t: the attention probability landing on the
      block's tokens, summed over every layer and query head and divided by
      ``Hq * L`` (so masses over resident blocks sum to 1).
    * Score: 0 when the block enters (prefill or its first decode token);
      ``score <- ema(score, mass)`` for resident blocks every step; frozen
      while evicted; unchanged by re-admission.
    * Clock: ``tref`` is the insertion step (0 for prefill blocks, t for a
      block opened by step t's token), set to t when the block's mean mass
      per token is at least ``tau_mult / |K_t|`` (|K_t| the resident token
      count, [MemDecay] §IV-A uses tau = 2/|K_t|), and to the current step
      count on re-admission.  ``idle = t - tref``.
    * Pinned: every block holding a token of a pinned region ([MemDecay]
      §IV-A: pinning protects whole pages) and the block holding the newest
      token (it is still being filled).
    * Decode tokens take ``decode_region`` (the scratch region).
    * Eviction happens once per step after the update whenever more than
      ``budget`` blocks are resident.
    """
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    alpha_new: float
    beta: float
    half_lives: tuple
    pinned_regions: tuple = (0,)
    decode_region: int = 4
    tau_mult: float = 2.0
    page: int = 16
    capacity: int = 0
    seqs: dict = field(default_factory=dict)

    @property
    def group_size(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def rates(self):
        return region_decay_rates(self.half_lives)

    def prefill(self, seq, K, V, labels, budget):
        """Store a sequence's prefill K/V ([L, Hkv, n, d]) and region labels."""
        K = np.asarray(K, dtype=np.float32)
        V = np.asarray(V, dtype=np.float32)
        L, H, n, d = K.shape
        cap = max(self.capacity, n + 1)
        s = _BlockSeq(K=np.zeros((L, H, cap, d), np.float64), V=np.zeros((L, H, cap, d), np.float64),
                      labels=[int(x) for x in labels], npos=n, budget=int(budget))
        if len(s.labels) != n:
            raise ValueError("one region label per prefill token")
        s.K[:, :, :n] = K
        s.V[:, :, :n] = V
        for j in range((n + self.page - 1) // self.page):
            s.score[j] = 0.0
            s.tref[j] = 0
            s.resident.add(j)
        self.seqs[seq] = s

    # -- block views ------------------------------------------------------
    def block_positions(self, seq, j):
        s = self.seqs[seq]
        return list(range(j * self.page, min((j + 1) * self.page, s.npos)))

    def tail_block(self, seq):
        return (self.seqs[seq].npos - 1) // self.page

    def is_pinned(self, seq, j):
        s = self.seqs[seq]
        if j == self.tail_block(seq):
            return True
        return any(s.labels[i] in self.pinned_regions for i in self.block_positions(seq, j))

    def priority(self, seq, j, t):
        s = self.seqs[seq]
        labels = [s.labels[i] for i in self.block_positions(seq, j)]
        return block_priority(s.score[j], labels, t - s.tref[j], self.beta, self.rates)

    def resident_positions(self, seq):
        s = self.seqs[seq]
        pos = []
        for j in sorted(s.resident):
            pos.extend(self.block_positions(seq, j))
        return np.asarray(pos, dtype=np.int64)

    # -- the step -----------------------------------------------------------
    def _grow(self, s):
        if s.npos < s.K.shape[2]:
            return
        extra = max(64, s.K.shape[2] // 4)
        pad = lambda a: np.concatenate(
            [a, np.zeros(a.shape[:2] + (extra,) + a.shape[3:], a.dtype)], axis=2)
        s.K, s.V = pad(s.K), pad(s.V)

    def decode_step(self, t, q, k_new, v_new, seqs):
        """Append, attend over the resident blocks, update score and clock.

        ``q``: [L, len(seqs), Hq, d]; ``k_new``, ``v_new``: [L, len(seqs),
        Hkv, d].  Returns ``out`` [L, len(seqs), Hq, d] (fp64).
        """
        q = np.asarray(q, dtype=np.float32)
        k_new = np.asarray(k_new, dtype=np.float32)
        v_new = np.asarray(v_new, dtype=np.float32)
        L, Hq, Hg, pg = self.n_layers, self.n_q_heads, self.group_size, self.page
        out = np.zeros((L, len(seqs), Hq, self.head_dim))
        for bi, seq in enumerate(seqs):
            s = self.seqs[seq]
            self._grow(s)
            p_new = s.npos
            s.K[:, :, p_new] = k_new[:, bi]
            s.V[:, :, p_new] = v_new[:, bi]
            s.labels.append(self.decode_region)
            s.npos += 1
            if p_new % pg == 0:                      # the token opens a block
                j = p_new // pg
                s.score[j] = 0.0
                s.tref[j] = t
                s.resident.add(j)
            pos = self.resident_positions(seq)
            tok_mass = np.zeros(len(pos))
            for l in range(L):
                for h in range(self.n_kv_heads):
                    o, p, _ = decode_attention(q[l, bi, h * Hg:(h + 1) * Hg],
                                               s.K[l, h, pos], s.V[l, h, pos])
                    out[l, bi, h * Hg:(h + 1) * Hg] = o
                    tok_mass += p.sum(axis=0)
            tok_mass /= Hq * L
            n_res = len(pos)
            s.last_nres = n_res
            s.last_mass = {}
            at = 0
            for j in sorted(s.resident):
                nb = len(self.block_positions(seq, j))
                mass = float(tok_mass[at:at + nb].sum())
                at += nb
                s.last_mass[j] = mass
                s.score[j] = ema_update(s.score[j], mass, self.alpha_new)
                if mass / nb >= self.tau_mult / n_res:
                    s.tref[j] = t
        return out

    def evict(self, t, seqs=None):
        """Evict down to each sequence's block budget at clock ``t``."""
        for seq in (self.seqs if seqs is None else seqs):
            s = self.seqs[seq]
            if len(s.resident) <= s.budget:
                continue
            ids = sorted(s.resident)
            prio = [self.priority(seq, j, t) for j in ids]
            pinned = [self.is_pinned(seq, j) for j in ids]
            s.resident = set(select_blocks(ids, prio, pinned, s.budget))

    def readmit(self, seq, j, t):
        """Bring evicted block ``j`` back: score restored, clock set to t.

        [LRFU-fig]: an evicted block's key and score persist and are
        restored on re-admission rather than reset.
        """
        s = self.seqs[seq]
        if j in s.resident or j not in s.score:
            raise ValueError("block is resident or was never cached")
        s.resident.add(j)
        s.tref[j] = t

    # -- views used by tests ------------------------------------------------
    def block_state(self, seq):
        """(ids, score, tref, resident) over every block seen so far."""
        s = self.seqs[seq]
        ids = np.arange((s.npos + self.page - 1) // self.page)
        score = np.array([s.score[j] for j in ids], dtype=np.float64)
        tref = np.array([s.tref[j] for j in ids], dtype=np.int64)
        res = np.array([j in s.resident for j in ids], dtype=bool)
        return ids, score, tref, res


class RoutingDiagnostics:
    """Selection churn and Global LIR of one layer's routing events.

    [QEvict] §3: selection churn is the Jaccard distance between the retained
    sets of consecutive routing events; Global LIR measures how often a
    window that stayed out of the full-precision set for a sustained period
    re-enters it.  Readings: the sets are taken over the event's candidates
    (aged windows not evicted before it): F = those routed to full
    precision, R = those kept (full precision or INT2); a window's run of
    consecutive events outside F is sustained once it reaches ``gap`` events
    (the review leaves the length open) and revived when the window then
    re-enters F.  Feed ``observe`` with each event's candidates and the
    tiers after it (0 full precision, 1 INT2, 2 evicted).
    """

    def __init__(self, gap):
        self.gap = int(gap)
        self.prev = None  # (F, R) of the previous event
        self.run = {}
        self.sums = {"events": 0, "pairs": 0, "sum_f_churn": 0.0, "sum_r_churn": 0.0,
                     "sustained": 0, "revived": 0}

    def observe(self, candidates, tiers):
        F = {int(w) for w in candidates if tiers[w] == 0}
        R = {int(w) for w in candidates if tiers[w] != 2}
        sm = self.sums
        sm["events"] += 1
        c = {"f_new": len(F), "r_new": len(R)}
        if self.prev is None:
            c.update(f_prev=0, f_overlap=0, r_prev=0, r_overlap=0)
        else:
            Fp, Rp = self.prev
            c.update(f_prev=len(Fp), f_overlap=len(F & Fp), r_prev=len(Rp), r_overlap=len(R & Rp))
            sm["pairs"] += 1
            sm["sum_f_churn"] += 1.0 - jaccard(F, Fp)
            sm["sum_r_churn"] += 1.0 - jaccard(R, Rp)
        for w in candidates:
            w = int(w)
            run = self.run.get(w, 0)
            if tiers[w] == 0:
                sm["revived"] += 1 if run >= self.gap else 0
                run = 0
            else:
                run += 1
                sm["sustained"] += 1 if run == self.gap else 0
            self.run[w] = run
        self.prev = (F, R)
        return c


class HostOffloadPool:
    """Which evicted blocks a host pool of ``capacity`` slots still holds.

    [MemDecay] §III-E: a tiered extension offloads pages to host memory
    before dropping them and recovers them when later queries make them
    relevant again; [LRFU-fig]: a block's policy state persists across its
    eviction.  Readings: one slot holds one block (every layer and KV head);
    slots are reused in ring order, so the pool keeps the latest evictions;
    within one selection the evicted blocks are ordered by (sequence, block
    id) and, when there are more than ``capacity`` of them, only the last
    ``capacity`` are kept; a re-admitted block's slot is released (a
    resident block holds no slot).  The graded rule of [MemDecay] §III-E
    (offload above a threshold, drop below it) is the caller's filter:
    ``offload`` receives only the evictions to keep.
    """

    def __init__(self, capacity):
        self.capacity = int(capacity)
        self.slots = [None] * self.capacity
        self.where = {}  # (seq, block) -> slot
        self.ring = 0

    def offload(self, evicted):
        """Record one selection's evictions, an iterable of (seq, block)."""
        order = sorted(evicted)
        kept = min(self.capacity, len(order))
        for i, key in enumerate(order[len(order) - kept:]):
            s = (self.ring + i) % self.capacity
            prev = self.slots[s]
            if prev is not None and self.where.get(prev) == s:
                del self.where[prev]
            self.slots[s] = key
            self.where[key] = s
        self.ring = (self.ring + kept) % self.capacity

    def readmit(self, key):
        s = self.where.pop(key)
        self.slots[s] = None

    def slot(self, key):
        return self.where.get(key, -1)


# ---------------------------------------------------------------------------
# Two-tier window routing: full precision / INT2 / evicted (QEvict)
# ---------------------------------------------------------------------------

def bf16_round(x):
    """fp32 -> nearest bf16 (ties to even), returned as fp32 (torch CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


@dataclass
class _TierLayer:
    """One layer's windows: FP storage, ledger, tier and cumulative score."""
    K: np.ndarray            # [Hkv, cap, d] fp32: full-precision values by position
    V: np.ndarray
    Kpre: np.ndarray         # [Hkv, cap, d] fp32: the keys before the rotation (rotary mode), else empty
    Keff: np.ndarray         # [Hkv, cap, d] fp64 holding fp32 values: what attention reads
                             # (full precision or the INT2 reconstruction)
    Veff: np.ndarray
    tier: dict = field(default_factory=dict)     # window -> "F" | "Q" | "E"
    S: dict = field(default_factory=dict)        # window -> cumulative score (fp64)
    ledger: dict = field(default_factory=dict)   # window -> per-head INT2 codes + params


@dataclass
class TieredOracle:
    """Per-layer window routing over a full-precision tier, a recoverable
    INT2 tier and permanent eviction ([QEvict] technical review, §4).

    Windows are the routing unit: window w holds positions
    [w*W, (w+1)*W).  Readings:

    * Pinned windows hold a sink position (< n_sink); local windows hold
      one of the n_recent newest positions or are not yet full.  Both stay
      full precision and are never routed.  Every other window is "aged";
      a window is routed from the step it ages out of the local region
      ([QEvict] §4.1 protected sink prefix and recent region; §4.4 Eq.4).
    * All windows start full precision ([QEvict] §2, Stage 1).
    * Score ([QEvict] §4.2 Eq.1 with a routing interval of one step): at
      every step each accessible window gains the attention probability
      landing on its tokens, summed over the layer's query heads and
      divided by Hq.  Scores start at 0 at the first decode step; a window
      opened during decoding starts at 0.  Evicted windows keep their last
      score and gain nothing.
    * Routing, per layer after every step ([QEvict] §4.4 Eq.4-5 and
      Algorithm 1): candidates = aged windows not evicted; F = the K_f best
      by (score, window index), Q = the next K_q, the rest evicted for good.
    * A window entering Q is quantized only if it has no ledger entry yet
      (its first demotion); otherwise the stored codes are reused.  Keys
      are quantized per channel over the window's tokens, values per token
      in 32-channel groups ([QEvict] §4.4 Algorithm 1; ``int2_quantize``).
      With ``key_groups="token32"`` the keys are grouped like the values,
      per token and 32-channel group (the 131k workload's wording read
      literally: a "per-32-channel-group" scale and zero for both).
    * A window promoted from Q to F gets its dequantized values rounded to
      bf16 as its full-precision storage.
    * Rotary mode (``rope_theta`` > 0; [QEvict] §4.4, "Positional handling
      for promoted keys"): prefill keys, appended keys and queries arrive
      before the rotation.  Full-precision storage holds the rotated keys
      rounded to bf16, ``bf16(rope(k, position))``; queries enter
      attention as ``bf16(rope(q, p))`` at the new token's position p (a
      bf16 model's rotated query).  Keys are quantized from the keys before
      the rotation; the reconstruction of a key is ``rope(code*scale +
      zero, original position)``, and a promotion stores it rounded to
      bf16.  Without rotary mode the keys carry no rotation and there is
      none to re-apply.
    * Attention reads full-precision windows from storage and INT2 windows
      through their reconstruction ([QEvict] §4.1, the accessible keys and
      values): exact (fp32 ``code*scale + zero``, rotated in fp64) by
      default, or rounded to bf16 when ``reconstruct_bf16`` is set.  With
      ``reconstruct_bf16`` the reconstruction also replaces the window's
      full-precision storage when it enters the INT2 tier, so that storage
      already holds what a later promotion writes.

    Layers are independent, so the object may hold any subset of them.
    """
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    k_f: int
    k_q: int
    window: int = 32
    n_sink: int = 0
    n_recent: int = 0
    capacity: int = 0
    route_interval: int = 1
    rope_theta: float = 0.0
    reconstruct_bf16: bool = False
    key_groups: str = "channel"
    layers: dict = field(default_factory=dict)
    npos: int = 0
    last_mass: dict = field(default_factory=dict)

    def routes_after(self, t):
        """Routing events follow the decode steps t with t = 0 mod Omega
        ([QEvict] §4.2 Eq.1, "every Omega generated tokens"; the scores
        accumulate every step, Eq.1's sum over the interval).  Omega <= 1:
        every step."""
        return t % max(self.route_interval, 1) == 0

    @property
    def group_size(self):
        return self.n_q_heads // self.n_kv_heads

    def prefill(self, K, V, layers=None):
        """Store the prefill cache: ``K``, ``V`` [len(layers), Hkv, n, d]."""
        K = np.asarray(K, dtype=np.float32)
        V = np.asarray(V, dtype=np.float32)
        nl, H, n, d = K.shape
        layers = list(range(nl)) if layers is None else list(layers)
        cap = max(self.capacity, n + 1)
        rot = self.rope_theta > 0
        for j, l in enumerate(layers):
            st = _TierLayer(K=np.zeros((H, cap, d), np.float32), V=np.zeros((H, cap, d), np.float32),
                            Kpre=np.zeros((H, cap if rot else 0, d), np.float32),
                            Keff=np.zeros((H, cap, d), np.float64), Veff=np.zeros((H, cap, d), np.float64))
            kj = K[j]
            if rot:
                st.Kpre[:, :n] = K[j]
                kj = np.stack([bf16_round(rope(K[j, h], np.arange(n), self.rope_theta)) for h in range(H)])
            for arr in (st.K, st.Keff):
                arr[:, :n] = kj
            for arr in (st.V, st.Veff):
                arr[:, :n] = V[j]
            for w in range(self.n_windows(n)):
                st.tier[w] = "F"
                st.S[w] = 0.0
            self.layers[l] = st
        self.npos = n

    # -- window geometry ----------------------------------------------------
    def n_windows(self, npos=None):
        npos = self.npos if npos is None else npos
        return -(-npos // self.window)

    def is_pinned(self, w):
        return w * self.window < self.n_sink

    def is_aged(self, w):
        """Full, older than the n_recent newest positions, and not pinned."""
        recent_lo = self.npos - self.n_recent
        return not self.is_pinned(w) and (w + 1) * self.window <= recent_lo

    def window_positions(self, w):
        return np.arange(w * self.window, min((w + 1) * self.window, self.npos))

    def accessible_positions(self, l):
        st = self.layers[l]
        ws = [w for w in range(self.n_windows()) if st.tier[w] != "E"]
        return np.concatenate([self.window_positions(w) for w in ws]).astype(np.int64), ws

    # -- the step ---------------------------------------------------------
    def _grow(self, st):
        if self.npos < st.K.shape[1]:
            return
        extra = max(64, st.K.shape[1] // 4)
        for name in ("K", "V", "Keff", "Veff") + (("Kpre",) if self.rope_theta > 0 else ()):
            a = getattr(st, name)
            setattr(st, name, np.concatenate([a, np.zeros((a.shape[0], extra, a.shape[2]), a.dtype)], 1))

    def decode_step(self, t, q, k_new, v_new):
        """Append, attend over the accessible windows, add window masses.

        ``q``: [len(held layers), Hq, d]; ``k_new``, ``v_new``: [len(held
        layers), Hkv, d] (held layers in ascending order).  Returns ``out``
        [len(held layers), Hq, d] in fp64.
        """
        q = np.asarray(q, dtype=np.float32)
        k_new = np.asarray(k_new, dtype=np.float32)
        v_new = np.asarray(v_new, dtype=np.float32)
        held = sorted(self.layers)
        p = self.npos
        rot = self.rope_theta > 0
        if rot:                                      # the query at the new token's position
            q = np.stack([bf16_round(rope(q[j], np.full(q.shape[1], p), self.rope_theta))
                          for j in range(q.shape[0])])
        for j, l in enumerate(held):
            st = self.layers[l]
            self._grow(st)
            kj = k_new[j]
            if rot:
                st.Kpre[:, p] = k_new[j]
                kj = bf16_round(rope(k_new[j], np.full(k_new.shape[1], p), self.rope_theta))
            for arr in (st.K, st.Keff):
                arr[:, p] = kj
            for arr in (st.V, st.Veff):
                arr[:, p] = v_new[j]
            w = p // self.window
            if w not in st.tier:                     # the token opens a window
                st.tier[w] = "F"
                st.S[w] = 0.0
        self.npos = p + 1
        Hg = self.group_size
        out = np.zeros((len(held), self.n_q_heads, self.head_dim))
        self.last_mass = {}
        for j, l in enumerate(held):
            st = self.layers[l]
            pos, ws = self.accessible_positions(l)
            tok_mass = np.zeros(len(pos))
            for h in range(self.n_kv_heads):
                o, pr, _ = decode_attention(q[j, h * Hg:(h + 1) * Hg], st.Keff[h, pos], st.Veff[h, pos])
                out[j, h * Hg:(h + 1) * Hg] = o
                tok_mass += pr.sum(axis=0)
            tok_mass /= self.n_q_heads
            at = 0
            masses = {}
            for w in ws:
                nb = len(self.window_positions(w))
                masses[w] = float(tok_mass[at:at + nb].sum())
                at += nb
                st.S[w] = cumulative_update(st.S[w], masses[w])
            self.last_mass[l] = masses
        return out

    def _quantize_window(self, st, w):
        sl = slice(w * self.window, (w + 1) * self.window)
        src = st.Kpre if self.rope_theta > 0 else st.K     # keys before the rotation
        entry = []
        for h in range(self.n_kv_heads):
            kc, ks, kz = int2_quantize(src[h, sl], self.key_groups)
            vc, vs, vz = int2_quantize(st.V[h, sl], "token32")
            entry.append((kc, ks, kz, vc, vs, vz))
        st.ledger[w] = entry

    def _reconstruct(self, st, w):
        sl = slice(w * self.window, (w + 1) * self.window)
        pos = np.arange(w * self.window, (w + 1) * self.window)
        for h, (kc, ks, kz, vc, vs, vz) in enumerate(st.ledger[w]):
            k = int2_dequantize(kc, ks, kz, self.key_groups).astype(np.float64)
            if self.rope_theta > 0:                  # re-rotated at the original positions
                k = rope(k, pos, self.rope_theta)
            v = int2_dequantize(vc, vs, vz, "token32")
            if self.reconstruct_bf16:
                k, v = bf16_round(k), bf16_round(v)
            st.Keff[h, sl] = k
            st.Veff[h, sl] = v

    def route(self):
        """One routing event in every held layer (after the step's attention)."""
        for l, st in self.layers.items():
            cand = [w for w in range(self.n_windows()) if self.is_aged(w) and st.tier[w] != "E"]
            S = np.zeros(self.n_windows())
            for w in cand:
                S[w] = st.S[w]
            F, Q, E = route_tiers(S, cand, self.k_f, self.k_q)
            sl = lambda w: slice(w * self.window, (w + 1) * self.window)
            for w in Q:
                if w not in st.ledger:                   # first demotion: quantize once
                    self._quantize_window(st, w)
                if st.tier[w] != "Q":                    # entering INT2: attention reads the reconstruction
                    self._reconstruct(st, w)
                    if self.reconstruct_bf16:            # which also becomes the stored full precision
                        st.K[:, sl(w)] = st.Keff[:, sl(w)]
                        st.V[:, sl(w)] = st.Veff[:, sl(w)]
                st.tier[w] = "Q"
            for w in F:
                if st.tier[w] == "Q":                    # promotion: dequantize into bf16 storage
                    self._reconstruct(st, w)
                    st.K[:, sl(w)] = bf16_round(st.Keff[:, sl(w)])
                    st.V[:, sl(w)] = bf16_round(st.Veff[:, sl(w)])
                st.Keff[:, sl(w)] = st.K[:, sl(w)]
                st.Veff[:, sl(w)] = st.V[:, sl(w)]
                st.tier[w] = "F"
            for w in E:                                  # evicted for good: the record is freed too
                st.tier[w] = "E"
                st.ledger.pop(w, None)

    # -- views used by tests ------------------------------------------------
    def window_state(self, l):
        """(scores [nw] fp64, tiers [nw] uint8: 0 full precision, 1 INT2,
        2 evicted, ledger [nw] bool) for windows 0 .. n_windows-1."""
        st = self.layers[l]
        nw = self.n_windows()
        code = {"F": 0, "Q": 1, "E": 2}
        return (np.array([st.S[w] for w in range(nw)], np.float64),
                np.array([code[st.tier[w]] for w in range(nw)], np.uint8),
                np.array([w in st.ledger for w in range(nw)], bool))
