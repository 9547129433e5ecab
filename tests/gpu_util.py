"""Lockstep comparison of the HIP library with the CPU oracle (GPU tests)."""
from __future__ import annotations

import sys
import time
from dataclasses import dataclass, field

import numpy as np

import oracle as orc


def log(*a):
    from conftest import progress
    progress(*a)


@dataclass
class Stats:
    steps: int = 0
    near_tie_resyncs: int = 0
    max_out_err: float = 0.0
    max_score_err: float = 0.0
    kv_checks: int = 0
    exact_selection_checks: int = 0
    notes: list = field(default_factory=list)


def rel_err_scores(x, ref):
    """max over elements of |x - ref| / (|ref| + 1e-30/rtol-floor)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.abs(x - ref), np.abs(ref)


def check_scores(gpu, ref, rtol, what):
    diff = np.abs(np.asarray(gpu, np.float64) - ref)
    bound = rtol * np.abs(ref) + 1e-30
    bad = np.flatnonzero(diff > bound)
    assert bad.size == 0, (f"{what}: {bad.size} scores outside tolerance; first slot {bad[0]}: "
                           f"gpu={gpu[bad[0]]!r} ref={ref[bad[0]]!r}")
    nz = np.abs(ref) > 0
    return float((diff[nz] / np.abs(ref[nz])).max()) if nz.any() else 0.0


def check_out(gpu, ref, rtol, what):
    """Per head: ||o - o_ref||_inf <= rtol ||o_ref||_inf."""
    worst = 0.0
    for h in range(ref.shape[0]):
        den = np.abs(ref[h]).max()
        err = np.abs(gpu[h] - ref[h]).max()
        assert err <= rtol * den, f"{what} head {h}: err {err} > {rtol} * {den}"
        worst = max(worst, err / den if den > 0 else 0.0)
    return worst


def expected_after_evict(scores, pos_pre, B, n_sink, n_recent):
    """The positions the oracle's selection keeps from the GPU's own
    pre-evict scores (fp32 widened to fp64 exactly), sorted."""
    keep = orc.select_keep(np.asarray(scores, np.float64), pos_pre, B, n_sink, n_recent)
    return np.sort(np.asarray(pos_pre)[keep])


def by_position(pos, *arrays):
    """Positions and per-slot arrays sorted by position.  The library keeps
    its own slot order (a single-token eviction leaves its slot free for the
    next token; larger evictions fill holes), so parity is checked position
    by position."""
    o = np.argsort(np.asarray(pos), kind="stable")
    return (np.asarray(pos)[o],) + tuple(np.asarray(a)[o] for a in arrays)


def rows_by_position(K, pos_ref, pos_want):
    """Rows (axis 1 of K [L, n, d]) of the positions pos_want, taken from an
    array laid out by pos_ref."""
    idx = {p: j for j, p in enumerate(np.asarray(pos_ref).tolist())}
    return K[:, [idx[p] for p in np.asarray(pos_want).tolist()]]


class OracleThreads:
    """Steps independent oracle objects (one per selection group, sequence or
    layer) in worker threads.  The oracle's arithmetic is unchanged; numpy
    releases the interpreter lock inside its array kernels, and the BLAS
    pool is held at one thread per call while this object is open so the
    workers do not oversubscribe the cores."""

    def __init__(self, n_items, threads=None):
        import os
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        n = threads if threads is not None else min(n_items, 16, os.cpu_count() or 1)
        self.ex = ThreadPoolExecutor(n) if n > 1 else None
        self._lim = threadpool_limits(limits=1, user_api="blas") if n > 1 else None

    def map(self, fn, items):
        items = list(items)
        if self.ex is None:
            return [fn(x) for x in items]
        return list(self.ex.map(fn, items))

    def close(self):
        if self.ex is not None:
            self.ex.shutdown()
            self._lim.restore_original_limits()


def near_tie_excused(gaps, theta, rtol):
    """The near-tie exemption for a retained-set mismatch: every differing
    item's oracle score lies within 1e-5 of the oracle's boundary score
    theta (absolute), and within 4*rtol*|theta| of it: a score known to
    rtol relative can only swap order with another inside that band."""
    g = max(gaps)
    return g < 1e-5 and g <= 4.0 * rtol * abs(theta) + 1e-30


def run_token_lockstep(w, steps, *, sample_seqs=None, sample_heads=None, rtol=None,
                       kv_every=1, budget=None, device="cuda", ctx_steps=None, fused=False,
                       twin=False, threads=None, sync_every=32, max_resyncs=None):
    """Run `steps` decode+evict steps of workload `w` on the GPU and the oracle.

    One oracle object per sampled (sequence, KV head) group, stepped in
    threads.  Modes:
    * fused=False: kvev_decode_step + kvev_evict; the pre-evict positions
      and utilities and the selection on the GPU's own utilities are checked
      every step;
    * fused=True: kvev_step (the benchmark's launch configuration); the
      post-evict state is checked;
    * twin=True: both contexts on the same inputs; the separate-call one is
      checked against the oracle as above, and the kvev_step one must equal
      it bit for bit every step (outputs, utilities and positions in slot
      order, and K/V at the K/V checks).
    On an excused near tie the GPU imports the oracle's group state
    (positions, utilities rounded to fp32, K/V); the oracle is never
    changed.  Every context is synchronised (and its consistency flag read)
    every `sync_every` steps and at the end."""
    import torch
    from decode_kv_cache_gqa_amd import kvev

    rtol = rtol if rtol is not None else (1e-5 if w.dtype == "f32" else 2e-3)
    B = w.budget if budget is None else budget
    sample_seqs = list(range(w.batch)) if sample_seqs is None else list(sample_seqs)
    sample_heads = list(range(w.n_kv_heads)) if sample_heads is None else list(sample_heads)
    keys = [(b, h) for b in sample_seqs for h in sample_heads]
    log(f"[lockstep] {w.name}: L={w.n_layers} batch={w.batch} L0={w.prefill_lens[:4]} steps={steps} "
        f"B={B} seqs={sample_seqs} heads={sample_heads} fused={fused} twin={twin}")
    t_start = time.time()
    nctx = 2 if twin else 1
    ctxs = [kvev.context_for(w, max_steps=ctx_steps or steps, budget=B) for _ in range(nctx)]
    sep = ctxs[0] if (twin or not fused) else None   # separate calls, checked pre-evict
    main = ctxs[0]                                    # the context checked against the oracle
    fus = ctxs[1] if twin else (ctxs[0] if fused else None)

    def new_oracle():
        return orc.TokenModeOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, budget=B,
                                   alpha_new=w.alpha_new,
                                   policy=w.policy if w.policy == "cumulative" else "ema",
                                   refresh_interval=w.refresh_interval, score_free=w.score_free,
                                   n_sink=w.n_sink, n_recent=w.n_recent,
                                   capacity=max(w.prefill_lens) + steps + 1, scorer=w.scorer,
                                   new_token_init="mean" if w.new_token_init == 1 else "zero")

    orcs = {k: new_oracle() for k in keys}
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device=device)
        for c in ctxs:
            c.prefill(b, K.contiguous(), V.contiguous())
        if b in sample_seqs:
            # the generator's rows, evaluated on the device (bit-identical to the CPU evaluation)
            sel = torch.tensor(sample_heads, device=K.device)
            Kc = K.index_select(1, sel).float().cpu().numpy()
            Vc = V.index_select(1, sel).float().cpu().numpy()
            for j, h in enumerate(sample_heads):
                orcs[(b, h)].prefill(b, Kc[:, j:j + 1], Vc[:, j:j + 1], heads=[h])
            del Kc, Vc
        del K, V
    torch.cuda.synchronize()
    log(f"[lockstep] prefill done in {time.time() - t_start:.1f}s")
    pool = OracleThreads(len(keys), threads)
    st = Stats()
    Hg = w.group_size
    outs = [torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32,
                        device=device) for _ in ctxs]
    seq_index = {b: i for i, b in enumerate(sample_seqs)}
    try:
        for t in range(1, steps + 1):
            q, kn, vn = w.step_inputs(t, device=device)
            for c, out in zip(ctxs, outs):
                if c is sep:
                    c.decode_step(q, kn, vn, out)
                else:
                    c.step(q, kn, vn, out, B)
            ss = torch.tensor(sample_seqs, device=q.device)
            qc = q.index_select(1, ss).float().cpu().numpy()
            knc = kn.index_select(1, ss).float().cpu().numpy()
            vnc = vn.index_select(1, ss).float().cpu().numpy()

            def ostep(k):
                bi = seq_index[k[0]]
                return orcs[k].decode_step(t, qc[:, bi:bi + 1], knc[:, bi:bi + 1], vnc[:, bi:bi + 1], [k[0]])

            refs = dict(zip(keys, pool.map(ostep, keys)))
            gout = outs[0].cpu().numpy()
            for (b, h) in keys:
                for l in range(w.n_layers):
                    st.max_out_err = max(st.max_out_err, check_out(
                        gout[l, b, h * Hg:(h + 1) * Hg], refs[(b, h)][l, 0, h * Hg:(h + 1) * Hg], rtol,
                        f"step {t} out l={l} b={b} kvh={h}"))
            if twin:
                assert torch.equal(outs[0], outs[1]), f"step {t}: kvev_step output differs from the separate calls"
            pre = {}
            if sep is not None:
                for (b, h) in keys:
                    gs = sep.scores(b, h)
                    gp = sep.retained(b, h)
                    gps, gss = by_position(gp, gs)
                    ops, oss = by_position(orcs[(b, h)].positions(b, h), orcs[(b, h)].scores(b, h))
                    np.testing.assert_array_equal(gps, ops, err_msg=f"step {t} pre-evict positions b={b} kvh={h}")
                    st.max_score_err = max(st.max_score_err, check_scores(
                        gss, oss, rtol, f"step {t} scores b={b} kvh={h}"))
                    pre[(b, h)] = (gs, gp)
                sep.evict(B)
            ref_pre = {k: (orcs[k].scores(*k), orcs[k].positions(*k)) for k in keys}
            pool.map(lambda k: orcs[k].evict(B), keys)
            for (b, h) in keys:
                got_slots = main.retained(b, h)
                if twin:
                    np.testing.assert_array_equal(fus.retained(b, h), got_slots,
                                                  err_msg=f"step {t} b={b} kvh={h}: kvev_step slots")
                    np.testing.assert_array_equal(fus.scores(b, h), main.scores(b, h),
                                                  err_msg=f"step {t} b={b} kvh={h}: kvev_step utilities")
                got = np.sort(got_slots)
                assert len(np.unique(got)) == len(got), f"step {t} b={b} kvh={h}: a position held twice"
                if sep is not None:
                    gs, gp = pre[(b, h)]
                    # selection on the GPU's own utilities: bit-exact
                    exp = expected_after_evict(gs, gp, B, w.n_sink, w.n_recent)
                    np.testing.assert_array_equal(got, exp, err_msg=f"step {t} selection on GPU scores b={b} kvh={h}")
                    st.exact_selection_checks += 1
                ms, pos_all = ref_pre[(b, h)]
                o = orcs[(b, h)]
                ref_pos = np.sort(o.positions(b, h))
                if not np.array_equal(got, ref_pos):
                    keep_ref = np.isin(pos_all, ref_pos)
                    prot = (pos_all < w.n_sink) | (pos_all > pos_all.max() - w.n_recent)
                    kept_scores = ms[keep_ref & ~prot]
                    theta = kept_scores.min() if kept_scores.size else 0.0
                    diff = set(got.tolist()) ^ set(ref_pos.tolist())
                    idx = {p: i for i, p in enumerate(pos_all.tolist())}
                    gaps = [abs(ms[idx[p]] - theta) for p in diff]
                    assert near_tie_excused(gaps, theta, rtol), (
                        f"step {t} b={b} kvh={h}: retained sets differ by {len(diff)} positions with oracle "
                        f"score gap {max(gaps):.3e} (boundary {theta:.3e})")
                    st.near_tie_resyncs += 1
                    g = o.groups[(b, h)]
                    kk = torch.from_numpy(g.K[:, :g.n].copy()).to(w.torch_dtype).to(device).contiguous()
                    vv = torch.from_numpy(g.V[:, :g.n].copy()).to(w.torch_dtype).to(device).contiguous()
                    for c in ctxs:
                        c.import_group(b, h, g.pos[:g.n], g.m[:g.n].astype(np.float32), kk, vv)
                    st.notes.append(f"t={t} b={b} h={h} near-tie resync ({len(diff)} positions, "
                                    f"gap {max(gaps):.2e})")
                    continue
                if sep is None:
                    _, gss = by_position(got_slots, main.scores(b, h))
                    _, oss = by_position(o.positions(b, h), o.scores(b, h))
                    st.max_score_err = max(st.max_score_err, check_scores(
                        gss, oss, rtol, f"step {t} post-evict scores b={b} kvh={h}"))
                if kv_every and (t % kv_every == 0 or t == steps):
                    gk, gv = main.export_kv(b, h)  # rows in the order of main.retained
                    g = o.groups[(b, h)]
                    rk = torch.from_numpy(rows_by_position(g.K, g.pos[:g.n], got_slots).copy()).to(w.torch_dtype)
                    rv = torch.from_numpy(rows_by_position(g.V, g.pos[:g.n], got_slots).copy()).to(w.torch_dtype)
                    assert torch.equal(gk.cpu(), rk), f"step {t} compacted K differs b={b} kvh={h}"
                    assert torch.equal(gv.cpu(), rv), f"step {t} compacted V differs b={b} kvh={h}"
                    if twin:
                        fk, fv = fus.export_kv(b, h)
                        assert torch.equal(fk, gk) and torch.equal(fv, gv), (
                            f"step {t} b={b} kvh={h}: kvev_step K/V differ from the separate calls")
                    st.kv_checks += 1
            st.steps = t
            if sync_every and t % sync_every == 0:
                for c in ctxs:
                    c.sync()
            if t == 1 or t % 16 == 0 or t == steps:
                log(f"[lockstep] step {t}: out_err {st.max_out_err:.2e} score_err {st.max_score_err:.2e} "
                    f"resyncs {st.near_tie_resyncs} ({time.time() - t_start:.1f}s)")
        for c in ctxs:
            c.sync()
    finally:
        pool.close()
        for c in ctxs:
            c.close()
    log(f"[lockstep] {w.name}: {st.steps} steps, {len(keys)} groups, near-tie resyncs "
        f"{st.near_tie_resyncs}, exact selections {st.exact_selection_checks}, K/V checks {st.kv_checks}")
    for n in st.notes:
        log(f"[lockstep]   {n}")
    if max_resyncs is not None:
        assert st.near_tie_resyncs <= max_resyncs, f"{st.near_tie_resyncs} near-tie resyncs > {max_resyncs}"
    return st


# ---------------------------------------------------------------------------
# Rank-trace diagnostics
# ---------------------------------------------------------------------------

def run_diag_lockstep(w, steps, k, *, sample_seqs=None, sample_heads=None, rtol=None,
                      check_values=True, fmm=False, device="cuda"):
    """Step workload `w` with diagnostics over the top-k and check, every step
    and for every sampled group:
    * the library's counts equal the oracle's rank-trace statistics computed
      from the library's own per-token inputs and retained set (the integer
      decisions taken on the same fp32 values: exact), and its sums agree;
    * (check_values) those inputs, position by position, equal the oracle's
      raw observation and utility within rtol.  A diagnostics context
      accepts no state import, so after an excused near tie the oracle (left
      unchanged) stops following that group's values; the counts are still
      checked against the library's own values every step;
    * (fmm) the missed mass against a never-evicting context equals the
      oracle's formula on the library's full-cache inputs and evicted sets.
    Returns the list of per-step diag_read() results of group 0."""
    import torch
    from decode_kv_cache_gqa_amd import kvev

    rtol = rtol if rtol is not None else (1e-5 if w.dtype == "f32" else 2e-3)
    B = w.budget
    Hkv = w.n_kv_heads
    sample_seqs = list(range(w.batch)) if sample_seqs is None else list(sample_seqs)
    sample_heads = list(range(Hkv)) if sample_heads is None else list(sample_heads)
    keys = [(b, h) for b in sample_seqs for h in sample_heads]
    log(f"[diag] {w.name}: L={w.n_layers} batch={w.batch} L0={w.prefill_lens[:4]} steps={steps} B={B} "
        f"k={k} groups={keys} values={check_values} fmm={fmm}")
    t_start = time.time()
    ctx = kvev.context_for(w, max_steps=steps, diag_topk=k)
    full = None
    if fmm:
        mt = max(w.prefill_lens) + steps + 1
        full = kvev.context_for(w, max_steps=steps, budget=mt, diag_topk=1)
    o = None
    if check_values:
        o = orc.TokenModeOracle(w.n_layers, w.n_q_heads, Hkv, w.head_dim, budget=B,
                                alpha_new=w.alpha_new,
                                policy=w.policy if w.policy == "cumulative" else "ema",
                                n_sink=w.n_sink, n_recent=w.n_recent,
                                capacity=max(w.prefill_lens) + steps + 1, scorer=w.scorer,
                                new_token_init="mean" if w.new_token_init == 1 else "zero")
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device=device)
        ctx.prefill(b, K.contiguous(), V.contiguous())
        if full is not None:
            full.prefill(b, K.contiguous(), V.contiguous())
        del K, V
        if o is not None and b in sample_seqs:
            Kc, Vc = w.prefill_kv(b, device="cpu", heads=sample_heads)
            o.prefill(b, Kc.float().numpy(), Vc.float().numpy(), heads=sample_heads)
    torch.cuda.synchronize()
    trackers = {key: orc.RankTraceDiagnostics(k) for key in keys}
    out = torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=device)
    out_full = torch.empty_like(out)
    history, resyncs, max_err = [], 0, 0.0
    following = set(keys)  # groups whose values the oracle still follows
    for t in range(1, steps + 1):
        q, kn, vn = w.step_inputs(t, device=device)
        ctx.step(q, kn, vn, out, B)
        if full is not None:
            full.step(q, kn, vn, out_full, 0)
        if o is not None:
            qc, knc, vnc = w.step_inputs(t, device="cpu", seqs=sample_seqs)
            o.decode_step(t, qc.float().numpy(), knc.float().numpy(), vnc.float().numpy(), sample_seqs)
        gd = ctx.diag_read()
        history.append(gd[0])
        pre = {}
        for (b, h) in keys:
            g = b * Hkv + h
            gpos, graw, gutil = ctx.diag_trace(b, h)
            kept = ctx.retained(b, h)
            exp = trackers[(b, h)].observe(gpos, graw.astype(np.float64), gutil.astype(np.float64), kept)
            got = {name: gd[g][name] for name in orc.RankTraceDiagnostics.COUNTS}
            assert got == exp, f"step {t} b={b} kvh={h}: counts {got} != oracle on the library's values {exp}"
            for name, val in trackers[(b, h)].sums.items():
                assert abs(gd[g][name] - val) <= 1e-12 * max(1.0, abs(val)), (
                    f"step {t} b={b} kvh={h}: {name} {gd[g][name]!r} != {val!r}")
            if o is not None and (b, h) in following:
                opos, oraw, outil = o.step_observation(b, h)
                gps, graw_s, gutil_s = by_position(gpos, graw, gutil)
                ops, oraw_s, outil_s = by_position(opos, oraw, outil)
                np.testing.assert_array_equal(gps, ops, err_msg=f"step {t} b={b} kvh={h}: step tokens")
                max_err = max(max_err, check_scores(graw_s, oraw_s, rtol, f"step {t} raw b={b} kvh={h}"),
                              check_scores(gutil_s, outil_s, rtol, f"step {t} util b={b} kvh={h}"))
                pre[(b, h)] = (kept, gps, gutil_s, ops, outil_s)
        if o is not None:
            o.evict(B)
            for (b, h) in list(following):
                kept, gps, gutil_s, ops, outil_s = pre[(b, h)]
                got = np.sort(kept)
                ref = np.sort(o.positions(b, h))
                if np.array_equal(got, ref):
                    continue
                # near tie: every differing position close to the kept minimum (oracle values)
                prot = (ops < w.n_sink) | (ops > ops.max() - w.n_recent)
                kept_ref = np.isin(ops, ref) & ~prot
                theta = outil_s[kept_ref].min() if kept_ref.any() else 0.0
                idx = {p: i for i, p in enumerate(ops.tolist())}
                gaps = [abs(outil_s[idx[p]] - theta) for p in set(got.tolist()) ^ set(ref.tolist())]
                assert near_tie_excused(gaps, theta, rtol), (
                    f"step {t} b={b} kvh={h}: retained sets differ (gap {max(gaps):.2e}, boundary {theta:.2e})")
                following.discard((b, h))
                resyncs += 1
                log(f"[diag] step {t} b={b} kvh={h}: excused near tie (gap {max(gaps):.2e}); "
                    f"the oracle stops following this group's values")
        if t % 32 == 0:
            ctx.sync()
        if full is not None:
            fm = kvev.diag_fmm(full, ctx)
            for (b, h) in keys:
                g = b * Hkv + h
                fpos, fraw, _ = full.diag_trace(b, h)
                assert len(fpos) == w.prefill_lens[b] + t, "the full context evicted"
                want = orc.future_missed_mass(fpos, fraw.astype(np.float64),
                                              trackers[(b, h)].evicted_before(t))
                assert abs(fm[g] - want) <= 1e-9 * max(want, 1e-12) + 1e-15, (
                    f"step {t} b={b} kvh={h}: fmm {fm[g]!r} != {want!r}")
        if t == 1 or t % 16 == 0 or t == steps:
            log(f"[diag] step {t}: value err {max_err:.2e} resyncs {resyncs} ({time.time() - t_start:.1f}s)")
    ctx.sync()
    ctx.close()
    if full is not None:
        full.sync()
        full.close()
    log(f"[diag] {w.name}: {steps} steps, near ties {resyncs}")
    return history


# ---------------------------------------------------------------------------
# Sequence-pooled token mode
# ---------------------------------------------------------------------------

def run_pooled_lockstep(w, steps, *, sample_seqs=None, rtol=None, device="cuda", fused=False,
                        kv_every=4, budget=None):
    """Run `steps` steps of a per-sequence (pooled) workload on the GPU and
    the oracle.  Every KV head of a sequence must report the same retained
    positions.  On an excused near tie every KV head of the sequence imports
    the oracle's state (positions, utilities rounded to fp32, K/V); the
    oracle is never changed."""
    import torch
    from decode_kv_cache_gqa_amd import kvev

    rtol = rtol if rtol is not None else (1e-5 if w.dtype == "f32" else 2e-3)
    B = w.budget if budget is None else budget
    sample = list(range(w.batch)) if sample_seqs is None else list(sample_seqs)
    Hkv, Hg = w.n_kv_heads, w.group_size
    log(f"[pooled] {w.name}: L={w.n_layers} Hq={w.n_q_heads} Hkv={Hkv} batch={w.batch} "
        f"L0={w.prefill_lens[:4]} steps={steps} B={B} sample={sample} fused={fused} scorer={w.scorer}")
    t_start = time.time()
    ctx = kvev.context_for(w, max_steps=steps, budget=B)
    o = orc.PooledTokenOracle(w.n_layers, w.n_q_heads, Hkv, w.head_dim, budget=B,
                              alpha_new=w.alpha_new,
                              policy=w.policy if w.policy == "cumulative" else "ema",
                              refresh_interval=w.refresh_interval, score_free=w.score_free,
                              n_sink=w.n_sink, n_recent=w.n_recent,
                              capacity=max(w.prefill_lens) + steps + 1, scorer=w.scorer,
                              new_token_init="mean" if w.new_token_init == 1 else "zero")
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device=device)
        ctx.prefill(b, K.contiguous(), V.contiguous())
        del K, V
        if b in sample:
            Kc, Vc = w.prefill_kv(b, device="cpu")
            o.prefill(b, Kc.float().numpy(), Vc.float().numpy())
    torch.cuda.synchronize()
    st = Stats()
    out = torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=device)

    def retained_all(b):
        pos = [ctx.retained(b, h) for h in range(Hkv)]
        for h in range(1, Hkv):
            np.testing.assert_array_equal(pos[h], pos[0], err_msg=f"seq {b}: KV head {h} holds other slots")
        return pos[0]

    for t in range(1, steps + 1):
        q, kn, vn = w.step_inputs(t, device=device)
        if fused:
            ctx.step(q, kn, vn, out, B)
        else:
            ctx.decode_step(q, kn, vn, out)
        qc, knc, vnc = w.step_inputs(t, device="cpu", seqs=sample)
        ref_out = o.decode_step(t, qc.float().numpy(), knc.float().numpy(), vnc.float().numpy(), sample)
        gout = out.cpu().numpy()
        for bi, b in enumerate(sample):
            for h in range(Hkv):
                for l in range(w.n_layers):
                    st.max_out_err = max(st.max_out_err, check_out(
                        gout[l, b, h * Hg:(h + 1) * Hg], ref_out[l, bi, h * Hg:(h + 1) * Hg], rtol,
                        f"step {t} out l={l} b={b} kvh={h}"))
        pre = {}
        if not fused:
            for b in sample:
                gp = retained_all(b)
                gs = ctx.scores(b, 0)
                gps, gss = by_position(gp, gs)
                ops, oss = by_position(o.positions(b), o.scores(b))
                np.testing.assert_array_equal(gps, ops, err_msg=f"step {t} pre-evict positions b={b}")
                st.max_score_err = max(st.max_score_err, check_scores(gss, oss, rtol,
                                                                      f"step {t} scores b={b}"))
                pre[b] = (gs, gp)
            ctx.evict(B)
        ref_pre = {b: (o.scores(b), o.positions(b)) for b in sample}
        o.evict(B)
        for b in sample:
            got_slots = retained_all(b)
            got = np.sort(got_slots)
            assert len(np.unique(got)) == len(got), f"step {t} b={b}: a position held twice"
            if not fused:
                gs, gp = pre[b]
                exp = expected_after_evict(gs, gp, B, w.n_sink, w.n_recent)
                np.testing.assert_array_equal(got, exp, err_msg=f"step {t} selection on GPU scores b={b}")
                st.exact_selection_checks += 1
            ref_pos = np.sort(o.positions(b))
            if not np.array_equal(got, ref_pos):
                ms, pos_all = ref_pre[b]
                keep_ref = np.isin(pos_all, ref_pos)
                prot = (pos_all < w.n_sink) | (pos_all > pos_all.max() - w.n_recent)
                kept = ms[keep_ref & ~prot]
                theta = kept.min() if kept.size else 0.0
                diff = set(got.tolist()) ^ set(ref_pos.tolist())
                idx = {p: i for i, p in enumerate(pos_all.tolist())}
                gaps = [abs(ms[idx[p]] - theta) for p in diff]
                assert near_tie_excused(gaps, theta, rtol), (
                    f"step {t} b={b}: retained sets differ by {len(diff)} positions with oracle score gap "
                    f"{max(gaps):.3e} (boundary {theta:.3e})")
                sst = o.seqs[b]
                for h in range(Hkv):
                    kk = torch.from_numpy(sst.K[:, h, :sst.n].copy()).to(w.torch_dtype).to(device).contiguous()
                    vv = torch.from_numpy(sst.V[:, h, :sst.n].copy()).to(w.torch_dtype).to(device).contiguous()
                    ctx.import_group(b, h, sst.pos[:sst.n], sst.m[:sst.n].astype(np.float32), kk, vv)
                st.near_tie_resyncs += 1
                st.notes.append(f"t={t} b={b} near-tie resync ({len(diff)} positions)")
                continue
            if fused:
                _, gss = by_position(got_slots, ctx.scores(b, 0))
                _, oss = by_position(o.positions(b), o.scores(b))
                st.max_score_err = max(st.max_score_err, check_scores(
                    gss, oss, rtol, f"step {t} post-evict scores b={b}"))
            if kv_every and t % kv_every == 0:
                sst = o.seqs[b]
                for h in range(Hkv):
                    gk, gv = ctx.export_kv(b, h)
                    rk = torch.from_numpy(rows_by_position(sst.K[:, h], sst.pos[:sst.n], got_slots).copy()
                                          ).to(w.torch_dtype)
                    rv = torch.from_numpy(rows_by_position(sst.V[:, h], sst.pos[:sst.n], got_slots).copy()
                                          ).to(w.torch_dtype)
                    assert torch.equal(gk.cpu(), rk), f"step {t} compacted K differs b={b} kvh={h}"
                    assert torch.equal(gv.cpu(), rv), f"step {t} compacted V differs b={b} kvh={h}"
                    st.kv_checks += 1
        st.steps = t
        if t == 1 or t % 16 == 0 or t == steps:
            log(f"[pooled] step {t}: out_err {st.max_out_err:.2e} score_err {st.max_score_err:.2e} "
                f"resyncs {st.near_tie_resyncs} ({time.time() - t_start:.1f}s)")
    ctx.sync()
    ctx.close()
    return st


# ---------------------------------------------------------------------------
# Block-granular LRFU mode
# ---------------------------------------------------------------------------

def block_rows(w, b, ids, device="cuda"):
    """K, V [L, Hkv, 16*len(ids), d] of blocks `ids` of sequence b: prefill
    rows regenerated from the seed, decoded rows from the step inputs that
    appended them."""
    import torch
    L0 = w.prefill_lens[b]
    pos = np.concatenate([np.arange(16 * j, 16 * j + 16) for j in ids]).astype(np.int64)
    K = torch.empty((w.n_layers, w.n_kv_heads, len(pos), w.head_dim), dtype=w.torch_dtype, device=device)
    V = torch.empty_like(K)
    pre = np.flatnonzero(pos < L0)
    if len(pre):
        Kp, Vp = w.prefill_rows(b, pos[pre], device=device)
        idx = torch.from_numpy(pre).to(device)
        K[:, :, idx] = Kp
        V[:, :, idx] = Vp
    for i in np.flatnonzero(pos >= L0).tolist():
        _, kn, vn = w.step_inputs(int(pos[i]) - L0 + 1, device=device, seqs=[b])
        K[:, :, i] = kn[:, 0]
        V[:, :, i] = vn[:, 0]
    return K.contiguous(), V.contiguous()


def _epoch_start(w, t):
    return w.epoch_steps > 0 and t > 1 and (t - 1) % w.epoch_steps == 0 and w.epoch_of(t) > w.epoch_of(t - 1)


def run_block_lockstep(w, steps, *, sample_seqs=None, rtol=None, device="cuda", fused=True,
                       readmit=True, kv_every=4, follow_steps=None, threads=None, sync_every=32,
                       readmit_all=True):
    """Run `steps` block-LRFU decode steps of workload `w` on the GPU and the
    oracle, with re-admission of each new epoch's heavy blocks.  One oracle
    object per sampled sequence, stepped in threads; follow_steps {seq: n}
    stops following a sequence after its first n steps (the GPU context
    keeps stepping the whole batch).  readmit_all=False re-admits only in
    the followed sequences (sequences are independent, so the others'
    re-admissions do not change the followed ones).  On an excused near tie
    the GPU imports the oracle's block state and K/V; the oracle is never
    changed."""
    import torch
    from decode_kv_cache_gqa_amd import kvev

    rtol = rtol if rtol is not None else (1e-5 if w.dtype == "f32" else 2e-3)
    sample = list(range(w.batch)) if sample_seqs is None else list(sample_seqs)
    follow = {b: steps for b in sample}
    if follow_steps:
        follow.update({b: min(n, steps) for b, n in follow_steps.items() if b in follow})
    log(f"[block] {w.name}: L={w.n_layers} batch={w.batch} L0={w.prefill_lens[:6]} steps={steps} "
        f"sample={sample} follow={follow} fused={fused} readmit={readmit}")
    t_start = time.time()
    ctx = kvev.context_for(w, max_steps=steps)

    def new_oracle():
        return orc.BlockLRFUOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, alpha_new=w.alpha_new,
                                   beta=w.beta, half_lives=tuple(w.region_half_lives),
                                   pinned_regions=tuple(w.pinned_regions), decode_region=w.decode_region,
                                   capacity=max(w.prefill_lens) + steps + 1)

    orcs = {b: new_oracle() for b in sample}
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device=device)
        lab = w.region_labels(b)
        ctx.prefill(b, K.contiguous(), V.contiguous(), lab)
        ctx.set_budget(b, w.block_budget(b))
        if b in orcs:
            orcs[b].prefill(b, K.float().cpu().numpy(), V.float().cpu().numpy(), lab, w.block_budget(b))
        del K, V
    torch.cuda.synchronize()
    log(f"[block] prefill done in {time.time() - t_start:.1f}s")
    pool = OracleThreads(len(sample), threads)
    st = Stats()
    st.readmitted = 0
    st.checked_seq_steps = 0
    out = torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=device)
    Hg = w.group_size
    try:
        for t in range(1, steps + 1):
            live = [b for b in sample if t <= follow[b]]
            if readmit and _epoch_start(w, t):
                e = w.epoch_of(t)
                for b in (range(w.batch) if readmit_all else live):
                    if b in live:
                        res = orcs[b].seqs[b].resident
                    else:
                        res = set(np.flatnonzero(ctx.block_state(b)[2]).tolist())
                    tail = (w.prefill_lens[b] + t - 2) // 16
                    ids = [j for j in w.heavy_blocks(b, e) if j not in res and j < tail]
                    if not ids:
                        continue
                    Kr, Vr = block_rows(w, b, ids, device)
                    ctx.readmit(b, ids, Kr, Vr)
                    st.readmitted += len(ids)
                    if b in live:
                        for j in ids:
                            orcs[b].readmit(b, j, t - 1)
            q, kn, vn = w.step_inputs(t, device=device)
            if fused:
                ctx.step(q, kn, vn, out)
            else:
                ctx.decode_step(q, kn, vn, out)
            if live:
                ls = torch.tensor(live, device=q.device)
                qs = q.index_select(1, ls).float().cpu().numpy()
                ks = kn.index_select(1, ls).float().cpu().numpy()
                vs = vn.index_select(1, ls).float().cpu().numpy()
                refs = dict(zip(live, pool.map(
                    lambda b: orcs[b].decode_step(t, qs[:, live.index(b):live.index(b) + 1],
                                                  ks[:, live.index(b):live.index(b) + 1],
                                                  vs[:, live.index(b):live.index(b) + 1], [b]), live)))
                gout = out.index_select(1, ls).cpu().numpy()
                for bi, b in enumerate(live):
                    for l in range(w.n_layers):
                        for h in range(w.n_kv_heads):
                            st.max_out_err = max(st.max_out_err, check_out(
                                gout[l, bi, h * Hg:(h + 1) * Hg], refs[b][l, 0, h * Hg:(h + 1) * Hg], rtol,
                                f"step {t} out l={l} b={b} kvh={h}"))
            if not fused:
                for b in live:
                    gsc, gtr, _ = ctx.block_state(b)
                    _, osc, otr, _ = orcs[b].block_state(b)
                    st.max_score_err = max(st.max_score_err, check_scores(gsc, osc, rtol, f"step {t} pre-evict b={b}"))
                ctx.evict()
            pool.map(lambda b: orcs[b].evict(t, seqs=[b]), live)
            for b in live:
                o = orcs[b]
                s = o.seqs[b]
                gsc, gtr, gres = ctx.block_state(b)
                ids, osc, otr, ores = o.block_state(b)
                assert len(gsc) == len(ids), f"step {t} b={b}: {len(gsc)} blocks on the GPU, {len(ids)} in the oracle"
                exempt = False
                for j in np.flatnonzero(gtr != otr).tolist():
                    # an access decision at the threshold: mass per token within 1e-5 of tau/|K|
                    nb = len(o.block_positions(b, j))
                    thr = 2.0 / s.last_nres
                    r = s.last_mass.get(j, -1.0) / nb
                    assert j in s.last_mass and abs(r - thr) <= 1e-5 * thr, (
                        f"step {t} b={b} block {j}: clock gpu {gtr[j]} oracle {otr[j]} (mass/token {r:.6e}, "
                        f"threshold {thr:.6e})")
                    exempt = True
                if not exempt and not np.array_equal(gres, ores):
                    kept = [j for j in np.flatnonzero(ores) if not o.is_pinned(b, j)]
                    theta = max(o.priority(b, j, t) for j in kept) if kept else 0.0
                    diff = np.flatnonzero(gres != ores).tolist()
                    gaps = [abs(o.priority(b, j, t) - theta) for j in diff]
                    assert near_tie_excused(gaps, theta, rtol), (
                        f"step {t} b={b}: resident blocks differ ({diff}) with oracle priority gap "
                        f"{max(gaps):.3e} (boundary {theta:.3e})")
                    exempt = True
                if exempt:
                    st.near_tie_resyncs += 1
                    st.notes.append(f"t={t} b={b} near-tie resync")
                    pos = o.resident_positions(b)
                    kk = torch.from_numpy(s.K[:, :, pos].copy()).to(w.torch_dtype).to(device).contiguous()
                    vv = torch.from_numpy(s.V[:, :, pos].copy()).to(w.torch_dtype).to(device).contiguous()
                    ctx.import_blocks(b, osc.astype(np.float32), otr.astype(np.int32), ores, kk, vv)
                    continue
                st.max_score_err = max(st.max_score_err, check_scores(gsc, osc, rtol, f"step {t} scores b={b}"))
                st.checked_seq_steps += 1
                if kv_every and (t % kv_every == 0 or t == follow[b]):
                    for h in range(w.n_kv_heads):
                        gpos = ctx.retained(b, h)
                        np.testing.assert_array_equal(np.sort(gpos), o.resident_positions(b),
                                                      err_msg=f"step {t} b={b} kvh={h} retained positions")
                        gk, gv = ctx.export_kv(b, h)
                        rk = torch.from_numpy(s.K[:, h, gpos].copy()).to(w.torch_dtype)
                        rv = torch.from_numpy(s.V[:, h, gpos].copy()).to(w.torch_dtype)
                        assert torch.equal(gk.cpu(), rk), f"step {t} K differs b={b} kvh={h}"
                        assert torch.equal(gv.cpu(), rv), f"step {t} V differs b={b} kvh={h}"
                        st.kv_checks += 1
            st.steps = t
            if sync_every and t % sync_every == 0:
                ctx.sync()
            if t == 1 or t % 16 == 0 or t == steps:
                log(f"[block] step {t}: out_err {st.max_out_err:.2e} score_err {st.max_score_err:.2e} "
                    f"resyncs {st.near_tie_resyncs} readmitted {st.readmitted} following {live} "
                    f"({time.time() - t_start:.1f}s)")
        ctx.sync()
    finally:
        pool.close()
        ctx.close()
    log(f"[block] {w.name}: {st.steps} steps, checked sequence-steps {st.checked_seq_steps}, near-tie "
        f"resyncs {st.near_tie_resyncs}, readmitted {st.readmitted}, K/V checks {st.kv_checks}")
    for n in st.notes:
        log(f"[block]   {n}")
    return st


# ---------------------------------------------------------------------------
# Host-offload tier of the block mode
# ---------------------------------------------------------------------------

def run_offload_twins(w, steps, capacity, *, fused=True, kv_every=4, device="cuda", prefetch=0,
                      min_score=0.0):
    """Two block contexts on the same inputs: `plain` (no pool) re-admits each
    epoch's heavy blocks with K/V regenerated from the seed, `off` (a host
    pool of `capacity` blocks) re-admits the same blocks from its pool.  Every
    step both must agree bit for bit (outputs, scores, clocks, residency,
    retained positions, exported K/V), and the pool's slot of every block
    must equal the oracle's HostOffloadPool fed with each selection's
    evictions.  Blocks no longer in the pool are refused by the offload
    re-admission and skipped by both.  prefetch > 0: `off` has that many
    device staging slots and, one step before each epoch starts, prefetches
    the heavy blocks it will re-admit (restored from the staged copies).
    min_score: evicted blocks scoring below it (the library's fp32 scores,
    compared in fp32) are dropped instead of offloaded."""
    import pytest
    import torch
    from decode_kv_cache_gqa_amd import kvev

    log(f"[offload] {w.name}: L={w.n_layers} batch={w.batch} L0={w.prefill_lens[:6]} steps={steps} "
        f"capacity={capacity} fused={fused}")
    ctxs = [kvev.context_for(w, max_steps=steps, offload_blocks=0),
            kvev.context_for(w, max_steps=steps, offload_blocks=capacity, prefetch_blocks=prefetch,
                             offload_min_score=min_score)]
    plain, off = ctxs
    pool = orc.HostOffloadPool(capacity)
    for b in range(w.batch):
        K, V = w.prefill_kv(b, device=device)
        lab = w.region_labels(b)
        for c in ctxs:
            c.prefill(b, K.contiguous(), V.contiguous(), lab)
            c.set_budget(b, w.block_budget(b))
        del K, V
    torch.cuda.synchronize()
    outs = [torch.empty((w.n_layers, w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=device)
            for _ in ctxs]
    stats = {"readmitted": 0, "refused": 0, "offloaded": 0, "dropped": 0, "prefetched": 0,
             "below_threshold": 0}

    def resident(c, b):
        return np.asarray(c.block_state(b)[2], dtype=bool)

    for t in range(1, steps + 1):
        if prefetch and t + 1 <= steps and _epoch_start(w, t + 1):
            # background copies of the next epoch's heavy blocks, overlapping this step
            e = w.epoch_of(t + 1)
            for b in range(w.batch):
                res = set(np.flatnonzero(resident(off, b)).tolist())
                tail = (w.prefill_lens[b] + t - 2) // 16
                ids = [j for j in w.heavy_blocks(b, e) if j not in res and j < tail and pool.slot((b, j)) >= 0]
                if ids:
                    off.prefetch_offloaded(b, ids[:prefetch])
                    stats["prefetched"] += len(ids[:prefetch])
        if _epoch_start(w, t):
            e = w.epoch_of(t)
            for b in range(w.batch):
                res = set(np.flatnonzero(resident(plain, b)).tolist())
                tail = (w.prefill_lens[b] + t - 2) // 16
                cand = [j for j in w.heavy_blocks(b, e) if j not in res and j < tail]
                ids = [j for j in cand if pool.slot((b, j)) >= 0]
                for j in cand:
                    if pool.slot((b, j)) < 0:
                        # dropped from the pool (or never offloaded): refused, state untouched
                        with pytest.raises(kvev.KvevError):
                            off.readmit_offloaded(b, [j])
                        stats["refused"] += 1
                        break
                if not ids:
                    continue
                Kr, Vr = block_rows(w, b, ids, device)
                plain.readmit(b, ids, Kr, Vr)
                off.readmit_offloaded(b, ids)
                for j in ids:
                    pool.readmit((b, j))
                stats["readmitted"] += len(ids)
        before = {b: resident(plain, b) for b in range(w.batch)}
        q, kn, vn = w.step_inputs(t, device=device)
        for c, o in zip(ctxs, outs):
            if fused:
                c.step(q, kn, vn, o)
            else:
                c.decode_step(q, kn, vn, o)
                c.evict()
        assert torch.equal(outs[0], outs[1]), f"step {t}: outputs differ"
        evicted = []
        for b in range(w.batch):
            sp, so = plain.block_state(b), off.block_state(b)
            for x, y, name in zip(sp, so, ("score", "clock", "resident")):
                np.testing.assert_array_equal(x, y, err_msg=f"step {t} b={b}: {name}")
            now = np.asarray(sp[2], dtype=bool)
            was = np.zeros_like(now)
            was[:len(before[b])] = before[b]
            for j in np.flatnonzero(was & ~now):
                if np.float32(so[0][j]) >= np.float32(min_score):
                    evicted.append((b, int(j)))
                else:
                    stats["below_threshold"] += 1
        pool.offload(evicted)
        stats["offloaded"] += min(capacity, len(evicted))
        stats["dropped"] += max(0, len(evicted) - capacity)
        for b in range(w.batch):
            got = off.offload_state(b)
            want = np.array([pool.slot((b, j)) for j in range(len(got))], dtype=np.int32)
            np.testing.assert_array_equal(got, want, err_msg=f"step {t} b={b}: pool slots")
            if kv_every and (t % kv_every == 0 or t == steps):
                for h in range(w.n_kv_heads):
                    np.testing.assert_array_equal(plain.retained(b, h), off.retained(b, h),
                                                  err_msg=f"step {t} b={b} kvh={h}: retained")
                    kp, vp = plain.export_kv(b, h)
                    ko, vo = off.export_kv(b, h)
                    assert torch.equal(kp, ko) and torch.equal(vp, vo), f"step {t} b={b} kvh={h}: K/V differ"
        if t == 1 or t % 16 == 0 or t == steps:
            log(f"[offload] step {t}: {stats}")
    for c in ctxs:
        c.sync()
        c.close()
    return stats


# ---------------------------------------------------------------------------
# Two-tier window mode (full precision / INT2 / evicted per layer)
# ---------------------------------------------------------------------------

def _tier_boundaries(S, tiers, cand):
    """The oracle's lowest full-precision and lowest INT2 candidate scores."""
    f = [S[w] for w in cand if tiers[w] == 0]
    q = [S[w] for w in cand if tiers[w] == 1]
    return [x for x in (min(f) if f else None, min(q) if q else None) if x is not None]


def run_tier_lockstep(w, steps, *, sample_layers=None, rtol=2e-3, device="cuda", fused=True,
                      kv_every=4, ledger_every=4, revival_gap=0, threads=None, sync_every=32):
    """Run `steps` decode + routing steps of tiered workload `w` on the GPU and
    the oracle (one oracle object per sampled layer, stepped in threads).
    revival_gap > 0: after every routing event each sampled layer's routing
    diagnostics must equal the oracle's, computed from the event's
    candidates and the library's own tiers (exact).  On an excused near tie
    the GPU imports the oracle's tiers and scores; the oracle is never
    changed."""
    import torch
    from decode_kv_cache_gqa_amd import kvev

    layers = list(range(w.n_layers)) if sample_layers is None else sorted(sample_layers)
    log(f"[tier] {w.name}: L={w.n_layers} L0={w.prefill_lens[0]} steps={steps} K_f={w.fp_windows} "
        f"K_q={w.int2_windows} sink={w.n_sink} recent={w.n_recent} layers={layers} fused={fused}")
    t_start = time.time()
    ctx = kvev.context_for(w, max_steps=steps, revival_gap=revival_gap)
    rdiag = {l: orc.RoutingDiagnostics(revival_gap) for l in layers} if revival_gap else None
    # 8-token windows, the rotary mode and per-token key groups read INT2
    # windows through their bf16 reconstruction, kept in the full-precision
    # storage
    mat = w.window_tokens == 8 or w.rope_theta > 0 or w.int2_key_groups == 1
    orcs = {l: orc.TieredOracle(w.n_layers, w.n_q_heads, w.n_kv_heads, w.head_dim, k_f=w.fp_windows,
                                k_q=w.int2_windows, window=w.window_tokens, n_sink=w.n_sink,
                                n_recent=w.n_recent, capacity=w.prefill_lens[0] + steps + 1,
                                route_interval=w.route_interval, rope_theta=w.rope_theta,
                                reconstruct_bf16=mat,
                                key_groups="token32" if w.int2_key_groups == 1 else "channel")
            for l in layers}
    W = w.window_tokens
    K, V = w.prefill_kv(0, device=device)
    ctx.prefill(0, K.contiguous(), V.contiguous())
    for l in layers:
        orcs[l].prefill(K[l:l + 1].float().cpu().numpy(), V[l:l + 1].float().cpu().numpy(), layers=[l])
    del K, V
    torch.cuda.synchronize()
    log(f"[tier] prefill done in {time.time() - t_start:.1f}s")
    pool = OracleThreads(len(layers), threads)
    o0 = orcs[layers[0]]  # window geometry and routing cadence (shared by every layer)
    st = Stats()
    st.ledger_checks = 0
    st.promotions = 0
    st.routing_events = 0
    Hg = w.group_size
    out = torch.empty((w.n_layers, 1, w.n_q_heads, w.head_dim), dtype=torch.float32, device=device)
    try:
        for t in range(1, steps + 1):
            # the library's tiers before this step's routing event
            gprev = {l: ctx.tier_state(l)[1] for l in layers} if rdiag else None
            q, kn, vn = w.step_inputs(t, device=device)
            if fused:
                ctx.step(q, kn, vn, out)
            else:
                ctx.decode_step(q, kn, vn, out)
            qc, knc, vnc = (x[:, 0].float().cpu().numpy() for x in (q, kn, vn))
            refs = dict(zip(layers, pool.map(
                lambda l: orcs[l].decode_step(t, qc[l:l + 1], knc[l:l + 1], vnc[l:l + 1]), layers)))
            gout = out.cpu().numpy()
            for l in layers:
                for h in range(w.n_kv_heads):
                    st.max_out_err = max(st.max_out_err, check_out(
                        gout[l, 0, h * Hg:(h + 1) * Hg], refs[l][0, h * Hg:(h + 1) * Hg], rtol,
                        f"step {t} out l={l} kvh={h}"))
            routes = o0.routes_after(t)
            if not fused:
                for l in layers:
                    gs, _, _ = ctx.tier_state(l)
                    os_, ot, _ = orcs[l].window_state(l)
                    live = ot != 2
                    st.max_score_err = max(st.max_score_err, check_scores(
                        gs[live], os_[live], rtol, f"step {t} pre-route scores l={l}"))
                if routes:
                    ctx.evict()
            prev = {l: orcs[l].window_state(l)[1] for l in layers}
            nw_pre = o0.n_windows()
            if routes:
                pool.map(lambda l: orcs[l].route(), layers)
                st.routing_events += 1
            for l in layers:
                o = orcs[l]
                gs, gt, gl = ctx.tier_state(l)
                os_, ot, ol = o.window_state(l)
                assert len(gt) == len(ot), f"step {t} l={l}: {len(gt)} windows on the GPU, {len(ot)} in the oracle"
                if rdiag and routes:
                    was = lambda x: gprev[l][x] if x < len(gprev[l]) else 0
                    cand = [x for x in range(nw_pre) if o.is_aged(x) and was(x) != 2]
                    exp = rdiag[l].observe(cand, gt)
                    got = ctx.tier_diag(l)
                    for k, v in exp.items():
                        assert got[k] == v, f"step {t} l={l}: routing diagnostic {k} {got[k]} != {v}"
                    for k, v in rdiag[l].sums.items():
                        assert abs(got[k] - v) <= 1e-12 * max(1.0, abs(v)), f"step {t} l={l}: {k} {got[k]!r} != {v!r}"
                    st.route_diag_checks = getattr(st, "route_diag_checks", 0) + 1
                st.promotions += int(((prev[l] == 1) & (ot == 0)).sum())
                if not np.array_equal(gt, ot) or not np.array_equal(gl, ol):
                    cand = [x for x in range(nw_pre) if o.is_aged(x) and prev[l][x] != 2]
                    thetas = _tier_boundaries(os_, ot, cand)
                    diff = np.flatnonzero((gt != ot) | (gl != ol)).tolist()
                    gaps, ths = [], []
                    for x in diff:
                        th = min(thetas, key=lambda v: abs(os_[x] - v))
                        gaps.append(abs(os_[x] - th))
                        ths.append(th)
                    worst = int(np.argmax(gaps))
                    assert near_tie_excused(gaps, ths[worst], rtol) and all(
                        near_tie_excused([g], th, rtol) for g, th in zip(gaps, ths)), (
                        f"step {t} l={l}: tiers differ at windows {diff[:8]} (gpu {gt[diff[:8]]}, oracle "
                        f"{ot[diff[:8]]}) with oracle score gap {max(gaps):.3e}")
                    st.near_tie_resyncs += 1
                    st.notes.append(f"t={t} l={l} near-tie resync ({len(diff)} windows, gap {max(gaps):.2e})")
                    ctx.tier_import(l, os_.astype(np.float32), ot)
                    continue
                st.max_score_err = max(st.max_score_err, check_scores(gs, os_, rtol, f"step {t} scores l={l}"))
                st.exact_selection_checks += 1
                if kv_every and (t % kv_every == 0 or t == 1 or t == steps):
                    lay = o.layers[l]
                    # full-precision windows (and, with bf16 reconstruction, INT2 windows, whose
                    # storage holds the reconstruction)
                    held = np.flatnonzero((ot == 0) | ((ot == 1) & mat))
                    rows = np.concatenate([np.arange(W * x, min(W * x + W, o.npos)) for x in held])
                    for h in range(w.n_kv_heads):
                        gk, gv = ctx.tier_export(l, h)
                        idx = torch.from_numpy(rows)
                        rk = torch.from_numpy(lay.K[h, rows].copy()).to(w.torch_dtype)
                        rv = torch.from_numpy(lay.V[h, rows].copy()).to(w.torch_dtype)
                        gkr = gk.cpu()[idx]
                        if w.rope_theta > 0 and not torch.equal(gkr, rk):
                            # rotated keys: the device's and numpy's fp64 sin / cos may differ in the
                            # last bit, which can move a bf16 rounding by one unit, rarely
                            d = (gkr.view(torch.int16).int() - rk.view(torch.int16).int()).abs()
                            nbad = int((d != 0).sum())
                            assert int(d.max()) == 1 and nbad <= max(2, rk.numel() // 100000), (
                                f"step {t} l={l} kvh={h}: rotated K differs in {nbad} elements (max {int(d.max())} ulp)")
                            st.rope_ulp = getattr(st, "rope_ulp", 0) + nbad
                        else:
                            assert torch.equal(gkr, rk), f"step {t} l={l} kvh={h}: full-precision K differs"
                        assert torch.equal(gv.cpu()[idx], rv), f"step {t} l={l} kvh={h}: full-precision V differs"
                        st.kv_checks += 1
                if ledger_every and (t % ledger_every == 0 or t == 1):
                    lay = o.layers[l]
                    wins = np.flatnonzero(ol)
                    if len(wins) > 24:
                        wins = wins[np.linspace(0, len(wins) - 1, 24).astype(int)]
                    for x in wins.tolist():
                        for h in range(w.n_kv_heads):
                            got = ctx.tier_ledger(l, h, x)
                            ref = lay.ledger[x][h]
                            for a, b, name in zip(got, ref, ("k_codes", "k_scale", "k_zero", "v_codes",
                                                               "v_scale", "v_zero")):
                                assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8)), (
                                    f"step {t} l={l} kvh={h} window {x}: ledger {name} differs")
                            st.ledger_checks += 1
            st.steps = t
            if sync_every and t % sync_every == 0:
                ctx.sync()
            if t == 1 or t % 16 == 0 or t == steps:
                log(f"[tier] step {t}: out_err {st.max_out_err:.2e} score_err {st.max_score_err:.2e} "
                    f"resyncs {st.near_tie_resyncs} promotions {st.promotions} ledger {st.ledger_checks} "
                    f"({time.time() - t_start:.1f}s)")
        ctx.sync()
    finally:
        pool.close()
        ctx.close()
    log(f"[tier] {w.name}: {st.steps} steps, {st.routing_events} routing events, near-tie resyncs "
        f"{st.near_tie_resyncs}, promotions {st.promotions}, ledger checks {st.ledger_checks}")
    for n in st.notes:
        log(f"[tier]   {n}")
    return st
