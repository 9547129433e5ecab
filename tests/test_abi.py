"""The C-ABI library loads, exports every declared symbol, and its host-side
validation rejects bad configurations (no GPU calls are made here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from decode_kv_cache_gqa_amd import kvev

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvev.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvev_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("kvev_create", "kvev_decode_step", "kvev_scores", "kvev_evict",
                     "kvev_destroy", "kvev_prefill", "kvev_last_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = kvev.lib()
    for name in _declared():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", kvev.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (kvev_\w+)", out))
    assert set(_declared()) <= exported


def test_config_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    fields = [f for f, _ in kvev.Config._fields_]
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(kvev_config, {f}));' for f in fields)
    src.write_text(f'#include <stdio.h>\n#include <stddef.h>\n#include "kvev.h"\n'
                   f'int main(void) {{\n{body}\n  printf("size %zu\\n", sizeof(kvev_config));\n'
                   f'  return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(kvev.Config, f).offset, f
    assert int(got["size"]) == ctypes.sizeof(kvev.Config)


def _create(**kw):
    base = dict(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=64, batch=1, dtype=kvev.F32,
                max_tokens=100, budget=10)
    base.update(kw)
    cfg = kvev.make_config(**base)
    h = ctypes.c_void_p()
    st = kvev.lib().kvev_create(ctypes.byref(cfg), None, ctypes.byref(h))
    return st, kvev.lib().kvev_last_error(None).decode(), h


@pytest.mark.parametrize("bad,msg", [
    (dict(head_dim=96), "head_dim"),
    (dict(n_q_heads=7), "multiple"),
    (dict(n_q_heads=18), "group size"),
    (dict(n_q_heads=4, n_kv_heads=2, policy=kvev.LRFU_BLOCK), "group size must be 4"),
    (dict(n_q_heads=16, n_kv_heads=2, policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128),
     "group size must be 4"),
    (dict(scorer=4), "scorer"),
    (dict(granularity=2), "granularity"),
    (dict(policy=kvev.LRFU_BLOCK, scorer=kvev.SCORE_VNORM), "token policies"),
    (dict(n_layers=64, n_q_heads=16, max_tokens=1 << 20), "max_tokens too large"),
    (dict(n_layers=64, n_q_heads=64, n_kv_heads=8, granularity=kvev.PER_SEQUENCE, max_tokens=4096),
     "per-sequence granularity"),
    (dict(budget=0), "budget"),
    (dict(n_sink=8, n_recent=4), "exceeds the budget"),
    (dict(page_tokens=32), "page_tokens"),
    (dict(alpha_new=0.0), "alpha_new"),
    (dict(alpha_new=1.5), "alpha_new"),
    (dict(refresh_interval=0), "refresh_interval"),
    (dict(dtype=7), "dtype"),
    (dict(max_tokens=1), "max_tokens"),
    (dict(batch=0), ">= 1"),
    (dict(policy=9), "policy"),
    (dict(policy=kvev.LRFU_BLOCK, max_tokens=70000), "65536"),
    (dict(policy=kvev.LRFU_BLOCK, n_sink=4), "n_sink"),
    (dict(policy=kvev.LRFU_BLOCK, refresh_interval=4), "refresh_interval"),
    (dict(policy=kvev.LRFU_BLOCK, beta=-1.0), "beta"),
    (dict(policy=kvev.LRFU_BLOCK, decode_region=8), "decode_region"),
    (dict(policy=kvev.LRFU_BLOCK, decode_region=0, pinned_region_mask=1), "pinned"),
    (dict(policy=kvev.LRFU_BLOCK, pinned_region_mask=0x100), "mask"),
    (dict(policy=kvev.LRFU_BLOCK, access_tau_mult=0.0), "access_tau_mult"),
    (dict(policy=kvev.LRFU_BLOCK, budget=5000), "4096"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.F32, head_dim=128), "bf16"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=64), "head_dim 128"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, batch=2), "batch"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, window_tokens=16), "window_tokens"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, fp_windows=-1), "capacities"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, max_tokens=400000), "12288 windows"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, window_tokens=8, max_tokens=100000),
     "12288 windows"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, rope_theta=-1.0), "rope_theta"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, rope_theta=float("inf")), "rope_theta"),
    (dict(rope_theta=10000.0), "rope_theta applies to the tiered mode only"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, int2_key_groups=2), "int2_key_groups must be 0 or 1"),
    (dict(int2_key_groups=1), "int2_key_groups applies to the tiered mode only"),
    (dict(new_token_init=2), "new_token_init must be 0 or 1"),
    (dict(policy=kvev.LRFU_BLOCK, dtype=kvev.BF16, head_dim=128, new_token_init=1),
     "new_token_init applies to the token policies only"),
    (dict(policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, refresh_interval=2), "refresh_interval"),
    (dict(diag_topk=-1), "diag_topk"),
    (dict(offload_blocks=-1), "offload_blocks"),
    (dict(revival_gap=-1), "revival_gap"),
    (dict(prefetch_blocks=-1), "prefetch_blocks"),
    (dict(policy=kvev.LRFU_BLOCK, offload_blocks=4, offload_min_score=float("nan")), "offload_min_score"),
    (dict(policy=kvev.LRFU_BLOCK, prefetch_blocks=4), "needs the host-offload tier"),
    (dict(revival_gap=4), "tiered mode only"),
    (dict(offload_blocks=8), "block mode only"),
    (dict(diag_topk=4, policy=kvev.LRFU_BLOCK, n_q_heads=8), "token policies"),
    (dict(diag_topk=4, policy=kvev.TIERED_INT2, dtype=kvev.BF16, head_dim=128, batch=1), "token policies"),
    (dict(diag_topk=4, granularity=kvev.PER_SEQUENCE), "diagnostics need"),
    (dict(diag_topk=4, refresh_interval=8), "diagnostics need"),
    (dict(diag_topk=4, score_free=1), "diagnostics need"),
])
def test_create_rejects_bad_config(bad, msg):
    st, err, h = _create(**bad)
    assert st == kvev.EINVAL
    assert msg in err
    assert not h.value


def test_diag_group_struct_layout_matches_c(tmp_path):
    src = tmp_path / "diag_layout.c"
    fields = [f for f, _ in kvev.DiagGroup._fields_]
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(kvev_diag_group, {f}));' for f in fields)
    src.write_text(f'#include <stdio.h>\n#include <stddef.h>\n#include "kvev.h"\n'
                   f'int main(void) {{\n{body}\n  printf("size %zu\\n", sizeof(kvev_diag_group));\n'
                   f'  return 0;\n}}\n')
    exe = tmp_path / "diag_layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(kvev.DiagGroup, f).offset, f
    assert int(got["size"]) == ctypes.sizeof(kvev.DiagGroup)


def test_route_diag_struct_layout_matches_c(tmp_path):
    src = tmp_path / "route_layout.c"
    fields = [f for f, _ in kvev.RouteDiag._fields_]
    body = "\n".join(f'  printf("{f} %zu\\n", offsetof(kvev_route_diag, {f}));' for f in fields)
    src.write_text(f'#include <stdio.h>\n#include <stddef.h>\n#include "kvev.h"\n'
                   f'int main(void) {{\n{body}\n  printf("size %zu\\n", sizeof(kvev_route_diag));\n'
                   f'  return 0;\n}}\n')
    exe = tmp_path / "route_layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    for f in fields:
        assert int(got[f]) == getattr(kvev.RouteDiag, f).offset, f
    assert int(got["size"]) == ctypes.sizeof(kvev.RouteDiag)


def test_diag_entry_points_reject_null_context():
    L = kvev.lib()
    assert L.kvev_diag_read(None, None, 1) == kvev.EINVAL
    assert L.kvev_diag_trace(None, 0, 0, None, None, None, 0, None) == kvev.EINVAL
    assert L.kvev_diag_fmm(None, None, None) == kvev.EINVAL
    assert L.kvev_readmit_offloaded(None, 0, 1, None) == kvev.EINVAL
    assert L.kvev_offload_state(None, 0, None, 0, None) == kvev.EINVAL
    assert L.kvev_tier_diag(None, 0, None) == kvev.EINVAL
    assert L.kvev_prefetch_offloaded(None, 0, 1, None) == kvev.EINVAL


def test_null_arguments():
    L = kvev.lib()
    assert L.kvev_create(None, None, None) == kvev.EINVAL
    assert L.kvev_destroy(None) == kvev.OK
    assert L.kvev_evict(None, 5) == kvev.EINVAL
    assert L.kvev_decode_step(None, None, None, None, None) == kvev.EINVAL
    assert L.kvev_step_index(None) == -1


def test_config_defaults():
    c = kvev.config_init()
    assert c.page_tokens == 16 and c.refresh_interval == 1 and c.policy == kvev.EMA
    assert abs(c.alpha_new - 0.05) < 1e-7
    assert abs(c.beta - 0.001) < 1e-9 and c.decode_region == 4 and c.access_tau_mult == 2.0
    assert c.pinned_region_mask == 0 and list(c.region_half_life) == [0.0] * 8
    assert c.window_tokens == 32 and c.fp_windows == 0 and c.int2_windows == 0 and c.rope_theta == 0.0
    assert c.int2_key_groups == 0 and c.new_token_init == 0


def test_tier_entry_points_reject_null_context():
    L = kvev.lib()
    assert L.kvev_tier_state(None, 0, None, None, None, 0, None) == kvev.EINVAL
    assert L.kvev_tier_export(None, 0, 0, None, None, 0, None) == kvev.EINVAL
    assert L.kvev_tier_ledger(None, 0, 0, 0, None, None, None, None, None, None) == kvev.EINVAL
    assert L.kvev_tier_import(None, 0, 0, None, None) == kvev.EINVAL
    assert L.kvev_tier_footprint(None, None, None, None, None, None) == kvev.EINVAL


def test_block_entry_points_reject_null_context():
    L = kvev.lib()
    assert L.kvev_set_budget(None, 0, 5) == kvev.EINVAL
    assert L.kvev_readmit(None, 0, 1, None, None, None) == kvev.EINVAL
    assert L.kvev_block_state(None, 0, None, None, None, 0, None) == kvev.EINVAL
    assert L.kvev_import_blocks(None, 0, 1, None, None, None, 0, None, None) == kvev.EINVAL


def test_tier_capacities_match_the_worked_example_and_the_oracle():
    """kvev_tier_capacities is host arithmetic ("QEvict" review, section 4.3
    Eq.3): the review's worked example (B_hist = 100 MB, q = 0.70, 1 MB and
    0.131 MB windows give 30 and 534) and the oracle's function agree."""
    import oracle as orc
    MB = 1024 * 1024
    assert kvev.tier_capacities(100 * MB, 0.70, MB, 0.131 * MB) == (30, 534)
    rng = np.random.default_rng(3)
    for _ in range(200):
        b, q = float(rng.uniform(0, 1e10)), float(rng.uniform(0, 1))
        mf, mq = float(rng.uniform(1e3, 1e7)), float(rng.uniform(1e2, 1e6))
        assert kvev.tier_capacities(b, q, mf, mq) == orc.tier_capacities(b, q, mf, mq)
    for bad in [(1.0, 1.5, 1.0, 1.0), (1.0, -0.1, 1.0, 1.0), (-1.0, 0.5, 1.0, 1.0),
                (1.0, 0.5, 0.0, 1.0), (1.0, 0.5, 1.0, float("nan")), (1e12, 0.5, 1.0, 1.0)]:
        with pytest.raises(kvev.KvevError):
            kvev.tier_capacities(*bad)
