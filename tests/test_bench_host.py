"""Host-side checks of bench.py (no GPU): every global name it reads is
defined, and every committed counter profile it reads parses."""
import ast
import builtins
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_reads_only_defined_globals():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    bound = set(dir(builtins)) | {"__file__"}
    for n in ast.walk(tree):
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            bound.add(n.name)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            bound.update((a.asname or a.name).split(".")[0] for a in n.names)
        elif isinstance(n, ast.arg):
            bound.add(n.arg)
        elif isinstance(n, ast.ExceptHandler) and n.name:
            bound.add(n.name)
        elif isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
            bound.add(n.id)
    read = {n.id for n in ast.walk(tree) if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load)}
    assert read <= bound, f"bench.py reads undefined names: {sorted(read - bound)}"


def test_counter_profiles_parse():
    b = _bench()
    pairs = [(b.TRAFFIC_PROFILE, b.ATTN_SOURCES), (b.SEQ_TRAFFIC_PROFILE, b.SEQ_SOURCES),
             (b.TIER_TRAFFIC_PROFILE, b.TIER_SOURCES)]
    for profile, sources in pairs:
        assert os.path.exists(profile), profile
        for f in sources:
            assert os.path.exists(f), f
        v = b.measured_traffic(profile, sources)
        assert v is None or (isinstance(v, int) and v > 0)
