import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    # short tracebacks: a failure report must not print device tensors (their repr runs
    # GPU work in a process whose device state may be what failed)
    if config.option.tbstyle == "auto":
        config.option.tbstyle = "short"
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test, skipped unless SPD_SLOW=1")


def pytest_collection_modifyitems(config, items):
    # a test module may declare deselect(item): parameter combinations it does not run
    kept, dropped = [], []
    for it in items:
        fn = getattr(it.module, "deselect", None) if getattr(it, "module", None) else None
        (dropped if fn is not None and fn(it) else kept).append(it)
    if dropped:
        config.hook.pytest_deselected(items=dropped)
        items[:] = kept
    if os.environ.get("SPD_SLOW") == "1":
        return
    skip = pytest.mark.skip(reason="slow CPU test; set SPD_SLOW=1")
    for it in items:
        if "slow" in it.keywords:
            it.add_marker(skip)


_cache = {}


def workload(name):
    """(cfg, weights, prompt) for a named workload, drawn once per session."""
    if name not in _cache:
        from spd_inputs import get, make_weights, make_prompt
        cfg = get(name)
        _cache[name] = (cfg, make_weights(cfg), make_prompt(cfg))
    return _cache[name]
