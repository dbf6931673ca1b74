import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (seconds to minutes)")


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is present; everything else runs anywhere.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def _install_oracle_mutant():
    """Swap in a mutated copy of the oracle (CPU only) when ORACLE_MUTANT is set.

    Used by test_oracle_mutants.py to check that the pins in test_oracle.py
    detect each planted slip; the oracle source on disk is never modified.
    """
    idx = os.environ.get("ORACLE_MUTANT")
    if idx is None:
        return
    import types
    from tests_mutants import MUTANTS  # noqa: E402
    old, new = MUTANTS[int(idx)][1:]
    path = os.path.join(ROOT, "oracle", "sdpa_oracle.py")
    src = open(path).read()
    assert old in src, "mutant %s no longer applies" % idx
    mod = types.ModuleType("oracle")
    mod.__file__ = path
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    sys.modules["oracle"] = mod


_install_oracle_mutant()
