import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# tests/test_sanitizers.py reruns host-only tests in a subprocess against an
# instrumented build (AddressSanitizer + UndefinedBehaviorSanitizer): these
# variables name that build, and the binding or the oracle is pointed at it
# before any test runs.
_SAN_LIB = os.environ.get("SSD_TEST_SANITIZED_LIB")
_SAN_ORACLE = os.environ.get("SSD_TEST_SANITIZED_ORACLE")
if _SAN_LIB:
    import ctypes

    import selective_state_space_04_amd as _ssd
    _ssd.lib = ctypes.CDLL(_SAN_LIB)
    _ssd.LIB_PATH = _SAN_LIB
    for _name, (_res, _args) in _ssd._SIGS.items():
        _f = getattr(_ssd.lib, _name)
        _f.restype, _f.argtypes = _res, _args
if _SAN_ORACLE:
    import oracle as _oracle
    _oracle._LIB_PATH = _SAN_ORACLE


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP path through the C ABI)")
    config.addinivalue_line("markers", "slow: long CPU-side oracle run")


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _has_gpu():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
