import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build what is missing (only then): the C oracle and libmoe.so."""
    import importlib.util
    lib = os.path.join(ROOT, "bit_dequant_expert_router_amd", "libmoe.so")
    if not os.path.exists(lib):
        spec = importlib.util.spec_from_file_location(
            "_moe_build", os.path.join(ROOT, "bit_dequant_expert_router_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        import oracle
        oracle.build()


_ensure_built()


def pytest_terminal_summary(terminalreporter):
    """How many routings were near ties that the GPU resolved the other way
    (either selection is correct; their outputs were checked against the
    oracle run with the GPU's selection)."""
    import sys
    mod = sys.modules.get("_parity")
    if mod is not None:
        terminalreporter.write_line(f"near ties met: {len(mod.NEAR_TIES)} {mod.NEAR_TIES[:8]}")
