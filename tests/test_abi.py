"""The HIP library loads on a machine without a GPU and exports every entry
point that include/moe.h declares; the binding fails loudly without it (CPU)."""
import ctypes
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"sizeof"})


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("moe_route", "moe_forward", "set_expert_table", "moe_create", "moe_destroy",
              "moe_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import __graft_entry__ as g
    path = os.path.join(ROOT, "bit_moe_expert_router_amd", "libmoe.so")
    if not os.path.exists(path):
        g.build_moe()
    lib = ctypes.CDLL(path)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_exports_match_header():
    import bit_moe_expert_router_amd as m
    assert sorted(m.EXPORTS) == _declared()
    for n in m.EXPORTS:
        assert callable(getattr(m, n))


def test_binding_constants_match_header():
    import bit_moe_expert_router_amd as m
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    defs = dict(re.findall(r"#define\s+(MOE_[A-Z_]+)\s+(\d+)", src))
    for n in ("MOE_WS_ERROR_OFFSET", "MOE_WS_COUNTER_BYTES", "MOE_ERR_ROUTING", "MOE_ERR_RANGE"):
        assert int(defs[n]) == getattr(m, n), n


def test_binding_refuses_missing_library(tmp_path, monkeypatch):
    import importlib
    import sys
    import pytest
    pkg_src = os.path.join(ROOT, "bit_moe_expert_router_amd")
    dst = tmp_path / "bit_moe_expert_router_amd"
    dst.mkdir()
    for f in ("__init__.py", "layer.py"):
        (dst / f).write_text(open(os.path.join(pkg_src, f)).read())
    monkeypatch.syspath_prepend(str(tmp_path))
    saved = {k: v for k, v in sys.modules.items() if k.startswith("bit_moe_expert_router_amd")}
    for k in saved:
        del sys.modules[k]
    try:
        with pytest.raises(RuntimeError, match="libmoe.so is missing"):
            importlib.import_module("bit_moe_expert_router_amd")
    finally:
        for k in list(sys.modules):
            if k.startswith("bit_moe_expert_router_amd"):
                del sys.modules[k]
        sys.modules.update(saved)


def test_host_side_argument_checks():
    """status codes that need no device: bad config, null arguments"""
    import bit_moe_expert_router_amd as m
    import pytest
    with pytest.raises(m.MoEError) as ei:
        m.moe_create(5120, 1536, 288, 8, 3, 64, 0, 0, 8)  # unsupported group
    assert ei.value.status == m.MOE_E_UNSUPPORTED
    with pytest.raises(m.MoEError) as ei:
        m.moe_create(5120, 1536, 288, 20, 3, 128, 0, 0, 8)  # top_k > 16
    assert ei.value.status == m.MOE_E_UNSUPPORTED
    with pytest.raises(m.MoEError) as ei:
        m.moe_create(5100, 1536, 288, 8, 3, 128, 0, 0, 8)  # hidden % 64
    assert ei.value.status == m.MOE_E_UNSUPPORTED
    assert m.lib.moe_workspace_bytes(None, 4) == 0
    assert m.lib.moe_route(None, None, 1, None, None, None, None, None, None, None, None, 0,
                           None) == m.MOE_E_ARG
