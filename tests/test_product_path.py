"""CPU checks that the product path has no way around the HIP library:

  * with the library missing, the binding raises instead of computing;
  * host (CPU) tensors are refused before any call reaches the library;
  * no module of the package imports the oracle (it is test infrastructure).
"""

import ast
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "token_routing_grouped_amd")


def test_missing_library_raises(tmp_path, monkeypatch):
    from token_routing_grouped_amd import _abi

    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "libtrg_moe.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(_abi.MoeError, match="not built"):
        _abi.lib()
    with pytest.raises(_abi.MoeError, match="not built"):
        _abi.moe_route_workspace_size(16, 8, 2)


@pytest.mark.skipif(not os.path.exists(os.path.join(PKG, "libtrg_moe.so")), reason="library not built")
def test_host_tensors_are_refused():
    from token_routing_grouped_amd import _abi

    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    pos = torch.zeros(4, 2, dtype=torch.int32)
    xp = torch.zeros(8, 64, dtype=torch.bfloat16)
    with pytest.raises(_abi.MoeError, match="expected the GPU"):
        _abi.moe_permute(x, pos, xp)
    with pytest.raises(_abi.MoeError, match="expected the GPU"):
        _abi.moe_unpermute_sum(xp, pos, x)


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield ("." * node.level) + (node.module or "")


def test_package_does_not_import_the_oracle():
    seen = []
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith(".py"):
                p = os.path.join(dirpath, f)
                seen.append(f)
                bad = [m for m in _imports(p) if m.split(".")[0] == "oracle" or m.startswith("..oracle")]
                assert not bad, (p, bad)
    assert "layer.py" in seen and "_abi.py" in seen
