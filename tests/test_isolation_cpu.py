"""Structure of the product path, checked on the host: the library package and its C sources
never reach the oracle, the oracle never reaches the library, and every call of the Python
binding fails loudly when libmla.so is missing (there is no CPU fallback)."""
import ast
import glob
import importlib
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_latent_attention_wkv_amd")


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_package_does_not_import_the_oracle():
    for path in glob.glob(os.path.join(PKG, "**", "*.py"), recursive=True):
        assert "oracle" not in _imports(path), path


def test_oracle_does_not_import_the_package_or_torch_gpu_code():
    for path in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        imps = _imports(path)
        assert "sparse_latent_attention_wkv_amd" not in imps, path
        assert "torch" not in imps, path


def test_c_sources_do_not_include_oracle_code():
    for path in glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*")):
        text = open(path).read()
        assert not re.search(r'#include\s+"[^"]*oracle', text), path


def test_binding_raises_without_the_library(monkeypatch):
    mla = importlib.import_module("sparse_latent_attention_wkv_amd")
    monkeypatch.setattr(mla, "_lib", None)
    monkeypatch.setattr(mla, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libmla.so"))
    with pytest.raises(mla.MLAError):
        mla.lib()
    with pytest.raises(mla.MLAError):
        mla.mla_default_softmax_scale()
    with pytest.raises(mla.MLAError):
        mla.mla_attn_workspace_bytes(1, 64, 16)
