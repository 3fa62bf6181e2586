"""The oracle and the HIP path share no code (CPU only, source scan)."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "sparse_attention_decode_page_amd"


def _sources(sub, exts):
    for dp, _, fs in os.walk(os.path.join(ROOT, sub)):
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(dp, f)


def test_oracle_imports_nothing_from_the_package():
    for path in _sources("oracle", (".py", ".c", ".h")):
        text = open(path).read()
        assert PKG not in text, path
        assert "csrc" not in text and "libspdec" not in text and "ctypes" not in text, path


def test_product_path_never_touches_the_oracle():
    pat = re.compile(r"^\s*(from|import)\s+oracle\b|oracle/|oracle\.", re.M)
    for path in _sources(PKG, (".py", ".hip", ".cpp", ".h")):
        assert not pat.search(open(path).read()), path
    for path in _sources("include", (".h",)):
        assert "oracle" not in open(path).read(), path
