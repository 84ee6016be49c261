"""Static checks of the separation between the product path and the oracle:
the package never imports the oracle, the oracle never includes or imports
the package's sources or header, and the seeded input generators (shared by
both) import neither."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "post_quantization_layernorm_amd")


def _files(top, exts):
    for d, _, names in os.walk(top):
        if "_build" in d or "__pycache__" in d:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def test_package_never_imports_the_oracle():
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle\b)|liboracle|rptq_oracle", re.M)
    hits = [f for f in _files(PKG, (".py", ".hip", ".cpp", ".hpp", ".h")) if pat.search(open(f).read())]
    assert not hits, hits


def test_oracle_shares_no_source_with_the_package():
    py = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert not re.search(r"^\s*(import|from)\s+(post_quantization_layernorm_amd|synthetic)\b", py, re.M)
    assert "librptq" not in py
    cpp = open(os.path.join(ROOT, "oracle", "rptq_oracle.cpp")).read()
    inc = re.findall(r'#include\s+[<"]([^>"]+)[>"]', cpp)
    assert inc and all("/" not in h and not h.startswith("rptq") for h in inc), inc
    assert "librptq" not in cpp and "dlopen" not in cpp


def test_input_generators_hold_no_method_code():
    s = open(os.path.join(ROOT, "synthetic", "__init__.py")).read()
    assert not re.search(r"^\s*(import|from)\s+(oracle|post_quantization_layernorm_amd)", s, re.M)
