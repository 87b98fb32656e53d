"""The kernel-sources digest that keys the committed traffic records (CPU
only): comments do not count, code, string literals and the build's flags do."""
import os
import shutil

import pytest

import bench


def test_strip_c_comments_keeps_code_and_literals():
    src = 'int a = 1; // one\n/* block\n comment */ const char* s = "// not a comment";\nchar c = \'/\';  \n\n'
    out = bench._strip_c_comments(src)
    assert "one" not in out and "block" not in out
    assert '"// not a comment"' in out and "'/'" in out
    assert out.splitlines() == ["int a = 1;", ' const char* s = "// not a comment";', "char c = '/';"]


def test_strip_c_comments_escaped_quote_in_literal():
    src = 'const char* s = "a\\"b // x"; // gone\n'
    assert bench._strip_c_comments(src) == 'const char* s = "a\\"b // x";'


@pytest.fixture()
def tree(tmp_path, monkeypatch):
    """A copy of the kernel sources, with bench's root pointed at it."""
    dst = tmp_path / "nvfp4_block_scaled_07_amd" / "csrc"
    shutil.copytree(os.path.join(bench.ROOT, "nvfp4_block_scaled_07_amd", "csrc"), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return dst


def test_digest_ignores_comments_but_not_code(tree):
    base = bench.kernel_sources_digest()
    f = tree / "gemm_tile.h"
    text = f.read_text()
    f.write_text("// an added comment line\n" + text.replace("namespace nvfp4 {", "namespace nvfp4 {  /* x */", 1))
    assert bench.kernel_sources_digest() == base
    f.write_text(text.replace("namespace nvfp4 {", "namespace nvfp4 {\nconstexpr int kUnused = 1;", 1))
    assert bench.kernel_sources_digest() != base


def test_digest_matches_the_committed_traffic_records():
    import json
    rec = os.path.join(bench.ROOT, "profiles", "traffic_large_n6144_k6144_m8192.json")
    if not os.path.exists(rec):
        pytest.skip("no committed record")
    assert json.load(open(rec))["sources_sha256_16"] == bench.kernel_sources_digest()
