"""Host-side logic of bench.py that needs no GPU."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_text_drops_comments_and_keeps_strings():
    src = 'int a = 1;  // note\n/* block\n   comment */\nasm("s_nop 0 // kept");\nchar c = \'/\';\n\n'
    assert bench.code_text(src) == 'int a = 1;\nasm("s_nop 0 // kept");\nchar c = \'/\';'


def test_source_digest_ignores_comment_edits_only(tmp_path):
    files = {"k.hip": "__global__ void k(int* p) { p[0] = 1; }  // store\n"}
    for n in bench.SHARED_HEADERS:
        files[n] = "#pragma once\n// shared\n"
    for n, t in files.items():
        (tmp_path / n).write_text(t)
    base = bench.sha256_of(str(tmp_path / "k.hip"))
    (tmp_path / "k.hip").write_text("// a kernel\n__global__ void k(int* p) { p[0] = 1; }  /* the store */\n")
    assert bench.sha256_of(str(tmp_path / "k.hip")) == base
    (tmp_path / "k.hip").write_text("__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.sha256_of(str(tmp_path / "k.hip")) != base
    (tmp_path / "k.hip").write_text(files["k.hip"])
    (tmp_path / bench.SHARED_HEADERS[0]).write_text("#pragma once\n#define X 1\n")
    assert bench.sha256_of(str(tmp_path / "k.hip")) != base
