"""The kernel-source digest that ties committed rocprofv3 counter summaries to the code
they were taken on: comments and layout do not change it, code does."""
import os
import shutil
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_code_text_drops_comments_keeps_strings():
    src = 'int a = 1; // note\n/* block\n comment */ const char *s = "x // y /* z */";\n'
    assert bench.code_text(src) == 'int a = 1; const char *s = "x // y /* z */";'
    assert bench.code_text("a  =\n\tb;") == "a = b;"


def test_digest_ignores_comments_not_code(tmp_path):
    for f in sorted(os.listdir(bench.KERNEL_DIR)):
        if f.endswith((".hip", ".hpp")):
            shutil.copy(os.path.join(bench.KERNEL_DIR, f), tmp_path / f)
    base = bench.kernel_sources_digest(str(tmp_path))
    assert base == bench.kernel_sources_digest()
    name = sorted(f for f in os.listdir(tmp_path) if f.endswith(".hip"))[0]
    text = (tmp_path / name).read_text()
    (tmp_path / name).write_text("// a comment\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_sources_digest(str(tmp_path)) == base
    (tmp_path / name).write_text(text + "\nstatic int extra_symbol;\n")
    assert bench.kernel_sources_digest(str(tmp_path)) != base

