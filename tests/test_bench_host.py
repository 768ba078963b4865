"""Host-side checks of bench.py's bookkeeping (no GPU): the kernel-source hash that decides
whether stored counter readings still apply ignores comments and follows every code change."""
import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    argv = sys.argv
    try:
        sys.argv = ["bench.py"]
        spec.loader.exec_module(mod)
    finally:
        sys.argv = argv
    return mod


def test_strip_comments_keeps_code_and_literals():
    b = _bench()
    src = ('int a = 1; // trailing\n'
           '/* block\n comment */ int b = 2;\n'
           '\n'
           'const char* s = "not // a comment /* either */";\n'
           "char c = '/'; char d = '\\\\'; // after an escaped backslash\n"
           'asm volatile("s_nop 7\\n\\ts_nop 7");\n')
    out = b.strip_comments(src)
    assert "trailing" not in out and "block" not in out and "after an" not in out
    assert "int a = 1;" in out and "int b = 2;" in out
    assert '"not // a comment /* either */"' in out
    assert "char c = '/'; char d = '\\\\';" in out
    assert 's_nop 7\\n\\ts_nop 7' in out
    assert "\n\n" not in out


def test_strip_comments_sees_code_changes_only():
    b = _bench()
    base = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    assert b.strip_comments(base) == b.strip_comments(base.replace("add one", "increment"))
    assert b.strip_comments(base) != b.strip_comments(base.replace("x + 1", "x + 2"))
