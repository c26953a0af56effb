"""Host logic of bench.py (no GPU): the source digest that ties counter-derived traffic to the
kernels it was measured on ignores comments and blank space, and nothing else."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_code_only_drops_comments_and_keeps_code():
    src = ('// header\n#include "a.hpp"  // trailing\n/* block\n comment */ int x = 1; /* inline */\n\n'
           'const char* s = "not // a comment /* either */";\nchar c = \'"\'; int y = 2;  // end\n')
    got = bench.code_only(src)
    assert got == ('#include "a.hpp"\nint x = 1;\n'
                   'const char* s = "not // a comment /* either */";\nchar c = \'"\'; int y = 2;')


def test_code_only_sees_code_changes():
    a = "int f() { return 1; }  // one\n"
    assert bench.code_only(a) == bench.code_only("// new note\nint f() {  return 1; }\n")
    assert bench.code_only(a) != bench.code_only("int f() { return 2; }  // one\n")
    assert bench.code_only('s = "x\\"//y";') == 's = "x\\"//y";'   # escaped quote inside a string


def test_source_digest_is_stable_and_per_call():
    d = {c: bench.source_digest(c) for c in ("compress", "index", "attend")}
    assert len(set(d.values())) == 3
    assert d == {c: bench.source_digest(c) for c in d}
