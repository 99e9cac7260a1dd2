"""Host-side helpers of bench.py: the kernel-source hash that decides whether
the committed counter profiles still describe the code."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

CODE = '''#include "x.h"
// a line comment
int f(int a) {  /* a block
                   comment */
    const char* s = "a // not a comment /* nor this */";
    char c = '"';
    return a + 1;   // trailing
}
'''


def test_comments_and_blank_lines_do_not_count():
    edited = CODE.replace("// a line comment", "// another comment\n\n").replace("trailing", "other words")
    assert bench._strip_comments(edited) == bench._strip_comments(CODE)


def test_string_and_char_literals_are_kept():
    out = bench._strip_comments(CODE)
    assert '"a // not a comment /* nor this */"' in out
    assert "'\"'" in out
    assert "comment" not in out.replace("not a comment", "")


def test_code_changes_count():
    assert bench._strip_comments(CODE.replace("a + 1", "a + 2")) != bench._strip_comments(CODE)
    assert bench._strip_comments(CODE.replace('"a // not', '"b // not')) != bench._strip_comments(CODE)


def test_source_hash_is_stable():
    assert bench.source_hash() == bench.source_hash()
    assert len(bench.source_hash()) == 64
