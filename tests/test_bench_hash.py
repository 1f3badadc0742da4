"""bench.py reports the committed HBM traffic only while the kernel sources'
code matches the sources the counters were taken on: a change to the code
changes the hash, a change to comments alone does not."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_comments_and_blank_lines_are_left_out():
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    b = "/* a block\n   comment */\nint f(int x) {\n\n    // a note\n    return x + 1;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)


def test_code_changes_are_seen():
    a = "int f(int x) {\n    return x + 1;\n}\n"
    b = "int f(int x) {\n    return x + 2;\n}\n"
    assert bench._code_only(a) != bench._code_only(b)


def test_every_workload_has_sources_and_a_hash():
    for wl, names in bench.KERNEL_SOURCES.items():
        assert names, wl
        h = bench.kernel_source_hash(wl)
        assert len(h) == 16 and int(h, 16) >= 0
