"""The HBM-traffic figures in profiles/hbm_traffic.json are reported by
bench.py only while the kernel code they were measured on is unchanged:
the hash covers the code of the kernel sources, not their comments."""

import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_comments_and_blank_lines_do_not_change_the_code():
    src = "int a = 1;  // one\n\n/* block\n comment */ int b = 2;   \n"
    assert bench._code_only(src) == "int a = 1;\n int b = 2;"
    assert bench._code_only(src.replace("// one", "// another")) == bench._code_only(src)


def test_code_changes_do_change_it():
    src = "int a = 1;  // one\n"
    assert bench._code_only(src) != bench._code_only(src.replace("1", "2"))

