"""Host logic of bench.py that decides whether committed counter traffic still applies:
the digest covers the kernel source with its comments, blank lines and spacing removed,
so a comment edit keeps a measurement and any code edit retires it."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)

SRC = """// a header comment
#include <x.h>
/* a block
   comment */
__global__ void k(int* p) {   // trailing note
  p[0] = 1;

  p[1] = 2;  /* inline */
}
"""


def test_comments_and_spacing_do_not_change_the_code():
    edited = SRC.replace("a header comment", "another header comment").replace("trailing note", "x")
    edited = edited.replace("  p[0] = 1;", "      p[0]   =   1;").replace("\n\n", "\n\n\n")
    assert bench.kernel_source_code(edited) == bench.kernel_source_code(SRC)
    assert "comment" not in bench.kernel_source_code(SRC)


def test_a_code_change_changes_the_code():
    assert bench.kernel_source_code(SRC.replace("p[1] = 2", "p[1] = 3")) != bench.kernel_source_code(SRC)

