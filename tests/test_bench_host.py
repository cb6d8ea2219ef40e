"""Host logic of bench.py (no GPU): the kernel-code hash that ties the
committed traffic counters to the kernel they were taken on."""
import bench


def test_kernel_code_drops_comments_and_whitespace():
    src = "int a; // note\nint /* block\n comment */ b;\n\n  int   c;  /* x */"
    assert bench.kernel_code(src) == "int a; int b; int c;"


def test_kernel_code_keeps_code_changes():
    assert bench.kernel_code("x = a + b; // c") != bench.kernel_code("x = a - b; // c")


def test_kernel_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
