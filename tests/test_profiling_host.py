"""Host-side checks of the counter bookkeeping (no GPU): the source digest
that ties a committed traffic summary to the kernel code it was measured on
ignores comments and layout but not code."""
from decode_lla_prefill_amd import profiling


def test_code_only_drops_comments_and_layout():
    src = 'int a = 1; // one\n/* two\n   lines */  int  b = "x // y /* z */";\nchar c = \'/\';'
    assert profiling.code_only(src) == 'int a = 1; int b = "x // y /* z */"; char c = \'/\';'
    assert profiling.code_only("a/*x*/b") == "a b"  # a comment separates tokens
    assert profiling.code_only('s = "\\"//";') == 's = "\\"//";'  # escaped quote inside a literal


def test_digest_changes_with_code_not_with_comments():
    base = "x += y;\n"
    assert profiling.code_only(base + "// note\n") == profiling.code_only(base)
    assert profiling.code_only(base + "x -= y;\n") != profiling.code_only(base)


def test_every_measured_kernel_names_its_sources():
    for name, (fragment, grid, summary, sources) in profiling.KERNELS.items():
        assert fragment.startswith("k_") and grid > 0 and summary.endswith("_traffic.txt")
        assert len(profiling.kernel_source_sha(name)) == 16
