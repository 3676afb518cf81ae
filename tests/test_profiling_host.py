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
    for name, (fragments, grid, summary, sources, workload) in profiling.KERNELS.items():
        assert all("k_" in f for f in fragments) and grid > 0 and summary.endswith("_traffic.txt")
        assert len(profiling.kernel_source_sha(name)) == 16
        assert workload in profiling.WORKLOADS


def test_kernel_grids_follow_the_plan():
    """The launch grid each summary keys on, recomputed from the library's
    plan (lla_prefill_segment_chunks) and the kernels' workgroup shapes."""
    import math
    import decode_lla_prefill_amd as lla
    import workloads

    def segments(name):
        c = workloads.CONFIGS[name]
        G = lla.prefill_segment_chunks(c.B, c.H, c.T, c.dk, c.dv, c.C)
        run_chunk = c.C if c.C <= 64 else (c.C + 1) // 2  # chunks over 64 tokens run as two
        return c, math.ceil(math.ceil(c.T / run_chunk) / G)

    c, n = segments("prefill_T8192")
    assert profiling.KERNELS["chunk_walk"][1] == c.B * c.H * n * 512       # one 8-wave group per segment
    assert profiling.KERNELS["chunk_walk_fp8"][1] == c.B * c.H * n * 512
    assert profiling.KERNELS["segment_states"][1] == c.B * c.H * (n - 1) * 512
    assert profiling.KERNELS["state_scan"][1] == c.B * c.H * math.ceil(c.dk * c.dv / 1024) * 256
    c, n = segments("prefill_B4_T1024")
    assert profiling.KERNELS["chunk_walk_T1024"][1] == c.B * c.H * n * 256  # four waves, d = 64: one value block
    c, n = segments("prefill_T131072")
    assert profiling.KERNELS["chunk_walk_T131072"][1] == c.B * c.H * n * 512
    c = workloads.CONFIGS["decode_B256"]
    assert profiling.KERNELS["decode_step"][1] == c.B * c.H * 512
    c = workloads.CONFIGS["decode_B256_gqa"]
    assert profiling.KERNELS["decode_group"][1] == c.B * c.kv_heads * 512
    # one persistent 8-wave workgroup per compute unit (2,048 states > 256)
    assert profiling.KERNELS["tokens_grouped"][1] == min(c.B * c.kv_heads, 256) * 512
    # the gated kernels: the plain wide ones' grids (the same plan)
    assert profiling.KERNELS["gated_walk"][1] == profiling.KERNELS["chunk_walk"][1]
    assert profiling.KERNELS["gated_segment_states"][1] == profiling.KERNELS["segment_states"][1]
    assert profiling.KERNELS["gated_decode"][1] == profiling.KERNELS["decode_step"][1]


def test_kernel_names_match_in_both_trace_forms():
    assert profiling.matches("_ZN3lla17k_chunk_walk_wideILi64EDF16bLb0EEEvPKT0_S3_S3_PfS4_PKfliiilliiS6_", "chunk_walk")
    assert profiling.matches("void lla::k_chunk_walk_wide<64, lla::fp8e4m3, false>(...)", "chunk_walk_fp8")
    assert not profiling.matches("void lla::k_chunk_walk_wide<64, lla::fp8e4m3, false>(...)", "chunk_walk")
    # the gated walk has the plain walk's grid: it must not be taken for it
    assert not profiling.matches("_ZN3lla17k_chunk_walk_wideILi64EDF16bLb1EEEvPKT0_S3_S3_PfS4_PKfliiilliiS6_",
                                 "chunk_walk")
    assert profiling.matches("lla::k_state_scan(float const*, float*, long, long, long, int)", "state_scan")
    assert not profiling.matches("_ZN3lla16k_decode_step_sqIDF16bLi128ELi512ELb1EEEvPKT_S3_S3_PfS4_PKf",
                                 "decode_step")
    assert profiling.matches("_ZN3lla16k_decode_step_sqIDF16bLi128ELi512ELb1EEEvPKT_S3_S3_PfS4_PKf",
                             "gated_decode")
    assert profiling.matches("_ZN3lla14k_decode_groupIDF16bLi128ELi512ELi16EEEvPKT_S3_S3_PfS4_i", "decode_group")
    assert profiling.matches("void lla::k_decode_group<__bf16, 128, 512, 16>(...)", "decode_group")
    # the general grouped kernel is another kernel
    assert not profiling.matches("void lla::k_decode_group_any<__bf16, 4, 16, 16>(...)", "decode_group")


def test_kernels_sharing_a_name_and_grid_are_measured_in_separate_runs():
    # the counters of a kernel are averaged over every dispatch of its name
    # at its grid, so two measured kernels that match each other's names at
    # the same grid must come from different runs
    keys = sorted(profiling.KERNELS)
    for i, a in enumerate(keys):
        for b in keys[i + 1:]:
            fa, ga, _, _, wa = profiling.KERNELS[a]
            fb, gb, _, _, wb = profiling.KERNELS[b]
            if ga != gb or wa == wb:
                continue
            clash = any(profiling.matches(f, b) for f in fa) or any(profiling.matches(f, a) for f in fb)
            if clash:
                assert (wa in profiling.DEFAULT_RUN) != (wb in profiling.DEFAULT_RUN), (a, b)
    assert set(profiling.DEFAULT_RUN) | set(profiling.RUN_ALONE) == set(profiling.WORKLOADS)
