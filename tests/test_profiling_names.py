"""Kernel names as rocprofv3 reports them -> the names of the library's own
trace, which bench.py and the traffic summaries key on."""
from selective_recompute_attention_attn_amd import profiling


def test_demangled_names():
    assert profiling.short_name("void srat::(anonymous namespace)::attn_bwd_dq_kernel<128, true, false, false>"
                                "(srat::AttnParams)") == "attn_bwd_dq"
    assert profiling.short_name("void srat::(anonymous namespace)::attn_bwd_sums_kernel<128>"
                                "(srat::AttnParams, int, int, int)") == "attn_bwd_sums"


def test_two_group_kernels_report_under_the_library_trace_names():
    assert profiling.short_name("void srat::(anonymous namespace)::attn_fwd_pp_kernel<128, true, false, false>"
                                "(srat::AttnParams)") == "attn_fwd_bf16"
    assert profiling.short_name("void srat::(anonymous namespace)::attn_bwd_dq_pp_kernel<128, true, false, false>"
                                "(srat::AttnParams)") == "attn_bwd_dq"
    assert profiling.short_name("_ZN4srat12_GLOBAL__N_123attn_bwd_dkdv_pc_kernelILi128ELb1ELb0ELb1ELb0EEEvNS_10AttnParamsE"
                                ) == "attn_bwd_dkdv"


def test_mangled_names_with_bf16_arguments():
    full = "_ZN4srat12_GLOBAL__N_118sp_norm_fwd_kernelIDF16bLi512ELi2ELb1ELb0ELb1EEEvNS_13NormFwdParamsE"
    assert profiling.short_name(full) == "sp_norm_fwd"
    assert profiling.pretty_name(full) == "sp_norm_fwd_kernel<bf16, 512, 2, true, false, true>"


def test_other_kernels_unchanged():
    assert profiling.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_every_trace_name_has_sources():
    for k in set(profiling.KERNEL_SOURCES) | set(profiling.TRACE_ALIASES.values()):
        assert k in profiling.KERNEL_SOURCES
        assert len(profiling.src_hash(k)) == 16
