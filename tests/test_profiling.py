"""Host-side helpers that turn rocprofv3 output into the committed summaries."""
from post_weight_quantization_autoround_amd import profiling


def test_role_reads_the_epilogue_template_argument():
    dma = "void ar::gemm::gemm_bf16_dma_kernel<{}>(ar::GemmArgs)"
    assert profiling.role(dma.format("256, 256, 64, 4, 2, 2, 2, 1")) == "gemm_wgrad_ste_update"
    assert profiling.role(dma.format("256, 128, 64, 4, 2, 3, 1, 2")) == "gemm_fwd_loss"
    assert profiling.role(dma.format("128, 128, 64, 2, 2, 2, 0, 1")).startswith("gemm_store")
    assert profiling.role(dma.format("256, 256, 64, 4, 2, 2, 2, 1, true")) == "gemm_wgrad_ste_update"
    # the group-size specialisations add trailing template arguments
    assert profiling.role(dma.format("256, 256, 64, 4, 2, 2, 2, 1, true, false, false, false, 16, true")) == \
        "gemm_wgrad_ste_update"
    assert profiling.role(dma.format("256, 128, 64, 4, 2, 3, 1, 2, false, false, false, false, 0, false")) == \
        "gemm_fwd_loss"
    assert profiling.role("ar::(anonymous namespace)::transpose_b16_kernel(unsigned short const*)") == "transpose"
    assert profiling.role("void ar::(anonymous namespace)::attn_bwd_dkdv_kernel<128>(unsigned short const*)") == \
        "attn_bwd_dkdv"
    reg = "void ar::gemm::gemm_f32_kernel<128, 128, 32, 2, 2, {}>(ar::GemmArgs)"
    assert profiling.role(reg.format(1)) == "gemm_fwd_loss"
    assert profiling.role(reg.format(2)) == "gemm_wgrad_ste_update"
    assert profiling.role("ar::(anonymous namespace)::loss_decide_kernel(double const*)") == "loss_decide"
    assert profiling.role("void ar::(anonymous namespace)::w4a16_decode_kernel<false, true>(ar::W4A16Args)") == \
        "w4a16_gemm_decode"
    assert profiling.role("ar::(anonymous namespace)::rmsnorm_fwd_vec_kernel(unsigned short const*)") == "rmsnorm_fwd"
    assert profiling.role("ar::(anonymous namespace)::swiglu_bwd_vec_kernel(float const*)") == "swiglu_bwd"
    assert profiling.role("ar::(anonymous namespace)::yref_combine_vec_kernel(float const*)") == "loss_target"
    assert profiling.role("__amd_rocclr_copyBuffer") == ""


def test_bench_refuses_more_than_one_gpu():
    # the benchmark measures one GPU; any other count exits before touching a device
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
