"""Host logic of the profile summaries: kernels of a traced training step are
mapped to the stages of the step in launch order (no GPU needed)."""
import csv

from sparse_mixture_experts_gate_amd import profile_summary as S

G = "void moe::gemm_bf16_kernel<{}>(moe::GemmParams)"
STEP = [  # one bf16 SwiGLU training step with the fused SGD, router logits split over K
    (G.format("2, false, false, 0, true, 256"), "router_logits"),
    ("moe::sum_partials_kernel(float const*, float*, long, int)", "router_logits"),
    ("moe::route_topk_kernel(moe::RouteArgs)", "route"),
    ("moe::expert_scan_kernel(moe::ScanArgs)", "route"),
    ("moe::slot_assign_kernel(moe::SlotArgs)", "route"),
    ("moe::finalize_kernel(moe::FinalizeArgs)", "route"),
    ("_ZN3moe13gather_kernelIDF16bLi8EEEvNS_10GatherArgsE", "gather"),
    (G.format("0, false, false, 3, false, 256"), "up_fwd"),
    (G.format("0, false, false, 0, false, 256"), "down_fwd"),
    ("_ZN3moe14combine_kernelIDF16bLb1ELi8EEEvNS_11CombineArgsE", "combine_loss"),
    ("moe::finalize_kernel(moe::FinalizeArgs)", "combine_loss"),
    ("_ZN3moe18combine_bwd_kernelIDF16bLi8EEEvNS_14CombineBwdArgsE", "combine_bwd"),
    (G.format("0, false, true, 4, false, 256"), "down_dgrad"),
    (G.format("1, true, true, 7, true, 256"), "down_wgrad"),
    (G.format("0, false, true, 0, false, 256"), "up_dgrad"),
    (G.format("1, true, true, 7, true, 128"), "up_wgrad"),
    ("_ZN3moe17router_bwd_kernelIDF16bEEvNS_13RouterBwdArgsE", "router_bwd"),
    (G.format("1, true, true, 0, true, 256"), "router_dwg"),
    ("moe::sum_partials_kernel(float const*, float*, long, int)", "router_dwg"),
    (G.format("2, false, true, 0, true, 256"), "router_dx"),
    ("_ZN3moe14scatter_kernelIDF16bLi8EEEvNS_11ScatterArgsE", "scatter"),
    ("_ZN3moe10sgd_kernelIDF16bEEvNS_7SgdArgsE", "sgd"),
]


def test_stage_of_one_step():
    state = {"stage": None, "wgrad": 0}
    for name, want in STEP:
        st = S._stage_of(name, state)
        assert st == want, (name, st, want)
        state["stage"] = st


def test_stage_of_mlp_step():
    """The bias + activation MLP: its down projection stores with a bias (epilogue 8), its
    bias gradients are column sums."""
    K = "void moe::kt64::gemm_bf16_kernel<{}>(moe::kt64::GemmParams)"
    step = [(G.format("2, false, false, 0, true, 256"), "router_logits"),
            ("moe::route_topk_kernel(moe::RouteArgs)", "route"),
            ("_ZN3moe13gather_kernelIDF16bLi8EEEvNS_10GatherArgsE", "gather"),
            (K.format("0, false, false, 3, false, 256"), "up_fwd"),
            (G.format("0, false, false, 8, false, 256"), "down_fwd"),
            ("_ZN3moe14combine_kernelIDF16bLb1ELi8EEEvNS_11CombineArgsE", "combine_loss"),
            ("_ZN3moe18combine_bwd_kernelIDF16bLi8EEEvNS_14CombineBwdArgsE", "combine_bwd"),
            (G.format("0, false, true, 6, false, 256"), "down_dgrad"),
            (G.format("1, true, true, 7, true, 256"), "down_wgrad"),
            (G.format("0, false, true, 0, false, 256"), "up_dgrad"),
            (G.format("1, true, true, 7, true, 128"), "up_wgrad"),
            ("_ZN3moe13colsum_kernelIDF16bEEvNS_10ColSumArgsE", "bias_grads")]
    state = {"stage": None, "wgrad": 0}
    for name, want in step:
        st = S._stage_of(name, state)
        assert st == want, (name, st, want)
        state["stage"] = st


def test_stage_durations_count_steps_at_the_router_gemm(tmp_path):
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        did, t = 0, 0
        wr.writerow([did, "void at::native::copy_kernel", t, t + 5])   # before the first step
        for step in range(3):
            for name, _ in STEP:
                did += 1
                wr.writerow([did, name, t, t + 1000])
                t += 2000
    steps, per = S.stage_durations(str(path))
    assert steps == 3
    assert per["router_logits"]["launches_per_step"] == 2      # the GEMM and the segment sum
    assert per["router_dwg"]["launches_per_step"] == 2
    assert per["route"]["launches_per_step"] == 4
    assert per["combine_loss"]["launches_per_step"] == 2
    assert all(abs(e["avg_launch_ms"] - 1e-3) < 1e-12 for e in per.values())
