"""The benchmark's work accounting, on the CPU: visible-pair counts from the
closed-form row intervals against a count of the oracle's visibility matrix,
and the per-workload pair counts the flop figures rest on."""
import pytest

import bench
from head_attention_attn_amd.inputs import WORKLOADS
from oracle import visible


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("sliding", 1),
                                         ("sliding", 7), ("sliding", 500), ("block", 1),
                                         ("block", 8), ("block", 48)])
@pytest.mark.parametrize("nq,nk", [(48, 48), (1, 1), (37, 100), (100, 37), (12, 48), (6, 96)])
def test_visible_pairs_match_the_oracle_mask(mask, window, nq, nk):
    if mask == "block" and (nk % window or nq % (nk // window)):
        pytest.skip("block-local needs Nk divisible by the window and Nq by the window count")
    assert bench.visible_pairs(mask, window, nq, nk) == int(visible(mask, window, nq, nk).sum())


def test_workload_pair_counts():
    """Per (batch, head) counts, by hand: 49 windows of 64^2; 196^2; the
    causal triangle N(N+1)/2; the sliding band sum of min(i+1, 1024)."""
    pc = {n: bench.visible_pairs(w.mask, w.window, w.Nq, w.Nk) for n, w in WORKLOADS.items()}
    assert pc["block_local_hiera"] == 49 * 64 * 64
    assert pc["block_pooled_hiera"] == 49 * 16 * 64
    assert pc["global_vision"] == 196 * 196
    assert pc["causal_lm"] == 8192 * 8193 // 2
    assert pc["sliding_pseudo_head"] == 1024 * 1025 // 2 + (4096 - 1024) * 1024
    assert pc["tiny_exact_fp32"] == 128 * 128


def test_kernel_work_sums_to_the_step():
    w = WORKLOADS["causal_lm"]
    pairs = bench.visible_pairs(w.mask, w.window, w.Nq, w.Nk)
    work = bench.kernel_work(w, pairs)
    fl = work["fwd"]["flops"] + work["dkdv"]["flops"] + work["dq"]["flops"]
    assert fl == 14 * w.d * pairs * w.B * w.H
    # block-local dK/dV pass: Q, dO, K, V, dK, dV in bf16 plus lse and D in fp32
    b = WORKLOADS["block_local_hiera"]
    rows = b.B * b.H * b.Nq
    assert bench.kernel_work(b, 49 * 64 * 64)["dkdv"]["bytes"] == rows * (6 * b.d * 2 + 8)


def test_more_than_one_gpu_is_refused(capsys):
    import sys
    argv = sys.argv
    sys.argv = ["bench.py", "--gpus", "2"]
    try:
        assert bench.main() == 2
    finally:
        sys.argv = argv
    assert "one GPU" in capsys.readouterr().err


def test_fused_backward_bytes():
    """Fused block-local backward: Q, dO, K, V read, dQ, dK, dV written (bf16)
    plus lse (fp32); 10 d flops per visible pair."""
    b = WORKLOADS["block_local_hiera"]
    rows = b.B * b.H * b.Nq
    wk = bench.kernel_work(b, 49 * 64 * 64)["bwd"]
    assert wk["bytes"] == rows * (7 * b.d * 2 + 4)
    assert wk["flops"] == 10 * b.d * 49 * 64 * 64 * b.B * b.H


def test_kept_ds_bytes():
    """With dS kept, the dK/dV pass writes 2 bytes per visible pair more and
    the dQ pass reads them back: workspace traffic of this library, reported
    apart; the compulsory bytes of both passes stay the method's."""
    w = WORKLOADS["causal_lm"]
    pairs = bench.visible_pairs(w.mask, w.window, w.Nq, w.Nk) * w.B * w.H
    rows = w.B * w.H * w.Nq
    plain = bench.kernel_work(w, pairs // (w.B * w.H))
    kept = bench.kernel_work(w, pairs // (w.B * w.H), kept_ds=True)
    for kn in ("dkdv", "dq"):
        assert kept[kn]["bytes"] == plain[kn]["bytes"]
        assert kept[kn]["flops"] == plain[kn]["flops"]
        assert plain[kn]["workspace_bytes"] == 0
        assert kept[kn]["workspace_bytes"] == 2 * pairs
    # dQ step: reads Q, dO (and K, V) and the row statistics, writes dQ
    assert plain["dq"]["bytes"] == rows * (5 * w.d * 2 + 8)


@pytest.mark.parametrize("name,bound,mbytes,gflops", [
    ("tiny_exact_fp32", "latency", 0.79, 0.0294),
    ("block_local_hiera", "hbm", 928.1, 34.5),
    ("global_vision", "hbm", 232.0, 26.4),
    ("causal_lm", "mfma", 504.6, 1203.0),
    ("sliding_pseudo_head", "mfma", 1009.0, 526.0),
])
def test_step_bound_per_config(name, bound, mbytes, gflops):
    """The step's compulsory bytes, flops and bound class of each benchmark
    configuration, against the figures worked out by hand from the shapes
    (forward reads Q, K, V and writes O, lse; backward reads Q, K, V, O, dO,
    lse and writes dQ, dK, dV; 14 d flops per visible pair; ridge point
    2.5 PFLOP/s over 8 TB/s)."""
    w = WORKLOADS[name]
    sw = bench.step_work(w, bench.visible_pairs(w.mask, w.window, w.Nq, w.Nk))
    assert sw["bound"] == bound
    assert abs(sw["bytes"] / 1e6 - mbytes) / mbytes < 2e-3
    assert abs(sw["flops"] / 1e9 - gflops) / gflops < 3e-3


def test_configs_cover_the_benchmark():
    assert bench.CONFIGS == ("tiny_exact_fp32", "block_local_hiera", "global_vision", "causal_lm",
                             "sliding_pseudo_head")
    assert all(c in WORKLOADS for c in bench.CONFIGS)


def test_kernel_roofline_by_bound():
    wk = {"flops": 2.5e12, "bytes": 8e9}
    mf = bench.kernel_roofline(wk, "mfma", 2500.0, 2.0)   # 2.5e12 flop in 2 ms
    assert mf["unit"] == "TFLOP/s" and mf["frac"] == 0.5
    hb = bench.kernel_roofline(wk, "hbm", 2500.0, 2.0)    # 8 GB in 2 ms
    assert hb["unit"] == "GB/s" and hb["frac"] == 0.5
    assert bench.kernel_roofline(wk, "latency", 2500.0, 2.0) is None


def test_host_cores_is_the_affinity_set():
    import os
    assert bench.host_cores() == len(os.sched_getaffinity(0))


def test_iha_workload_accounting():
    """The IHA workload: 20 heads, 8192 tokens x 4 pseudo-heads = 32768
    pseudo-tokens, a causal window of 1024 pseudo-tokens (the pages' N = 8192
    row: WSL = N / (2P) - 1 = 1023); the premix moves, per Q/K/V tensor, the
    [B, N, H, d] input and the P times larger pseudo-token output."""
    w = WORKLOADS["iha_joint"]
    N = w.Nq // w.P
    assert (w.H, N, w.P, w.window, w.Nq) == (20, 8192, 4, 1024, 32768)
    assert w.window == N // (2 * w.P)
    pairs = bench.visible_pairs(w.mask, w.window, w.Nq, w.Nk)
    assert pairs == 32768 * 1024 - 1024 * 1023 // 2
    work = bench.kernel_work(w, pairs)
    x = N * 20 * 128
    assert work["premix"]["bytes"] == 3 * 2 * (x + 4 * x + 20 * 4 * 20)
    assert work["premix"]["flops"] == 3 * 2 * 20 * (4 * x)
    assert "premix" not in bench.kernel_work(WORKLOADS["causal_lm"], 1)


def test_step_spread_percentiles():
    """p10 / median / p90 of the step and per-kernel times from events
    recorded before a step and after each of its kernels."""
    class Ev:
        def __init__(self, t):
            self.t = t

        def elapsed_time(self, other):
            return other.t - self.t

    # step s: fwd takes 1 + s ms, bwd 2 ms; steps 0..10
    events = [[Ev(100.0 * s), Ev(100.0 * s + 1 + s), Ev(100.0 * s + 3 + s)] for s in range(11)]
    rec = bench.step_spread(events, ("fwd", "bwd"))
    assert rec["per_kernel_ms"]["fwd"] == {"p10": 2.0, "median": 6.0, "p90": 10.0}
    assert rec["per_kernel_ms"]["bwd"] == {"p10": 2.0, "median": 2.0, "p90": 2.0}
    assert rec["ms_per_step"] == {"p10": 4.0, "median": 8.0, "p90": 12.0}


def test_stored_profiles_follow_the_sources(tmp_path, monkeypatch):
    """Counter readings stored under profiles/ are used only while their
    recorded source digest matches the kernel sources; otherwise the bench
    reports null."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    digest = bench.source_digest()
    (prof / "traffic_w.txt").write_text(
        f"# header\nsource_sha256: {digest}\ntraffic_bytes_per_launch.bwd: 123.0\n")
    (prof / "mfma_w.txt").write_text(
        f"# header\nsource_sha256: {digest}\nkernel dur_us clock_GHz\nbwd 64.5 2.48\nfwd 25.0 -\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: digest)
    assert bench.stored_traffic("w", "bwd") == 123.0
    assert bench.stored_clock("w", "bwd") == 2.48
    assert bench.stored_clock("w", "fwd") is None          # too short to time
    assert bench.stored_traffic("w", "fwd") is None
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 64)
    assert bench.stored_traffic("w", "bwd") is None
    assert bench.stored_clock("w", "bwd") is None
    assert bench.stored_clock("missing", "bwd") is None
