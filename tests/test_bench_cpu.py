"""Host logic of bench.py on the CPU: the per-batch quantiles and the parity
gate of the cpu_baseline leg (the oracle's own output passes, a perturbed one
fails).  No GPU: the "GPU output" here is a CPU tensor."""

import numpy as np
import torch

import bench
import oracle.paged_attention as O
from paged_kv_cache_195_amd.workloads import make_workload


def test_quantile():
    v = [1.0, 2.0, 3.0, 4.0, 5.0]
    assert bench._quantile(v, 0.5) == 3.0
    assert bench._quantile(v, 0.0) == 1.0 and bench._quantile(v, 1.0) == 5.0
    assert abs(bench._quantile(v, 0.1) - 1.4) < 1e-12
    assert abs(bench._quantile(v, 0.9) - 4.6) < 1e-12
    assert bench._quantile([7.0], 0.9) == 7.0


def _oracle_out(w):
    xo, _ = O.attention(w.q.double().numpy(), w.k_cache.double().numpy(),
                        w.v_cache.double().numpy(), w.table_host.numpy(),
                        np.array(w.seq_lens_host), w.scale, w.causal)
    return torch.from_numpy(xo[:, 0]).float()


def test_cpu_baseline_parity_gate():
    w = make_workload("tiny_f32", device="cpu")
    out = _oracle_out(w)
    res = bench.cpu_baseline(w, out, budget_s=5.0, threads=2)
    assert res["parity"]["ok"] and res["parity"]["elements_out_of_tolerance"] == 0
    assert res["sample"].startswith("2 of 2 sequences") and res["cores"] == 2
    assert res["value"] > 0 and res["unit"] == "GB/s"
    # one element off by more than the f32 bar (1e-5 + 1e-5 |x|) fails the gate
    bad = out.clone()
    bad[1, 3, 17] += 1e-3
    res = bench.cpu_baseline(w, bad, budget_s=5.0, threads=2)
    assert not res["parity"]["ok"] and res["parity"]["elements_out_of_tolerance"] == 1
    assert abs(res["max_abs_err_vs_gpu"] - 1e-3) < 1e-6
