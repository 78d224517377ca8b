"""The cpu_baseline leg of bench.py compares the GPU outputs of the timed run
with the oracle head by head. Host-side check of that comparison: the oracle's
own outputs rounded to bf16 are within the bar, and a planted offset in one
tensor is reported outside it."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bench  # noqa: E402
import oracle  # noqa: E402
from workloads import Workload, make_inputs  # noqa: E402


def _outputs(w):
    vals = {k: v[1] for k, v in make_inputs(w, with_grad=True).items()}
    o, lse = oracle.forward(vals["q"], vals["k"], vals["v"], w.scale, w.causal, w.dropout_p, w.dropout_seed)
    dq, dk, dv, _ = oracle.backward(vals["q"], vals["k"], vals["v"], vals["do"], w.scale, w.causal,
                                    w.dropout_p, w.dropout_seed)
    bf = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)  # noqa: E731
    return {"O": bf(o), "LSE": torch.from_numpy(lse.astype(np.float32)), "dQ": bf(dq), "dK": bf(dk),
            "dV": bf(dv)}


W = Workload(90, "bf16_B1_H2_N96_d64_causal_dropout_test", 1, 2, 96, 64, "bf16", True, 0.1, True)


def test_parity_of_rounded_oracle_outputs_is_within_the_bar():
    r = bench.cpu_baseline(W, 0.0, _outputs(W))  # 0 s: one head
    par = r["parity"]
    assert par["heads"] == 1 and par["within"]
    assert set(par["tensors"]) == {"O", "LSE", "dQ", "dK", "dV"}
    assert par["tensors"]["LSE"]["max_abs"] < 1e-5
    assert 0 < par["tensors"]["O"]["max_abs"] <= 2e-2


def test_planted_offset_is_reported():
    out = _outputs(W)
    out["dV"] = out["dV"] + 0.05
    par = bench.cpu_baseline(W, 0.0, out)["parity"]
    assert not par["within"]
    assert par["tensors"]["dV"]["max_abs"] > 0.04
