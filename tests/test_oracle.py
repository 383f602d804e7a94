"""The CPU oracle against its pins (no GPU needed)."""

import json
import os

import numpy as np
import pytest

import oracle
from linear_attention_recurrence_forward_amd.workloads import WORKLOADS, make_inputs

from pins import ALL_PINS, GOLDEN, assert_within


@pytest.fixture(scope="module", autouse=True)
def built_oracle():
    oracle.build(force=False)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.reference)


def test_capture_size_golden():
    """The capture buffer of the pages' memory-cost example is 2 MB per call."""
    with open(os.path.join(GOLDEN, "capture_size.json")) as f:
        fx = json.load(f)
    s = fx["shape"]
    rng = np.random.default_rng(0)
    S, T, Hk, Hv, Dk, Dv = (s["n_seqs"], s["n_tokens"], s["n_k_heads"],
                            s["n_v_heads"], s["d_k"], s["d_v"])
    x = dict(q=rng.standard_normal((S, T, Hk, Dk)), k=rng.standard_normal((S, T, Hk, Dk)),
             v=rng.standard_normal((S, T, Hv, Dv)), g=np.zeros((S, T, Hv)),
             beta=np.zeros((S, T, Hv)), state_in=np.zeros((S, Hv, Dv, Dk)))
    _, _, cap = oracle.reference(**x, capture=True)
    assert cap.nbytes == fx["capture_bytes"]


def test_rejects_bad_shapes():
    x = make_inputs(WORKLOADS["tiny"])
    with pytest.raises(ValueError):
        oracle.reference(**dict(x, g=x["g"][:, :1]))
    y = make_inputs(WORKLOADS["tiny"].with_(n_k_heads=2, n_v_heads=3))
    with pytest.raises(ValueError):  # n_v_heads % n_k_heads != 0
        oracle.reference(**y)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_f32_within_budget_of_f64_shadow(name):
    """P11: on every benchmark workload the float32 oracle sits within
    rel 1e-4 / abs 1e-5 of the float64 shadow (the error budget of the f32
    recurrence itself, including drift over 512 tokens)."""
    w = WORKLOADS[name]
    x = make_inputs(w)
    if name == "prefill":  # keep the CPU suite short: one sequence of four
        x = {n: (a[:1] if hasattr(a, "shape") else a) for n, a in x.items()}
    res32 = oracle.reference(**x, capture=w.capture)
    res64 = oracle.reference(**x, capture=w.capture, precision="f64")
    for a, e, what in zip(res32, res64, ("output", "state_out", "capture")):
        assert_within(a, e, 1e-5 + 1e-4 * np.abs(e), f"{name} {what}")
