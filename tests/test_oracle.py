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


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_threaded_oracle_is_bit_identical(threads):
    """The all-core timing splits the independent (sequence, value head) pairs
    over threads: the result equals one whole call bit for bit, with and
    without capture, and the threaded rollback equals the plain one."""
    w = WORKLOADS["spec_verify"].with_(n_seqs=3, n_v_heads=8, n_k_heads=4, d_v=40)
    x = make_inputs(w, seed=3)
    bits = x["q_scale_bits"]
    names = ("q", "k", "v", "g", "beta", "state_in")
    for capture in (False, True):
        one = oracle.reference(**{n: x[n] for n in names}, q_scale_bits=bits,
                               capture=capture)
        par = oracle.reference_threads(**{n: x[n] for n in names}, q_scale_bits=bits,
                                       capture=capture, threads=threads)
        for a, b in zip(one, par):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    one = oracle.reference(**{n: x[n] for n in names}, precision="f64")
    par = oracle.reference_threads(**{n: x[n] for n in names}, precision="f64",
                                   threads=threads)
    for a, b in zip(one, par):
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
    _, _, cap = oracle.reference(**{n: x[n] for n in names}, capture=True)
    acc = np.array([0, w.n_tokens, 2], np.uint32)
    base = np.full(x["state_in"].shape, 3.0, np.float32)
    assert np.array_equal(oracle.rollback_threads(cap, acc, base, threads=threads),
                          oracle.rollback(cap, acc, base))
