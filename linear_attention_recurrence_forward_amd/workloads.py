"""Seeded synthetic inputs for the Gated DeltaNet forward step.

This module only draws numbers: it holds none of the recurrence's arithmetic, so
the tests can feed the same inputs to the HIP path and to the CPU oracle.

Every array is numpy float32 in the row-major shapes that equal the pages'
innermost-first layouts (mlx-native 0.4.0 "src/ops/gated_delta_net.rs", module
doc "Memory layouts"): q, k (S, T, H_k, D_k); v (S, T, H_v, D_v); g, beta
(S, T, H_v); state_in (S, H_v, D_v, D_k).

Recipe (PCG64, fixed draw order q, k, v, g, beta-logits, state_in):
  q      N(0, 1), divided by sqrt(D_k) when the workload pre-scales q
         (q_scale_bits = 0); otherwise left unscaled and the binary32 bits of
         1/sqrt(D_k) are passed as q_scale_bits;
  k      N(0, 1), then L2-normalised over D_k for every (s, t, k-head), in
         float64, rounded once to float32;
  v      N(0, 1);
  g      U(0, g_high);
  beta   sigmoid(N(0, 1)), in float64, rounded once to float32;
  state  N(0, 0.1) (standard deviation 0.1), or zeros for a cold prefill.
"""

from __future__ import annotations

import struct
from dataclasses import dataclass, replace

import numpy as np

SEED_BASE = 20260


def f32_bits(x: float) -> int:
    """IEEE-754 binary32 bit pattern of x (rounded to float32)."""
    return struct.unpack("<I", struct.pack("<f", x))[0]


def q_scale_bits_for(d_k: int) -> int:
    """Bits of the float32 value of 1/sqrt(D_k), the usual folded-in q scale."""
    return f32_bits(float(np.float32(1.0 / np.sqrt(np.float64(d_k)))))


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    d_k: int
    d_v: int
    n_k_heads: int
    n_v_heads: int
    n_tokens: int
    n_seqs: int
    fold_q_scale: bool = False
    g_high: float = 1.0
    state_zero: bool = False
    capture: bool = False
    description: str = ""

    @property
    def q_scale_bits(self) -> int:
        return q_scale_bits_for(self.d_k) if self.fold_q_scale else 0

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def rows(self) -> int:
        return self.n_seqs * self.n_v_heads * self.d_v

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def algorithmic_bytes(self, io_bytes: int = 4) -> int:
        """Bytes the step must move once: state read and written, q and k read
        once per k-head, v, g, beta read and output written once, capture
        written once when present. io_bytes is the element size of q, k, v and
        output (4 for f32, 2 for bf16); everything else is f32."""
        S, T = self.n_seqs, self.n_tokens
        state = self.d_k * self.d_v * self.n_v_heads * S
        io = 2 * self.d_k * self.n_k_heads + 2 * self.d_v * self.n_v_heads
        cap = T * state if self.capture else 0
        return 4 * (2 * state + T * S * 2 * self.n_v_heads + cap) + io_bytes * T * S * io

    def state_bytes(self) -> int:
        return 4 * 2 * self.d_k * self.d_v * self.n_v_heads * self.n_seqs

    def flops(self) -> int:
        """One multiply and three multiply-adds per state cell per token."""
        return 7 * self.d_k * self.d_v * self.n_v_heads * self.n_tokens * self.n_seqs


WORKLOADS = {
    w.name: w for w in (
        Workload("tiny", 0, 32, 32, 1, 2, 8, 1,
                 description="tiny GDN forward, D_k=D_v=32, H_k=1, H_v=2, T=8, S=1"),
        Workload("decode", 1, 128, 128, 16, 48, 1, 1,
                 description="single-layer decode, dense shape, D_k=D_v=128, "
                             "H_k=16, H_v=48, T=1, S=1"),
        Workload("batched_decode", 2, 128, 128, 16, 32, 1, 64, fold_q_scale=True,
                 description="batched decode, MoE shape, D_k=D_v=128, H_k=16, "
                             "H_v=32, T=1, S=64, q_scale folded in"),
        Workload("spec_verify", 3, 128, 128, 8, 8, 4, 8, capture=True,
                 description="speculative-decode verify with per-token state "
                             "capture, D_k=D_v=128, H_k=H_v=8, T=4, S=8"),
        Workload("prefill", 4, 128, 128, 16, 48, 512, 4, fold_q_scale=True,
                 g_high=0.5, state_zero=True,
                 description="prefill run, D_k=D_v=128, H_k=16, H_v=48, T=512, "
                             "S=4, state_in=0, q_scale folded in"),
    )
}


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """Draw one input set for workload w (seed defaults to w.seed)."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    S, T, Hk, Hv, Dk, Dv = (w.n_seqs, w.n_tokens, w.n_k_heads, w.n_v_heads,
                            w.d_k, w.d_v)
    q = rng.standard_normal((S, T, Hk, Dk))
    if not w.fold_q_scale:
        q = q / np.sqrt(np.float64(Dk))
    k = rng.standard_normal((S, T, Hk, Dk))
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((S, T, Hv, Dv))
    g = rng.uniform(0.0, w.g_high, size=(S, T, Hv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((S, T, Hv))))
    if w.state_zero:
        state = np.zeros((S, Hv, Dv, Dk))
    else:
        state = rng.normal(0.0, 0.1, size=(S, Hv, Dv, Dk))
    f = lambda a: np.ascontiguousarray(a, dtype=np.float32)  # noqa: E731
    return dict(q=f(q), k=f(k), v=f(v), g=f(g), beta=f(beta), state_in=f(state),
                q_scale_bits=w.q_scale_bits)
