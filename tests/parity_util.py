"""Helpers shared by the GPU parity tests (test-side only).

The bar on bf16 layer outputs is the plain one: max|y - y_ref| <= 2e-2 * rms(y_ref),
rms over every output of the layer call, y_ref the fp64 oracle. A test may ask for the
bar beyond each output's own bf16 rounding (|y - y_ref| <= 2e-2 * rms + ulp_bf16(y_ref) / 2
elementwise) only where the plain bar is out of reach of any bf16 output: where rounding
the exact result itself to bf16 already misses it. check_close asserts that condition
before it applies the relaxed form.
"""

from __future__ import annotations

import sys

import numpy as np

from oracle import moe_ref as R
from synth import gen

DEV = "cuda:0"
TOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def y_f64(y):
    return y.float().cpu().numpy().astype(np.float64)


class OracleExperts:
    """Oracle experts built on demand from the seeded generator (never from the GPU)."""

    def __init__(self, w, layer):
        self.w, self.layer, self.cache = w, layer, {}

    def __call__(self, e):
        if e not in self.cache:
            self.cache[e] = R.Expert(gen.expert_tensors(self.w.seed, self.layer, e, self.w.H, self.w.I), self.w.H,
                                     self.w.I)
        return self.cache[e]


def oracle_layer(w, layer, x_bits, logits=None, renorm=False):
    wr = gen.router_weight(w.seed, layer, w.E, w.H) if w.router == "gemv" else None
    shared = None
    if w.shared:
        shared = R.Expert(gen.expert_tensors(w.seed, layer, gen.SHARED_EXPERT, w.H, w.I), w.H, w.I)
    return R.moe_layer(x_bits, OracleExperts(w, layer), w.K, logits=logits, w_router=wr, shared=shared,
                       renorm=renorm)


def bf16_half_ulp(y):
    """Half the bf16 spacing at each value: the rounding any bf16 output of it carries."""
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def bf16_nearest(y):
    """fp64 values rounded to the nearest bf16 (ties to even), as fp64 (normal range)."""
    a = np.abs(y)
    ulp = np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7)
    return np.where(a > 0, np.round(y / ulp) * ulp, 0.0)


def check_close(y_gpu, y_ref, what, beyond_half_ulp=False):
    """Assert the bar on one layer call's outputs (see the module docstring).

    beyond_half_ulp: use the relaxed form; allowed only when the bf16 rounding of y_ref
    itself exceeds 2e-2 * rms (asserted), i.e. where no bf16 output can meet the plain bar.
    """
    d = np.abs(y_gpu - y_ref)
    rms = np.sqrt(np.mean(y_ref**2))
    floor = np.abs(bf16_nearest(y_ref) - y_ref).max()
    beyond = np.max(d - bf16_half_ulp(y_ref))
    r = (lambda v: v / rms) if rms else (lambda v: float("nan"))
    say(f"{what}: max|err| / rms = {r(d.max()):.3e} (bar {TOL:.0e}), bf16 rounding floor of the oracle "
        f"{r(floor):.3e}, beyond the bf16 half-ulp {r(beyond):.3e}, max|y_ref| / rms = "
        f"{np.abs(y_ref).max() / rms if rms else 0:.1f}")
    if rms == 0:
        assert d.max() == 0
    elif beyond_half_ulp:
        assert floor > TOL * rms, "the plain bar is within reach here: use it"
        assert beyond <= TOL * rms
    else:
        assert d.max() <= TOL * rms
