"""Helpers for comparing the HIP path with the oracle.

Comparison is teacher-forced: the oracle generates greedily and both sides
consume the oracle's tokens, so one argmax flip cannot cascade. Per step the
logits are compared by relative L2 (||gpu - oracle|| / ||oracle||); the
argmax must agree at every step whose oracle top-2 gap exceeds
delta = 2 * tol * ||l|| / sqrt(V), twice the per-logit error the tolerance
allows (smaller gaps are near-ties, reported, not failed).
"""
from __future__ import annotations

import numpy as np

import oracle


def rel_l2(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))


def first_argmax(v) -> int:
    return int(np.argmax(v))  # numpy returns the lowest index of the maximum


def oracle_greedy(cfg, W, prompt, n_decode, max_ctx=None, chunk_prompt=False):
    """Token-by-token prompt, then greedy decode. Returns (fed, logits) where
    fed[i] is the token fed at step i and logits[i] the logits after it."""
    m = oracle.Model(cfg, W, max_ctx=max_ctx)
    fed, out = [], []
    for t in prompt:
        fed.append(int(t))
        out.append(m.forward([t]))
    for _ in range(n_decode):
        t = first_argmax(out[-1])
        fed.append(t)
        out.append(m.forward([t]))
    m.close()
    return fed, out


def near_tie(ref, tol) -> bool:
    s = np.sort(np.asarray(ref, np.float64))
    delta = 2.0 * tol * np.linalg.norm(ref) / np.sqrt(ref.size)
    return (s[-1] - s[-2]) <= delta


def check_steps(gpu_logits, ref_logits, tol, what=""):
    """Assert rel-L2 <= tol at every step and argmax agreement off near-ties.
    Returns (worst rel-L2, near-tie count)."""
    worst, ties = 0.0, 0
    for i, (g, r) in enumerate(zip(gpu_logits, ref_logits)):
        e = rel_l2(g, r)
        assert np.isfinite(g).all(), f"{what} step {i}: non-finite logits"
        assert e <= tol, f"{what} step {i}: rel-L2 {e:.3e} > {tol:.1e}"
        worst = max(worst, e)
        if first_argmax(g) != first_argmax(r):
            assert near_tie(r, tol), f"{what} step {i}: argmax {first_argmax(g)} vs {first_argmax(r)}"
            ties += 1
    return worst, ties
