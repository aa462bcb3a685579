"""The oracle arbitrates the matrix-core paths that the full-size bulk
prefills run (page "Execution contract", "Forward phase": bulk prefill
matches token-by-token within epsilon; "Invariants across paths": the CPU
reference is the arbiter).

The kernels a bulk prefill runs depend on the rows and the matrix widths
only (df_prefill_plan reports them), so models with the real widths and
fewer layers and a smaller vocabulary exercise exactly the GEMM tiles,
attention tiles and epilogues of the full-size runs, at a size the oracle
finishes in seconds to a minute:

* qwen3-8B shape, 2 layers, one bulk prefill of 2048 rows (the C5 prompt):
  q/k/v on the 256 x 192 direct-to-LDS tiles, gate/up on 256 x 256
  direct-to-LDS, o and down on the 128 x 256 tiles;
* llama-8B shape, 2 layers, one bulk prefill of 4096 rows (the bench's
  context): q/k/v on 256 x 192 direct-to-LDS, o, gate/up and down on
  256 x 256 direct-to-LDS;
* llama-8B shape with 8-bit blocks, 2 layers, 2100 rows: the matrices are
  dequantised to f16 first and run the f16 tiles (o and down, with their
  residual epilogue, on 256 x 192);
* qwen3-0.6B shape, all 28 layers, its stated workload: 512 prompt tokens
  and 256 greedy steps token by token (1e-4, teacher-forced), and the
  512-row bulk prefill against the oracle (its down GEMM's grid is small
  and its K long, so each tile's K loop is split over 4 work-groups and the
  last one adds the partial sums).

Each bulk check compares the last position's logits (rel-L2 <= 5e-3, greedy
token identical), every K and V row of every layer and position, and then
decode steps on the bulk-built cache. Weights are seeded host arrays (the
vocab cut to 4096 where stated: the logits matrix is a matvec either way).
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check_steps, first_argmax, rel_l2

pytestmark = pytest.mark.gpu
TOL = 5e-3


@pytest.fixture(scope="module")
def dfa():
    import torch
    assert torch.cuda.is_available()
    import decoder_forward_amd as dfa
    dfa.lib()
    return dfa


def say(*a):
    print(*a, flush=True)


def top2_gap(v):
    s = np.sort(np.asarray(v, np.float64))
    return float(s[-1] - s[-2])


def check_bulk_logits(got, ref, what):
    e = rel_l2(got, ref)
    say(f"  {what}: rel-L2 {e:.2e}, argmax {first_argmax(got)} vs {first_argmax(ref)} "
        f"(oracle top-2 gap {top2_gap(ref):.3e})")
    assert np.isfinite(got).all(), what
    assert e <= TOL, f"{what}: rel-L2 {e:.3e} > {TOL}"
    assert first_argmax(got) == first_argmax(ref), f"{what}: greedy token differs"


def check_all_kv_rows(m, om, cfg, n):
    """Every K / V row of every layer: per position, rel-L2 of the row (all
    KV heads) within the bulk tolerance."""
    worst = 0.0
    for layer in range(cfg["n_layers"]):
        for which in (0, 1):
            a = m.read_kv(layer, which, 0, n).transpose(1, 0, 2).reshape(n, -1).astype(np.float64)
            b = om.kv_read(layer, which, 0, n).transpose(1, 0, 2).reshape(n, -1).astype(np.float64)
            err = np.linalg.norm(a - b, axis=1) / np.linalg.norm(b, axis=1)
            worst = max(worst, float(err.max()))
            bad = np.nonzero(err > TOL)[0]
            assert bad.size == 0, (f"layer {layer} {'KV'[which]} rows {bad[:8].tolist()} "
                                   f"rel-L2 up to {err.max():.3e}")
    say(f"  every KV row of {cfg['n_layers']} layers x {n} positions: worst rel-L2 {worst:.2e}")


def bulk_vs_oracle(dfa, cfg, S, n_decode, expect_plan):
    W = synth.make_weights(cfg)
    toks = synth.make_prompt(cfg, S)
    m = dfa.Model(cfg, W)
    plan = dfa.df_prefill_plan(m.h, S)
    say(f"  GEMM plan at {S} rows: {plan}")
    assert plan == expect_plan, plan
    got = m.forward(toks).cpu().numpy().copy()
    assert m.kv_len == S
    say(f"  oracle: {S} tokens one at a time")
    om = oracle.Model(cfg, W)
    om.forward(toks[:-1], logits=False)
    ref = om.forward([toks[-1]])
    check_bulk_logits(got, ref, f"bulk {S}")
    check_all_kv_rows(m, om, cfg, S)
    t = first_argmax(ref)
    for i in range(n_decode):
        r = om.forward([t])
        g = m.forward([t]).cpu().numpy()
        check_bulk_logits(g, r, f"decode step {i} on the bulk-built cache")
        t = first_argmax(r)
    assert m.kv_len == S + n_decode
    m.close()
    om.close()


def test_qwen3_8b_width_bulk_2048(dfa):
    cfg = synth.config("qwen3_8b", n_layers=2, vocab=4096, max_ctx=2048 + 8)
    say("[qwen3-8B width, 2 layers, vocab 4096] bulk prefill of 2048 vs the oracle, then 2 decode steps")
    bulk_vs_oracle(dfa, cfg, 2048, 2, {
        "qkv": ("256x192_lds", False, False, 1), "o": ("128x256", False, False, 1),
        "gate_up": ("256x256_lds", False, False, 1), "down": ("128x256", False, False, 1)})


def test_llama_8b_width_bulk_4096(dfa):
    cfg = synth.config("llama_8b", n_layers=2, vocab=4096, max_ctx=4096 + 8)
    say("[llama-8B width, 2 layers, vocab 4096] bulk prefill of 4096 vs the oracle, then 2 decode steps")
    bulk_vs_oracle(dfa, cfg, 4096, 2, {
        "qkv": ("256x192_lds", False, False, 1), "o": ("256x256_lds", False, False, 1),
        "gate_up": ("256x256_lds", False, False, 1), "down": ("256x256_lds", False, False, 1)})


def test_llama_8b_q8_width_bulk_2100(dfa):
    cfg = synth.config("llama_8b_q8", n_layers=2, vocab=4096, max_ctx=2100 + 8)
    say("[llama-8B width, 8-bit blocks, 2 layers, vocab 4096] bulk prefill of 2100 "
        "(matrices dequantised first) vs the oracle, then 2 decode steps")
    bulk_vs_oracle(dfa, cfg, 2100, 2, {
        "qkv": ("256x256_lds", False, True, 1), "o": ("256x192_lds", False, True, 1),
        "gate_up": ("256x256_lds", False, True, 1), "down": ("256x192_lds", False, True, 1)})


def test_qwen3_0p6b_stated_workload(dfa):
    """C2 as stated: 28 layers, a 512-token prompt token by token, then 256
    greedy steps (teacher-forced on the oracle's tokens), every step within
    1e-4; and the same prompt as one bulk prefill of 512 rows within 5e-3."""
    cfg = synth.config("qwen3_0p6b")
    P, D = cfg["prompt_len"], cfg["decode_steps"]
    say(f"[qwen3-0.6B shape, 28 layers] {P} prompt tokens + {D} greedy steps, token by token, vs the oracle")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, P)
    om = oracle.Model(cfg, W, max_ctx=P + D)
    m = dfa.Model(cfg, W, max_ctx=P + D)
    ref, got = [], []
    for t in prompt[:-1]:
        om.forward([t], logits=False)
        m.forward([t], logits=False)
    fed = [int(prompt[-1])]
    for i in range(D + 1):
        ref.append(om.forward([fed[-1]]))
        got.append(m.forward([fed[-1]]).cpu().numpy().copy())
        fed.append(first_argmax(ref[-1]))
    worst, ties = check_steps(got, ref, 1e-4, "qwen3-0.6B decode")
    free_run = sum(first_argmax(g) == first_argmax(r) for g, r in zip(got, ref))
    say(f"  {D + 1} steps: worst rel-L2 {worst:.2e}, near-ties {ties}, "
        f"greedy tokens equal at {free_run}/{D + 1}")
    assert m.kv_len == om.kv_len == P + D
    m.close()
    # the prompt as one bulk prefill: the logits after it and every KV row
    b = dfa.Model(cfg, W, max_ctx=P + 8)
    plan = dfa.df_prefill_plan(b.h, P)
    say(f"  GEMM plan at {P} rows: {plan}")
    assert plan == {"qkv": ("128x256", False, False, 1), "o": ("128x128", False, False, 1),
                    "gate_up": ("128x256", False, False, 1), "down": ("128x128", False, False, 4)}, plan
    lb = b.forward(prompt).cpu().numpy()
    check_bulk_logits(lb, ref[0], f"bulk {P}")
    check_all_kv_rows(b, om, cfg, P)
    b.close()
    om.close()
