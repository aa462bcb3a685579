"""Parity of the persistent decode step (one launch per token, opt-in with
DF_FLAG_PERSISTENT_STEP) on the GPU.

The step kernel runs where the weights are f16 or 8-bit blocks and
head_dim is 64 or 128. These cases use small shapes the oracle finishes in
seconds but that still cover every template the kernel has: head_dim 64 and
128, query heads per KV head 1, 2, 3, 4, 7 and 8, the three architectures
and both rope pairings, f16 and
8-bit weights with an f16 or an 8-bit logits matrix, a model dimension that
is not a whole number of 512-value chunks, a ragged vocabulary, and contexts
long enough for many attention splits. Bars as for the other decode tests:
logits rel-L2 <= 1e-4 (f16) / 1e-3 (8-bit), KV rows and lengths exact where
the two sides must agree exactly.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check_steps, first_argmax, near_tie, oracle_greedy, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dfa():
    import torch
    assert torch.cuda.is_available()
    import decoder_forward_amd as dfa
    dfa.lib()
    return dfa


def say(*a):
    print(*a, flush=True)


def small(arch, wdtype, hd, n_kv, tied=True, **over):
    base = dict(arch=arch, wdtype=wdtype, n_layers=2, d_model=192, n_heads=8,
                n_kv_heads=n_kv, head_dim=hd, ffn_dim=416, vocab=1000,
                tied=tied, max_ctx=96)
    base.update(over)
    return synth.config("tiny", **base)


CASES = [("qwen3", "f16", 64, 8, True, {}), ("llama", "f16", 64, 4, True, {}),
         ("qwen3", "f16", 128, 2, True, {}), ("llama", "f16", 128, 1, False, {}),
         ("qwen3", "q8", 128, 4, False, {}), ("llama", "q8", 64, 2, True, {}),
         ("qwen2", "f16", 128, 1, False, dict(n_heads=7)),
         ("qwen2", "q8", 64, 2, True, dict(n_heads=6, rope_pairing="adjacent"))]


@pytest.mark.parametrize("arch,wdtype,hd,n_kv,tied,over", CASES,
                         ids=lambda v: "-".join(f"{k}{x}" for k, x in v.items())
                         if isinstance(v, dict) else str(v))
def test_step_kernel_teacher_forced(dfa, arch, wdtype, hd, n_kv, tied, over):
    cfg = small(arch, wdtype, hd, n_kv, tied, **over)
    G = cfg["n_heads"] // n_kv
    say(f"[{arch} {wdtype} hd {hd} G {G} tied {tied}] 24-token prompt + 12 greedy steps")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 24)
    fed, ref = oracle_greedy(cfg, W, prompt, 12)
    m = dfa.Model(cfg, W, persistent_step=True)
    t = m.timings()
    assert t["persistent_step"] == 1 and t["step_blocks"] > 0, t
    got = [m.forward([x]).cpu().numpy().copy() for x in fed]
    tol = 1e-3 if wdtype == "q8" else 1e-4
    worst, ties = check_steps(got, ref, tol, cfg["name"])
    say(f"  worst rel-L2 {worst:.2e}, near-ties {ties}")
    assert m.kv_len == len(fed)
    om = oracle.Model(cfg, W)
    om.forward(fed, logits=False)
    for layer in range(cfg["n_layers"]):
        for which in (0, 1):
            a = m.read_kv(layer, which, 0, len(fed))
            b = om.kv_read(layer, which, 0, len(fed))
            assert np.linalg.norm(a - b) / np.linalg.norm(b) <= tol, (layer, which)
    om.close()
    m.close()


def test_step_kernel_many_splits_restored_context(dfa):
    """1500 restored positions: 24 tiles of 64 rows, split over the grid."""
    cfg = small("qwen3", "f16", 128, 2, max_ctx=1600)
    n_ctx = 1500
    say(f"[qwen3 f16 hd 128 G 4] {n_ctx} restored positions + 4 steps")
    W = synth.make_weights(cfg)
    om = oracle.Model(cfg, W)
    m = dfa.Model(cfg, W, persistent_step=True)
    assert m.timings()["persistent_step"] == 1
    for layer in range(cfg["n_layers"]):
        K, V = synth.make_kv_rows(cfg, layer, n_ctx)
        om.kv_write(layer, 0, 0, K)
        om.kv_write(layer, 1, 0, V)
        m.write_kv(layer, 0, 0, K, n_ctx)
        m.write_kv(layer, 1, 0, V, n_ctx)
    om.set_kv_len(n_ctx)
    toks = synth.make_prompt(cfg, 4, stream=3)
    ref = [om.forward([x]) for x in toks]
    got = [m.forward([x]).cpu().numpy().copy() for x in toks]
    worst, _ = check_steps(got, ref, 1e-4, "many splits")
    say(f"  worst rel-L2 {worst:.2e}")
    a = m.read_kv(1, 0, n_ctx, 4)
    b = om.kv_read(1, 0, n_ctx, 4)
    assert np.linalg.norm(a - b) / np.linalg.norm(b) <= 1e-4
    om.close()
    m.close()


def test_step_kernel_generate_equals_forward_and_argmax(dfa):
    cfg = small("llama", "f16", 64, 2)
    say("[llama f16 hd 64] df_generate vs df_forward + df_argmax (bitwise)")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 20)
    n = 24
    a = dfa.Model(cfg, W, persistent_step=True)
    a.forward(prompt[:-1], logits=False)
    toks = a.generate(int(prompt[-1]), n).cpu().numpy()
    la = a.logits.cpu().numpy().copy()
    b = dfa.Model(cfg, W, persistent_step=True)
    b.forward(prompt[:-1], logits=False)
    t = int(prompt[-1])
    seq = []
    for _ in range(n):
        b.forward([t])
        t = b.argmax()
        seq.append(t)
    assert list(toks) == seq
    assert np.array_equal(la.view(np.uint32), b.logits.cpu().numpy().view(np.uint32))
    assert a.kv_len == b.kv_len == len(prompt) - 1 + n
    # a second generate continues from the device state
    more = a.generate(int(toks[-1]), 4).cpu().numpy()
    for x in more:
        b.forward([t])
        t = b.argmax()
        assert x == t
    a.close()
    b.close()


def test_step_kernel_agrees_with_separate_launches(dfa):
    cfg = small("qwen3", "f16", 128, 4)
    say("[qwen3 f16 hd 128] persistent step vs one launch per operation class")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 40)
    a = dfa.Model(cfg, W, persistent_step=True)
    b = dfa.Model(cfg, W)
    assert a.timings()["persistent_step"] == 1
    assert b.timings()["persistent_step"] == 0
    for i, x in enumerate(prompt):
        la = a.forward([x]).cpu().numpy()
        lb = b.forward([x]).cpu().numpy()
        assert rel_l2(la, lb) <= 1e-5, i
    for layer in range(cfg["n_layers"]):
        ka, kb = a.read_kv(layer, 0, 0, 40), b.read_kv(layer, 0, 0, 40)
        assert np.linalg.norm(ka - kb) / np.linalg.norm(kb) <= 1e-5
    with pytest.raises(dfa.DecFwdError) as ei:
        dfa.df_time_kernel(b.h, "step", 2)
    assert ei.value.status == "UNSUPPORTED_OP"
    us = dfa.df_time_kernel(a.h, "step", 4)
    assert us > 0
    a.close()
    b.close()


def test_step_kernel_rerun_is_bitwise_identical(dfa):
    cfg = small("llama", "q8", 128, 8, tied=False)
    say("[llama q8 hd 128 G 1] rerun after reset and a second load: bitwise equal")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 30)

    def run(m):
        return np.stack([m.forward([x]).cpu().numpy().copy() for x in prompt])
    a = dfa.Model(cfg, W, persistent_step=True)
    x = run(a)
    a.reset()
    y = run(a)
    b = dfa.Model(cfg, W, persistent_step=True)
    z = run(b)
    assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(x.view(np.uint32), z.view(np.uint32))
    a.close()
    b.close()


def test_step_kernel_prompt_token_loop_without_logits(dfa):
    """A prompt fed token by token with the logits phase skipped (logits
    only on the last call) through the step kernel still matches the
    oracle."""
    cfg = small("qwen3", "q8", 64, 4, tied=False)
    say("[qwen3 q8 hd 64] 30-token prompt one token per call, logits on the last only")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 30)
    m = dfa.Model(cfg, W, persistent_step=True)
    for t in prompt[:-1]:
        m.forward([t], logits=False)
    got = m.forward([prompt[-1]]).cpu().numpy()
    om = oracle.Model(cfg, W)
    ref = om.forward(prompt)
    assert rel_l2(got, ref) <= 1e-3
    if first_argmax(got) != first_argmax(ref):
        assert near_tie(ref, 1e-3)
    assert m.kv_len == 30
    om.close()
    m.close()
