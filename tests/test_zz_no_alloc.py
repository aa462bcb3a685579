"""df_forward_noalloc, the entry point for callers that cannot allocate:
the same logits and KV rows as df_forward called one token at a time, on
two calls in a row (the second with fewer tokens), for the llama / qwen3
step list and for gemma3's (its extra norm input also lives in the fixed
array); a model whose step activations do not fit the array is refused
before any launch."""
import numpy as np
import pytest

import synth
from parity import rel_l2

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


def compare(dfa, cfg, calls, tol):
    import torch
    W = synth.make_weights(cfg)
    toks = synth.make_prompt(cfg, sum(calls))
    a = dfa.Model(cfg, W)  # df_forward, one token per call
    b = dfa.Model(cfg, W)  # df_forward_noalloc
    lb = torch.empty(cfg["vocab"], dtype=torch.float32, device="cuda")
    at = 0
    for n in calls:
        chunk = toks[at:at + n]
        for t in chunk:
            la = a.forward([t]).cpu().numpy().copy()
        b._enter()
        dfa.df_forward_noalloc(b.h, chunk, lb)
        b._leave()
        got = lb.cpu().numpy()
        at += n
        e = rel_l2(got, la)
        say(f"  call of {n} tokens: rel-L2 {e:.2e}, bit-identical {np.array_equal(got, la)}")
        assert e <= tol
        assert int(np.argmax(got)) == int(np.argmax(la))
        assert b.kv_len == a.kv_len == at
        for layer in (0, cfg["n_layers"] - 1):
            for which in (0, 1):
                ka, kb = a.read_kv(layer, which, 0, at), b.read_kv(layer, which, 0, at)
                assert rel_l2(kb, ka) <= tol
    a.close()
    b.close()


def test_noalloc_matches_forward_qwen3(dfa):
    cfg = synth.config("qwen3_0p6b", n_layers=4, max_ctx=64)
    say("[qwen3-0.6B shape, 4 layers, f16] df_forward_noalloc of 9 then 3 tokens vs df_forward")
    compare(dfa, cfg, [9, 3], 1e-4)


def test_noalloc_matches_forward_gemma3(dfa):
    cfg = synth.config("tiny_gemma3", max_ctx=48)
    say("[tiny gemma3 f32] df_forward_noalloc of 20 then 5 tokens vs df_forward")
    compare(dfa, cfg, [20, 5], 1e-4)


def test_noalloc_refuses_activations_past_the_array(dfa):
    # 128 query heads of 256 and 16 KV heads: q|k|v 40960 + attention 32768
    # + ffn 32768 floats, more than the array's 256 KiB
    cfg = synth.config("tiny", n_layers=1, n_heads=128, n_kv_heads=16, head_dim=256,
                       ffn_dim=32768, wdtype="f16", max_ctx=8)
    say("[tiny f16, 128 heads of 256, ffn 32768] df_forward_noalloc is refused")
    m = dfa.Model(cfg, synth.make_weights(cfg))
    with pytest.raises(dfa.DecFwdError) as ei:
        dfa.df_forward_noalloc(m.h, [1, 2], m.logits)
    say(f"  {ei.value}")
    assert ei.value.status == "UNSUPPORTED_OP"
    assert m.kv_len == 0
    m.forward([1, 2])  # the allocating path still takes it
    assert m.kv_len == 2
    m.close()
