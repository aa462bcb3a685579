"""The observability calls on the GPU (page "Execution contract",
"Observability": a timing breakdown of every forward): df_profile /
df_profile_read count the launches of a kernel class and their device time,
df_time_kernel replays one decode step's launches of a class, and
df_time_prefill replays one bulk-prefill class. Each returns positive
times, and a model used for timing keeps producing the oracle's logits:
the replays overwrite only activation buffers and cache rows at or past
kv_len, which the next forward rewrites.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check_steps, oracle_greedy, rel_l2

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


def test_profile_counts_launches_and_time(dfa):
    cfg = synth.config("tiny", wdtype="f16", max_ctx=64)
    W = synth.make_weights(cfg)
    say("[tiny qwen3 f16] df_profile on the gate/up and attention classes over 5 decode steps")
    fed, ref = oracle_greedy(cfg, W, synth.make_prompt(cfg, 10), 4, max_ctx=64)
    m = dfa.Model(cfg, W)
    dfa.df_profile(m.h, "gate_up", True)
    got = [m.forward([t]).cpu().numpy().copy() for t in fed[:5]]
    n, ms = dfa.df_profile_read(m.h, "gate_up")
    assert n == 5 * cfg["n_layers"] and ms > 0.0, (n, ms)
    n2, _ = dfa.df_profile_read(m.h, "gate_up")  # reading clears the record
    assert n2 == 0
    dfa.df_profile(m.h, "gate_up", False)
    got += [m.forward([t]).cpu().numpy().copy() for t in fed[5:]]
    check_steps(got, ref, 1e-4, "profiled run")
    m.close()


@pytest.mark.parametrize("kernel", ["qkv", "attn", "attn_merge", "o", "gate_up", "down", "logits", "argmax",
                                    "embed"])
def test_time_kernel_then_forward_matches(dfa, kernel):
    cfg = synth.config("tiny", arch="llama", wdtype="f16", max_ctx=96)
    W = synth.make_weights(cfg)
    say(f"[tiny llama f16] df_time_kernel({kernel}) between decode steps")
    fed, ref = oracle_greedy(cfg, W, synth.make_prompt(cfg, 70), 6, max_ctx=96)
    m = dfa.Model(cfg, W)
    got = [m.forward([t]).cpu().numpy().copy() for t in fed[:40]]
    us = dfa.df_time_kernel(m.h, kernel, 3)
    assert us >= 0.0 and (us > 0.0 or kernel == "attn_merge"), us
    assert m.kv_len == 40
    got += [m.forward([t]).cpu().numpy().copy() for t in fed[40:]]
    check_steps(got, ref, 1e-4, f"after df_time_kernel({kernel})")
    m.close()


@pytest.mark.parametrize("kernel", ["qkv", "rows", "attn", "o", "gate_up", "down"])
def test_time_prefill_then_bulk_matches(dfa, kernel):
    cfg = synth.config("tiny", arch="qwen3", wdtype="f16", max_ctx=160)
    W = synth.make_weights(cfg)
    say(f"[tiny qwen3 f16] df_time_prefill({kernel}, 100 rows) on a 20-token context, then bulk 30")
    toks = synth.make_prompt(cfg, 50)
    m = dfa.Model(cfg, W)
    m.forward(toks[:20], logits=False)
    before = [m.read_kv(layer, which, 0, 20) for layer in range(cfg["n_layers"]) for which in (0, 1)]
    us = dfa.df_time_prefill(m.h, kernel, 100, 2)
    assert us > 0.0
    assert m.kv_len == 20
    # the replays wrote only rows past kv_len: the context is intact, bit for bit
    after = [m.read_kv(layer, which, 0, 20) for layer in range(cfg["n_layers"]) for which in (0, 1)]
    for a, b in zip(before, after):
        assert np.array_equal(a, b)
    # a bulk call on top of the kept context against the oracle
    got = m.forward(toks[20:]).cpu().numpy()
    om = oracle.Model(cfg, W)
    om.forward(toks[:-1], logits=False)
    ref = om.forward([toks[-1]])
    e = rel_l2(got, ref)
    say(f"  bulk 30 on 20: rel-L2 {e:.2e}")
    assert e <= 5e-3
    # more rows than the cache has free past kv_len: refused
    with pytest.raises(dfa.DecFwdError) as ei:
        dfa.df_time_prefill(m.h, kernel, 160 - 50 + 1, 1)
    assert ei.value.status == "INVALID_ARGUMENT"
    om.close()
    m.close()


def test_time_kernel_refuses_attention_on_a_full_cache(dfa):
    cfg = synth.config("tiny", arch="llama", wdtype="f16", max_ctx=24)
    W = synth.make_weights(cfg)
    say("[tiny llama f16] df_time_kernel(attn) on a full cache is refused; the context stays intact")
    m = dfa.Model(cfg, W)
    m.forward(synth.make_prompt(cfg, 24), logits=False)
    assert m.kv_len == 24
    before = m.read_kv(0, 0, 0, 24)
    with pytest.raises(dfa.DecFwdError) as ei:
        dfa.df_time_kernel(m.h, "attn", 1)
    assert ei.value.status == "CONTEXT_FULL"
    assert dfa.df_time_kernel(m.h, "gate_up", 1) > 0.0  # classes that only read the position
    assert np.array_equal(before, m.read_kv(0, 0, 0, 24))
    m.close()
