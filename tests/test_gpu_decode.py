"""Decode parity on the GPU: the HIP path through the C ABI against the
oracle on identical seeded inputs (teacher-forced, per-step logits).

Tolerances: decode logits rel-L2 <= 1e-4 with f32 / f16 weights and <= 1e-3
with 8-bit blocks; KV-cache positions and lengths exact. One token per call
follows page "Execution contract", "Forward phase" (prefill token by token,
then decode).
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check_steps, first_argmax, oracle_greedy, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "gpu tests need a GPU"
    return torch


@pytest.fixture(scope="module")
def dfa(torch_dev):
    import decoder_forward_amd as dfa
    dfa.lib()
    return dfa


def say(*a):
    print(*a, flush=True)


def gpu_teacher_forced(dfa, cfg, W, fed, max_ctx=None):
    m = dfa.Model(cfg, W, max_ctx=max_ctx)
    out = []
    for t in fed:
        out.append(m.forward([t]).cpu().numpy().copy())
    return m, out


@pytest.mark.parametrize("arch,wdtype,over", [
    ("qwen3", "f32", {}), ("llama", "f32", {}), ("qwen3", "f16", {}), ("llama", "q8", {}),
    ("qwen2", "f32", {}), ("qwen2", "f16", dict(rope_pairing="adjacent")),
    ("qwen2", "q8", dict(n_heads=6, n_kv_heads=2)),
    ("llama", "f32", dict(rope_pairing="adjacent", n_heads=14, n_kv_heads=2)),
    ("qwen3", "f16", dict(rope_pairing="adjacent", n_heads=10, n_kv_heads=2)),
    # odd vocabularies: the logits matvec runs one row per unit instead of
    # row pairs
    ("llama", "f16", dict(vocab=257)), ("qwen3", "q8", dict(vocab=251))],
    ids=lambda v: "-".join(f"{k}{x}" for k, x in v.items()) if isinstance(v, dict) else str(v))
def test_tiny_token_by_token_and_decode(dfa, arch, wdtype, over):
    say(f"[tiny {arch} {wdtype} {over}] 32-token prompt + 16 greedy steps")
    cfg = synth.config("tiny", arch=arch, wdtype=wdtype, **over)
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, cfg["prompt_len"])
    fed, ref = oracle_greedy(cfg, W, prompt, cfg["decode_steps"])
    m, got = gpu_teacher_forced(dfa, cfg, W, fed)
    tol = 1e-3 if wdtype == "q8" else 1e-4
    worst, ties = check_steps(got, ref, tol, f"tiny {arch} {wdtype}")
    say(f"  worst rel-L2 {worst:.2e}, near-ties {ties}")
    assert m.kv_len == len(fed)
    om = oracle.Model(cfg, W)
    om.forward(fed, logits=False)
    for layer in range(cfg["n_layers"]):
        for which in (0, 1):
            a = m.read_kv(layer, which, 0, len(fed))
            b = om.kv_read(layer, which, 0, len(fed))
            assert np.max(np.abs(a - b)) <= 1e-4 * max(1.0, np.max(np.abs(b))), (layer, which)
    m.close()


@pytest.mark.parametrize("hd,n_heads,n_kv", [(32, 4, 2), (64, 4, 1), (64, 6, 3)])
def test_head_dims_across_attention_tiles(dfa, hd, n_heads, n_kv):
    # head_dim 32 (two dims per lane) and 64 (one float4 group per lane) at
    # positions that span several 64-row attention tiles and a ragged tail
    say(f"[tiny qwen3 f16, head_dim {hd}, {n_heads}/{n_kv} heads] 150-token prompt + 8 steps")
    cfg = synth.config("tiny", wdtype="f16", head_dim=hd, n_heads=n_heads, n_kv_heads=n_kv, max_ctx=192)
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 150)
    fed, ref = oracle_greedy(cfg, W, prompt, 8, max_ctx=192)
    m, got = gpu_teacher_forced(dfa, cfg, W, fed, max_ctx=192)
    worst, ties = check_steps(got, ref, 1e-4, f"head_dim {hd}")
    say(f"  worst rel-L2 {worst:.2e}, near-ties {ties}")
    m.close()


def test_tiny_long_context_multi_chunk(dfa):
    say("[tiny qwen3 f32] 200-token prompt (4 attention chunks, ragged) + 8 steps")
    cfg = synth.config("tiny", max_ctx=256)
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 200)
    fed, ref = oracle_greedy(cfg, W, prompt, 8, max_ctx=256)
    m, got = gpu_teacher_forced(dfa, cfg, W, fed, max_ctx=256)
    worst, _ = check_steps(got, ref, 1e-4, "tiny long")
    say(f"  worst rel-L2 {worst:.2e}")
    m.close()


def test_generate_matches_forward_and_argmax(dfa, torch_dev):
    say("[tiny] df_generate vs df_forward + df_argmax, and vs the oracle's greedy tokens")
    cfg = synth.config("tiny")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 20)
    n = 16
    a = dfa.Model(cfg, W)
    a.forward(prompt[:-1], logits=False)
    toks = a.generate(int(prompt[-1]), n).cpu().numpy()
    gen_logits = a.logits.cpu().numpy().copy()
    b = dfa.Model(cfg, W)
    b.forward(prompt[:-1], logits=False)
    t = int(prompt[-1])
    seq = []
    for _ in range(n):
        b.forward([t])
        t = b.argmax()
        seq.append(t)
    assert list(toks) == seq
    assert np.array_equal(gen_logits, b.logits.cpu().numpy())
    assert a.kv_len == b.kv_len == 19 + n
    fed, ref = oracle_greedy(cfg, W, prompt, n - 1)
    oracle_toks = [first_argmax(r) for r in ref[len(prompt) - 1:]]
    assert toks[0] == oracle_toks[0]
    agree = 0
    for x, y in zip(toks, oracle_toks):
        if x != y:
            break
        agree += 1
    say(f"  free-running agreement with the oracle: {agree}/{n} tokens")
    assert agree >= 4
    a.close()
    b.close()


def test_bulk_call_matches_single_calls(dfa):
    say("[tiny] df_forward with n > 1 vs n single calls")
    cfg = synth.config("tiny")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 24)
    a = dfa.Model(cfg, W)
    la = a.forward(prompt).cpu().numpy()
    b = dfa.Model(cfg, W)
    for t in prompt:
        lb = b.forward([t]).cpu().numpy()
    assert rel_l2(la, lb) <= 5e-3
    for layer in range(cfg["n_layers"]):
        ka, kb = a.read_kv(layer, 0, 0, 24), b.read_kv(layer, 0, 0, 24)
        assert np.max(np.abs(ka - kb)) <= 5e-3 * np.max(np.abs(kb))
    a.close()
    b.close()


def test_reset_rerun_and_second_load_are_bitwise_identical(dfa):
    say("[tiny] rerun after reset_kv_cache and a second load")
    cfg = synth.config("tiny")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 30)

    def run(m):
        return np.stack([m.forward([t]).cpu().numpy().copy() for t in prompt])
    a = dfa.Model(cfg, W)
    x = run(a)
    a.reset()
    assert a.kv_len == 0
    y = run(a)
    b = dfa.Model(cfg, W)
    z = run(b)
    assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(x.view(np.uint32), z.view(np.uint32))
    a.close()
    b.close()


def test_errors_are_codes_and_leave_state(dfa):
    say("[tiny] context full, bad token, kv rows past kv_len untouched")
    cfg = synth.config("tiny")
    W = synth.make_weights(cfg)
    m = dfa.Model(cfg, W)
    canary = np.full((cfg["n_kv_heads"], 8, cfg["head_dim"]), 12345.0, np.float32)
    for layer in range(cfg["n_layers"]):
        m.write_kv(layer, 0, 10, canary, 0)
        m.write_kv(layer, 1, 10, canary, 0)
    m.forward(synth.make_prompt(cfg, 10))
    assert m.kv_len == 10
    for layer in range(cfg["n_layers"]):
        assert np.array_equal(m.read_kv(layer, 0, 10, 8), canary)
        assert np.array_equal(m.read_kv(layer, 1, 10, 8), canary)
    with pytest.raises(dfa.DecFwdError) as ei:
        m.forward(np.zeros(cfg["max_ctx"], np.int32))
    assert ei.value.status == "CONTEXT_FULL"
    with pytest.raises(dfa.DecFwdError) as ei:
        m.forward([cfg["vocab"]])
    assert ei.value.status == "INVALID_ARGUMENT"
    with pytest.raises(dfa.DecFwdError) as ei:
        m.forward([-1])
    assert ei.value.status == "INVALID_ARGUMENT"
    assert m.kv_len == 10
    m.close()
    m.close()


def test_qwen3_0p6b_shape_decode(dfa):
    cfg = synth.config("qwen3_0p6b")
    say("[qwen3-0.6B shape, 28 layers, f16] 24-token prompt + 8 greedy steps")
    W = synth.make_weights(cfg)
    prompt = synth.make_prompt(cfg, 24)
    fed, ref = oracle_greedy(cfg, W, prompt, 8, max_ctx=64)
    m, got = gpu_teacher_forced(dfa, cfg, W, fed, max_ctx=64)
    worst, ties = check_steps(got, ref, 1e-4, "qwen3-0.6B")
    say(f"  worst rel-L2 {worst:.2e}, near-ties {ties}")
    m.close()


def test_qwen3_0p6b_shape_long_context_from_restored_kv(dfa):
    cfg = synth.config("qwen3_0p6b")
    n_ctx = 700
    say(f"[qwen3-0.6B shape] {n_ctx} positions of synthetic KV restored on both sides, 4 steps")
    W = synth.make_weights(cfg)
    om = oracle.Model(cfg, W, max_ctx=768)
    m = dfa.Model(cfg, W, max_ctx=768)
    for layer in range(cfg["n_layers"]):
        K, V = synth.make_kv_rows(cfg, layer, n_ctx)
        om.kv_write(layer, 0, 0, K)
        om.kv_write(layer, 1, 0, V)
        m.write_kv(layer, 0, 0, K, n_ctx)
        m.write_kv(layer, 1, 0, V, n_ctx)
    om.set_kv_len(n_ctx)
    toks = synth.make_prompt(cfg, 4, stream=1)
    ref = [om.forward([t]) for t in toks]
    got = [m.forward([t]).cpu().numpy().copy() for t in toks]
    worst, _ = check_steps(got, ref, 1e-4, "qwen3-0.6B ctx 700")
    say(f"  worst rel-L2 {worst:.2e}")
    assert m.kv_len == n_ctx + 4
    m.close()
