"""Pins of the oracle's whole forward pass (CPU only).

* the float64 brute force (full-sequence, explicit causal mask) on the tiny
  decoder in all three architectures, both RoPE pairings and with 8-bit
  weights, and on one-layer
  slices of the real shapes with a small vocabulary;
* closed forms: zero layers, zero-output layers, qwen2 with zero biases ==
  llama, add_bias on exact sums, adjacent RoPE == halves on permuted lanes;
* the step list and steps-per-layer counts the pages print;
* runtime invariants: bulk == token by token, reset, KV positions;
* planted mistakes in the oracle, each of which one of these pins catches.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from brute_f64 import forward_all, rel_l2

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "step_lists.txt")


def run_token_by_token(cfg, W, toks):
    m = oracle.Model(cfg, W, max_ctx=max(cfg["max_ctx"], len(toks)))
    out = np.stack([m.forward([t]) for t in toks])
    m.close()
    return out


def tiny(**kw):
    base = "tiny_gemma3" if kw.get("arch") == "gemma3" else "tiny"
    cfg = synth.config(base, **kw)
    return cfg, synth.make_weights(cfg)


@pytest.mark.parametrize("arch,wdtype,pairing", [
    ("qwen3", "f32", "halves"), ("llama", "f32", "halves"),
    ("qwen3", "f16", "halves"), ("llama", "q8", "halves"),
    ("qwen2", "f32", "halves"), ("qwen2", "f16", "adjacent"),
    ("qwen2", "q8", "halves"), ("llama", "f32", "adjacent"),
    ("qwen3", "f32", "adjacent"), ("gemma3", "f32", "halves"),
    ("gemma3", "f16", "halves"), ("gemma3", "q8", "adjacent")])
def test_tiny_matches_f64_brute_force_every_step(arch, wdtype, pairing):
    cfg, W = tiny(arch=arch, wdtype=wdtype, rope_pairing=pairing)
    toks = synth.make_prompt(cfg, 40)
    cfg["max_ctx"] = 48
    got = run_token_by_token(cfg, W, toks)
    ref = forward_all(cfg, W, toks)
    worst = max(rel_l2(got[s], ref[s]) for s in range(len(toks)))
    assert worst < 2e-6, worst


@pytest.mark.parametrize("name,vocab,n", [("qwen3_0p6b", 512, 6),
                                          ("llama_8b", 384, 3),
                                          ("qwen3_8b", 256, 3)])
def test_one_layer_real_shape_matches_brute_force(name, vocab, n):
    cfg = synth.config(name, n_layers=1, vocab=vocab, max_ctx=8)
    W = synth.make_weights(cfg)
    toks = synth.make_prompt(cfg, n)
    got = run_token_by_token(cfg, W, toks)
    ref = forward_all(cfg, W, toks)
    for s in range(n):
        assert rel_l2(got[s], ref[s]) < 2e-6


def test_one_layer_q8_real_shape_matches_brute_force():
    cfg = synth.config("llama_8b_q8", n_layers=1, vocab=256, max_ctx=4,
                       d_model=1024, ffn_dim=2048, n_heads=8, n_kv_heads=2)
    W = synth.make_weights(cfg)
    toks = synth.make_prompt(cfg, 3)
    got = run_token_by_token(cfg, W, toks)
    ref = forward_all(cfg, W, toks)
    for s in range(3):
        assert rel_l2(got[s], ref[s]) < 2e-6


def test_zero_layers_closed_form_tied():
    # x = e_t, y = x * r with unit norm weight, logit_t = r * |e_t|^2.
    cfg, W = tiny(n_layers=0)
    W["output_norm.weight"] = np.ones_like(W["output_norm.weight"])
    m = oracle.Model(cfg, W)
    E = W["token_embd.weight"].astype(np.float64)
    for t in (0, 5, 255):
        m.reset()
        lg = m.forward([t])
        r = 1.0 / np.sqrt(np.mean(E[t] ** 2) + cfg["rms_eps"])
        assert lg[t] == pytest.approx(r * np.sum(E[t] ** 2), rel=1e-6)
        assert np.allclose(lg, E @ (E[t] * r), rtol=1e-5, atol=1e-6)


def test_zero_output_layers_reduce_to_zero_layers_bitwise():
    cfg, W = tiny()
    for i in range(cfg["n_layers"]):
        for s in ("attn_output", "ffn_down"):
            W[f"blk.{i}.{s}.weight"] = np.zeros_like(W[f"blk.{i}.{s}.weight"])
    toks = synth.make_prompt(cfg, 6)
    a = run_token_by_token(cfg, W, toks)
    cfg0 = dict(cfg, n_layers=0)
    b = run_token_by_token(cfg0, W, toks)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def golden_lists():
    ops, steps = {}, {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, rest = line.split(":", 1)
        if key == "steps_per_layer":
            arch, n = rest.split()
            steps[arch] = int(n)
        else:
            ops[key] = rest.split()
    return ops, steps


@pytest.mark.parametrize("arch", ["qwen3", "llama", "qwen2", "gemma3"])
def test_step_list_matches_the_printed_definition(arch):
    gold, steps = golden_lists()
    cfg, W = tiny(arch=arch)
    m = oracle.Model(cfg, W)
    m.forward(synth.make_prompt(cfg, 2))
    sections = m.trace().split("|")
    assert len(sections) - 2 == cfg["n_layers"]
    assert sections[0].split(",") == gold[f"{arch} prologue"]
    for blk in sections[1:-1]:
        assert blk.split(",") == gold[f"{arch} block"]
        assert len(blk.split(",")) == steps[arch]
    assert sections[-1].split(",") == gold[f"{arch} epilogue"]


def test_qwen2_with_zero_biases_is_llama_bitwise():
    # qwen2's definition is llama's plus three bias lines (page "Local
    # inference and architectures", "The format"): with every bias zero the
    # two must give the same bits (x + 0 == x in f32).
    cfg, W = tiny(arch="qwen2")
    for k in list(W):
        if k.endswith(".bias"):
            W[k] = np.zeros_like(W[k])
    toks = synth.make_prompt(cfg, 8)
    a = run_token_by_token(cfg, W, toks)
    Wl = {k: v for k, v in W.items() if not k.endswith(".bias")}
    b = run_token_by_token(dict(cfg, arch="llama"), Wl, toks)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_qwen2_biases_move_the_logits():
    cfg, W = tiny(arch="qwen2")
    toks = synth.make_prompt(cfg, 4)
    a = run_token_by_token(cfg, W, toks)
    Wl = {k: v for k, v in W.items() if not k.endswith(".bias")}
    b = run_token_by_token(dict(cfg, arch="llama"), Wl, toks)
    assert rel_l2(a[-1], b[-1]) > 1e-2


def test_add_bias_exact():
    # One rounding of an exact sum: values whose sum is exact in f32.
    y = np.array([1.0, -2.5, 3.0e7, 0.125], np.float32)
    b = np.array([0.5, 2.5, 1.0, -0.125], np.float32)
    assert np.array_equal(oracle.add_bias(y.copy(), b),
                          np.array([1.5, 0.0, 3.0e7 + 1.0, 0.0], np.float32))
    # 1 + 2^-24 rounds to 1 (ties to even), 1 + 3*2^-24 to 1 + 2^-22
    y = np.ones(2, np.float32)
    b = np.array([2.0 ** -24, 3 * 2.0 ** -24], np.float32)
    assert np.array_equal(oracle.add_bias(y, b),
                          np.array([1.0, 1.0 + 2.0 ** -22], np.float32))


def test_rope_adjacent_is_halves_on_permuted_lanes():
    # Pairing (2i, 2i+1) is pairing (i, i + hd/2) after the permutation that
    # deals even lanes to the first half and odd lanes to the second.
    hd, heads = 16, 3
    cos, sin = oracle.rope_table(9, hd, 10000.0)
    t = np.random.default_rng(4).standard_normal(heads * hd).astype(np.float32)
    perm = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])
    for p in (0, 1, 8):
        adj = oracle.rope(t.copy(), hd, cos[p], sin[p], pairing="adjacent")
        tp = t.reshape(heads, hd)[:, perm].reshape(-1).copy()
        hal = oracle.rope(tp, hd, cos[p], sin[p], pairing="halves")
        assert np.array_equal(adj.reshape(heads, hd)[:, perm].reshape(-1), hal)
        if p:
            assert not np.array_equal(
                adj, oracle.rope(t.copy(), hd, cos[p], sin[p]))


def test_window_wider_than_the_context_is_no_window_bitwise():
    # A window that covers every position leaves the causal mask as it is;
    # with one theta for all layers the two models are the same bits.
    cfg, W = tiny(arch="gemma3")
    cfg["rope_theta_local"] = cfg["rope_theta"]
    toks = synth.make_prompt(cfg, 20)
    a = run_token_by_token(dict(cfg, sliding_window=1000), W, toks)
    b = run_token_by_token(dict(cfg, sliding_window=0), W, toks)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    c = run_token_by_token(cfg, W, toks)  # window 8 over 20 tokens: differs
    assert rel_l2(c[-1], b[-1]) > 1e-3


def test_window_of_one_sees_only_itself():
    # Window 1 on every layer: each attention weight is exactly 1 on the
    # position's own V, so the last logits depend on the last token only.
    cfg, W = tiny(arch="gemma3")
    cfg.update(sliding_window=1, window_pattern=cfg["n_layers"] + 1)
    toks = synth.make_prompt(cfg, 9)
    a = run_token_by_token(cfg, W, toks)[-1]
    b = run_token_by_token(cfg, W, toks[-1:])[-1]
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_gelu_tanh_pins():
    x = np.linspace(-6, 6, 2001).astype(np.float32)
    g = oracle.gelu_tanh(x).astype(np.float64)
    gm = oracle.gelu_tanh(-x).astype(np.float64)
    assert oracle.gelu_tanh(np.zeros(1, np.float32))[0] == 0.0
    # tanh is odd, so gelu_tanh(x) - gelu_tanh(-x) = x
    assert np.max(np.abs(g - gm - x) / np.maximum(1, np.abs(x))) < 4e-7
    big = oracle.gelu_tanh(np.array([12.0, -12.0], np.float32))
    assert big[0] == np.float32(12.0) and abs(big[1]) < 1e-30
    # the tanh form is within about 1e-3 of the erf form and is not it
    from math import erf
    ge = np.array([0.5 * v * (1 + erf(v / np.sqrt(2.0))) for v in x.astype(np.float64)])
    dev = np.max(np.abs(g - ge))
    assert 1e-4 < dev < 1e-3, dev
    # one value against the formula evaluated by hand: x = 1
    # 0.5 * (1 + tanh(0.7978845608 * 1.044715)) = 0.8411919906
    assert abs(oracle.gelu_tanh(np.ones(1, np.float32))[0] - 0.8411919906) < 1e-7


def test_scale_is_one_rounding():
    x = np.array([1.0, -3.0, 1e-3, 3.0e37], np.float32)
    assert np.array_equal(oracle.scale(x, 4.0), x * np.float32(4.0))
    s = np.float32(np.sqrt(2560.0))
    y = np.array([0.3, -1.7, 2.2e-5], np.float32)
    want = (y.astype(np.float64) * np.float64(s)).astype(np.float32)
    assert np.array_equal(oracle.scale(y, float(s)), want)


def test_norm_heads_before_rope_matters():
    # The qwen3 definition puts norm_heads before rope; the other order is
    # a different model (page "Local inference and architectures", "The
    # format"). The planted swap must move the logits.
    cfg, W = tiny()
    toks = synth.make_prompt(cfg, 8)
    good = run_token_by_token(cfg, W, toks)
    oracle.set_mutation("norm_after_rope")
    try:
        bad = run_token_by_token(cfg, W, toks)
    finally:
        oracle.set_mutation("none")
    # at position 0 RoPE is the identity, so only later steps can differ
    assert np.array_equal(good[0], bad[0])
    assert max(rel_l2(bad[s], good[s]) for s in range(1, 8)) > 1e-4


def test_bulk_equals_token_by_token_bitwise():
    cfg, W = tiny()
    toks = synth.make_prompt(cfg, 20)
    a = oracle.Model(cfg, W)
    la = a.forward(toks[:13])
    lb_model = oracle.Model(cfg, W)
    for t in toks[:12]:
        lb_model.forward([t], logits=False)
    lb = lb_model.forward([toks[12]])
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    for layer in range(cfg["n_layers"]):
        for which in (0, 1):
            assert np.array_equal(a.kv_read(layer, which, 0, 13),
                                  lb_model.kv_read(layer, which, 0, 13))
    # and continuing after a bulk call uses absolute positions
    assert np.array_equal(a.forward(toks[13:20]), lb_model.forward(toks[13:20]))


def test_reset_rerun_is_bitwise_identical_and_thread_count_free():
    cfg, W = tiny()
    toks = synth.make_prompt(cfg, 10)
    m = oracle.Model(cfg, W)
    a = m.forward(toks)
    m.reset()
    assert m.kv_len == 0
    b = m.forward(toks)
    assert np.array_equal(a, b)
    n0 = oracle.threads()
    oracle.set_threads(1)
    try:
        m.reset()
        c = m.forward(toks)
    finally:
        oracle.set_threads(n0)
    assert np.array_equal(a, c)


def test_kv_rows_and_positions():
    cfg, W = tiny(arch="llama")
    toks = synth.make_prompt(cfg, 5)
    m = oracle.Model(cfg, W)
    m.forward(toks)
    assert m.kv_len == 5
    # layer 0, position 0: k = W_k rmsnorm(embed(t0)), RoPE at 0 is identity
    x = oracle.embed(W["token_embd.weight"], int(toks[0]))
    h = oracle.rmsnorm(x, W["blk.0.attn_norm.weight"], cfg["rms_eps"])
    k = oracle.matvec(W["blk.0.attn_k.weight"], h)
    v = oracle.matvec(W["blk.0.attn_v.weight"], h)
    hd = cfg["head_dim"]
    assert np.array_equal(m.kv_read(0, 0, 0, 1).reshape(-1), k)
    assert np.array_equal(m.kv_read(0, 1, 0, 1).reshape(-1), v)
    # layer 0, position 3: that token's k rotated by RoPE at position 3
    c, s = oracle.rope_table(8, hd, cfg["rope_theta"])
    x3 = oracle.embed(W["token_embd.weight"], int(toks[3]))
    h3 = oracle.rmsnorm(x3, W["blk.0.attn_norm.weight"], cfg["rms_eps"])
    k3 = oracle.rope(oracle.matvec(W["blk.0.attn_k.weight"], h3), hd, c[3], s[3])
    assert np.array_equal(m.kv_read(0, 0, 3, 1).reshape(-1), k3)
    with pytest.raises(RuntimeError):
        m.forward(np.zeros(cfg["max_ctx"], np.int32))
    assert m.kv_len == 5
    with pytest.raises(RuntimeError):
        m.forward([cfg["vocab"]])


# ---- planted mistakes -----------------------------------------------------

def _brute_tiny_fails(arch):
    cfg, W = tiny(arch=arch)
    toks = synth.make_prompt(cfg, 12)
    got = run_token_by_token(cfg, W, toks)
    ref = forward_all(cfg, W, toks)
    worst = max(rel_l2(got[s], ref[s]) for s in range(len(toks)))
    return not worst <= 1e-4  # NaN counts as caught


def _rmsnorm_closed_form_fails():
    x = np.full(64, 1e-3, np.float32)
    got = oracle.rmsnorm(x, np.ones(64, np.float32), 1e-6)
    ref = 1e-3 / np.sqrt(1e-6 + 1e-6)
    return abs(float(got[0]) - ref) > 1e-5


def _one_hot_fails():
    W = (0.02 * np.random.default_rng(1).standard_normal((8, 8))).astype(np.float32)
    h = np.zeros(8, np.float32)
    h[3] = 1.0
    return not np.array_equal(oracle.matvec(W, h), W[:, 3])


def _gelu_fails():
    # the tanh form sits 1e-4..1e-3 away from the erf form near |x| = 2
    x = np.linspace(-4, 4, 801).astype(np.float32)
    from math import erf
    ge = np.array([0.5 * v * (1 + erf(v / np.sqrt(2.0))) for v in x.astype(np.float64)])
    dev = np.max(np.abs(oracle.gelu_tanh(x).astype(np.float64) - ge))
    return not (1e-4 < dev < 1e-3)


def _kv_row_fails():
    # K cached at position 0 of layer 0 is the unrotated k of token 0 (RoPE
    # at position 0 is the identity). A constant position offset leaves the
    # logits unchanged (scores depend only on m - n) but not the cache.
    cfg, W = tiny(arch="llama")
    toks = synth.make_prompt(cfg, 2)
    m = oracle.Model(cfg, W)
    m.forward(toks)
    x = oracle.embed(W["token_embd.weight"], int(toks[0]))
    h = oracle.rmsnorm(x, W["blk.0.attn_norm.weight"], cfg["rms_eps"])
    k = oracle.matvec(W["blk.0.attn_k.weight"], h)
    return not np.array_equal(m.kv_read(0, 0, 0, 1).reshape(-1), k)


@pytest.mark.parametrize("mutation", [m for m in oracle.MUTATIONS if m != "none"])
def test_each_planted_mistake_is_caught(mutation):
    oracle.set_mutation(mutation)
    try:
        caught = (_rmsnorm_closed_form_fails() or _one_hot_fails()
                  or _kv_row_fails() or _gelu_fails()
                  or _brute_tiny_fails("qwen3") or _brute_tiny_fails("llama")
                  or _brute_tiny_fails("qwen2") or _brute_tiny_fails("gemma3"))
    finally:
        oracle.set_mutation("none")
    assert caught, mutation


def test_pins_pass_without_mistakes():
    assert not _rmsnorm_closed_form_fails()
    assert not _one_hot_fails()
    assert not _kv_row_fails()
    assert not _gelu_fails()
    assert not _brute_tiny_fails("qwen3")
    assert not _brute_tiny_fails("llama")
    assert not _brute_tiny_fails("qwen2")
    assert not _brute_tiny_fails("gemma3")
