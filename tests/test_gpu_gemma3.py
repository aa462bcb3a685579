"""gemma3-style decoder on the GPU against the oracle: the embedding scale,
norm_heads, the rms_norm of the o and down outputs before each residual add,
gelu_tanh, and sliding-window attention with the local RoPE theta on the
pattern's local layers.

Bars as for the other architectures: decode logits rel-L2 <= 1e-4 (f32 /
f16 weights) or 1e-3 (8-bit blocks), teacher-forced, argmax identical off
near-ties; bulk prefill <= 5e-3; KV rows within the same bars. Windows are
exercised where they start inside an attention tile and span several tiles
(decode) and inside a 16-row query block (prefill); head_dim 256 (the
gemma3 shapes') with 1, 2 and 4 query heads per KV head.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check_steps, first_argmax, oracle_greedy, rel_l2

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


def tiny(**over):
    cfg = synth.config("tiny_gemma3", **over)
    return cfg, synth.make_weights(cfg)


def decode_case(dfa, cfg, W, n_prompt, n_decode, tol, **model_kw):
    prompt = synth.make_prompt(cfg, n_prompt)
    fed, ref = oracle_greedy(cfg, W, prompt, n_decode, max_ctx=cfg["max_ctx"])
    m = dfa.Model(cfg, W, **model_kw)
    got = [m.forward([t]).cpu().numpy().copy() for t in fed]
    worst, ties = check_steps(got, ref, tol, cfg["name"])
    say(f"  worst rel-L2 {worst:.2e}, near-ties {ties}")
    om = oracle.Model(cfg, W)
    om.forward(fed, logits=False)
    for layer in range(cfg["n_layers"]):
        for which in (0, 1):
            a = m.read_kv(layer, which, 0, len(fed))
            b = om.kv_read(layer, which, 0, len(fed))
            assert np.linalg.norm(a - b) / np.linalg.norm(b) <= tol, (layer, which)
    om.close()
    return m


@pytest.mark.parametrize("wdtype,over", [
    ("f32", {}), ("f16", {}), ("q8", {}),
    ("f16", dict(rope_pairing="adjacent", n_heads=6, n_kv_heads=2))],
    ids=lambda v: "-".join(f"{k}{x}" for k, x in v.items()) if isinstance(v, dict) else str(v))
def test_tiny_decode(dfa, wdtype, over):
    cfg, W = tiny(wdtype=wdtype, **over)
    say(f"[tiny gemma3 {wdtype} {over}] window 8 on layer 0, 32-token prompt + 16 greedy steps")
    m = decode_case(dfa, cfg, W, 32, 16, 1e-3 if wdtype == "q8" else 1e-4)
    m.close()


def test_window_across_tiles(dfa):
    # window 150 over positions up to ~330: the window starts inside a
    # 64-row tile and covers several; the global layer reads everything
    cfg, W = tiny(wdtype="f16", sliding_window=150, window_pattern=2, max_ctx=352)
    say("[tiny gemma3 f16] window 150, 300-token prompt + 24 greedy steps")
    m = decode_case(dfa, cfg, W, 300, 24, 1e-4)
    m.close()


@pytest.mark.parametrize("n_heads,n_kv", [(2, 2), (4, 2), (4, 1)])
def test_head_dim_256(dfa, n_heads, n_kv):
    cfg, W = tiny(wdtype="f16", d_model=256, head_dim=256, n_heads=n_heads, n_kv_heads=n_kv,
                  ffn_dim=320, vocab=512, sliding_window=24, max_ctx=96)
    say(f"[gemma3 f16 head_dim 256, {n_heads}/{n_kv} heads] 60-token prompt + 12 steps")
    m = decode_case(dfa, cfg, W, 60, 12, 1e-4)
    # bulk prefill of the same prompt on a fresh model
    toks = synth.make_prompt(cfg, 60)
    m2 = dfa.Model(cfg, W)
    got = m2.forward(toks).cpu().numpy()
    om = oracle.Model(cfg, W)
    for t in toks[:-1]:
        om.forward([t], logits=False)
    ref = om.forward([toks[-1]])
    e = rel_l2(got, ref)
    say(f"  bulk 60: rel-L2 {e:.2e}")
    assert e <= 5e-3
    om.close()
    m2.close()
    m.close()


@pytest.mark.parametrize("wdtype", ["f16", "q8"])
def test_tiny_bulk_then_decode(dfa, wdtype):
    cfg, W = tiny(wdtype=wdtype, sliding_window=24, d_model=192, ffn_dim=416, max_ctx=160)
    say(f"[tiny gemma3 {wdtype}] window 24: bulk 101 + bulk 23 on top + 6 decode steps")
    toks = synth.make_prompt(cfg, 124)
    om = oracle.Model(cfg, W, max_ctx=160)
    refs = []
    for ch in (toks[:101], toks[101:]):
        for t in ch[:-1]:
            om.forward([t], logits=False)
        refs.append(om.forward([ch[-1]]))
    m = dfa.Model(cfg, W)
    g1 = m.forward(toks[:101]).cpu().numpy().copy()
    g2 = m.forward(toks[101:]).cpu().numpy().copy()
    for g, r, what in ((g1, refs[0], "after 101"), (g2, refs[1], "after 124")):
        e = rel_l2(g, r)
        say(f"  {what}: rel-L2 {e:.2e}")
        assert e <= 5e-3
        assert first_argmax(g) == first_argmax(r), what
    for layer in range(cfg["n_layers"]):
        for which in (0, 1):
            a = m.read_kv(layer, which, 0, 124)
            b = om.kv_read(layer, which, 0, 124)
            assert np.linalg.norm(a - b) / np.linalg.norm(b) <= 5e-3
    nxt = first_argmax(refs[1])
    for i in range(6):
        r = om.forward([nxt])
        g = m.forward([nxt]).cpu().numpy()
        assert rel_l2(g, r) <= 5e-3, i
        nxt = first_argmax(r)
    om.close()
    m.close()


def test_gemma3_4b_shape_two_layers_bulk(dfa):
    # the 4B layer shape (d 2560, 8/4 heads of 256, ffn 10240) with a local
    # and a global layer; the window shortened to 128 so that a 300-token
    # prompt crosses it while the oracle stays within seconds
    cfg = synth.config("gemma3_4b", n_layers=2, window_pattern=2, sliding_window=128,
                       vocab=4096, max_ctx=320)
    S = 300
    say(f"[gemma3-4B layer shape, 2 layers (local, global), window 128, vocab 4096] "
        f"bulk {S} + 1 decode step")
    W = synth.make_weights(cfg)
    toks = synth.make_prompt(cfg, S)
    om = oracle.Model(cfg, W)
    om.forward(toks[:-1], logits=False)
    ref = om.forward([toks[-1]])
    m = dfa.Model(cfg, W)
    got = m.forward(toks).cpu().numpy()
    e = rel_l2(got, ref)
    say(f"  bulk {S}: rel-L2 {e:.2e}")
    assert e <= 5e-3
    assert first_argmax(got) == first_argmax(ref)
    t = first_argmax(ref)
    e2 = rel_l2(m.forward([t]).cpu().numpy(), om.forward([t]))
    say(f"  next decode step: rel-L2 {e2:.2e}")
    assert e2 <= 5e-3
    om.close()
    m.close()
