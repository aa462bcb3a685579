"""The f16 copies of the KV cache that the bulk-prefill attention reads
(head_dim 64 and 128 with f16 or 8-bit block weights).

Every cache row a later bulk call reads must be in the copies, whichever
path wrote it: a bulk call's own rows (the other prefill tests), rows
appended one at a time by decode steps, and rows restored with
df_write_kv. Each case ends in a bulk call whose keys span all of these,
checked against the oracle fed the same tokens (and the same restored rows)
one position at a time, at the bulk tolerance (page "Execution contract",
"Forward phase": bulk and token-by-token agree within epsilon).
"""
import numpy as np
import pytest

import oracle
import synth
from parity import first_argmax, rel_l2

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


def check(got, ref, what, bulk=True):
    """rel-L2 within the bulk tolerance. After a bulk call the greedy token
    must be identical; after a decode step too, unless the reference's top
    two logits are closer than twice the largest difference seen (a genuine
    near-tie, where either token is correct)."""
    e = rel_l2(got, ref)
    say(f"  {what}: rel-L2 {e:.2e}")
    assert e <= TOL, f"{what}: rel-L2 {e:.3e}"
    top2 = np.sort(np.asarray(ref, np.float64))[-2:]
    if bulk or top2[1] - top2[0] > 2.0 * float(np.max(np.abs(np.asarray(got, np.float64) - ref))):
        assert first_argmax(got) == first_argmax(ref), f"{what}: greedy token differs"


@pytest.mark.parametrize("hd,n_heads,n_kv,wdtype", [(128, 8, 2, "f16"), (64, 6, 3, "f16"),
                                                     (128, 4, 4, "q8")])
def test_bulk_reads_rows_appended_by_decode(dfa, hd, n_heads, n_kv, wdtype):
    # bulk 50, then 9 decode steps (rows 50..58 reach the copies through the
    # decode attention), then bulk 61 whose keys 0..119 span both kinds of
    # rows and two 64-key tiles, then 2 more decode steps
    say(f"[tiny qwen3 {wdtype}, head_dim {hd}, {n_heads}/{n_kv} heads] bulk 50 + 9 decode + bulk 61 + 2 decode")
    extra = dict(d_model=192, ffn_dim=416) if wdtype == "q8" else {}
    cfg = synth.config("tiny", wdtype=wdtype, head_dim=hd, n_heads=n_heads, n_kv_heads=n_kv,
                       max_ctx=160, **extra)
    W = synth.make_weights(cfg)
    toks = synth.make_prompt(cfg, 120)
    om = oracle.Model(cfg, W, max_ctx=160)
    m = dfa.Model(cfg, W)
    for t in toks[:49]:
        om.forward([t], logits=False)
    check(m.forward(toks[:50]).cpu().numpy().copy(), om.forward([toks[49]]), "after bulk 50")
    nxt = [int(t) for t in toks[50:59]]
    for i, t in enumerate(nxt):
        check(m.forward([t]).cpu().numpy().copy(), om.forward([t]), f"decode {i}", bulk=False)
    for t in toks[59:119]:
        om.forward([t], logits=False)
    ref = om.forward([toks[119]])
    got = m.forward(toks[59:120]).cpu().numpy().copy()
    assert m.kv_len == 120
    check(got, ref, "after bulk 61 on top")
    t = first_argmax(ref)
    for i in range(2):
        r = om.forward([t])
        check(m.forward([t]).cpu().numpy().copy(), r, f"decode after bulk {i}", bulk=False)
        t = first_argmax(r)
    m.close()


@pytest.mark.parametrize("hd,n_heads,n_kv", [(128, 8, 2), (64, 4, 2)])
def test_bulk_on_restored_rows(dfa, hd, n_heads, n_kv):
    # 130 synthetic rows restored with df_write_kv (K and V in separate
    # calls, the copies follow each), then a bulk call of 45 tokens on top:
    # its keys are the restored rows and its own
    n_ctx = 130
    say(f"[tiny llama f16, head_dim {hd}, {n_heads}/{n_kv} heads] {n_ctx} restored rows + bulk 45")
    cfg = synth.config("tiny", arch="llama", wdtype="f16", head_dim=hd, n_heads=n_heads,
                       n_kv_heads=n_kv, max_ctx=192)
    W = synth.make_weights(cfg)
    om = oracle.Model(cfg, W, max_ctx=192)
    m = dfa.Model(cfg, W)
    for layer in range(cfg["n_layers"]):
        K, V = synth.make_kv_rows(cfg, layer, n_ctx)
        om.kv_write(layer, 0, 0, K)
        om.kv_write(layer, 1, 0, V)
        m.write_kv(layer, 0, 0, K, n_ctx)
        m.write_kv(layer, 1, 0, V, n_ctx)
    om.set_kv_len(n_ctx)
    toks = synth.make_prompt(cfg, 45, stream=2)
    for t in toks[:-1]:
        om.forward([t], logits=False)
    ref = om.forward([toks[-1]])
    got = m.forward(toks).cpu().numpy().copy()
    assert m.kv_len == n_ctx + 45
    check(got, ref, f"bulk 45 on {n_ctx} restored rows")
    # rewriting some restored rows must reach the copies too: overwrite
    # rows 10..19 of every layer on both sides, rewind to 130 and run the
    # bulk call again
    for layer in range(cfg["n_layers"]):
        K, V = synth.make_kv_rows(cfg, layer, 20)
        K2, V2 = np.ascontiguousarray(K[:, 10:] * -0.5), np.ascontiguousarray(V[:, 10:] * 2.0)
        om.kv_write(layer, 0, 10, K2)
        om.kv_write(layer, 1, 10, V2)
        m.write_kv(layer, 0, 10, K2, n_ctx)
        m.write_kv(layer, 1, 10, V2, n_ctx)
    om.set_kv_len(n_ctx)
    for t in toks[:-1]:
        om.forward([t], logits=False)
    ref2 = om.forward([toks[-1]])
    got2 = m.forward(toks).cpu().numpy().copy()
    assert rel_l2(ref2, ref) > 1e-3, "the rewrite did not change the reference"
    check(got2, ref2, "bulk 45 after rewriting rows 10..19")
    m.close()


@pytest.mark.parametrize("hd", [128, 64])
def test_stale_rows_past_the_context_do_not_leak(dfa, hd):
    # rows 0..127 restored with values that have no f16 form (1e6 -> inf in
    # the copies) and NaNs, then a reset: a bulk call of 45 tokens reads a
    # 64-key tile whose keys 45..63 still hold those rows in the copies; they
    # must weigh exactly nothing, as in a fresh model
    say(f"[tiny llama f16, head_dim {hd}] stale non-finite rows, reset, bulk 45")
    cfg = synth.config("tiny", arch="llama", wdtype="f16", head_dim=hd, n_heads=4, n_kv_heads=2, max_ctx=192)
    W = synth.make_weights(cfg)
    m = dfa.Model(cfg, W)
    for layer in range(cfg["n_layers"]):
        K, V = synth.make_kv_rows(cfg, layer, 128)
        K = np.full_like(K, 1e6)
        V = np.full_like(V, 1e6)
        V[..., 1::2, :] = np.nan
        m.write_kv(layer, 0, 0, np.ascontiguousarray(K), 128)
        m.write_kv(layer, 1, 0, np.ascontiguousarray(V), 128)
    m.reset()
    om = oracle.Model(cfg, W, max_ctx=192)
    toks = synth.make_prompt(cfg, 45, stream=4)
    for t in toks[:-1]:
        om.forward([t], logits=False)
    ref = om.forward([toks[-1]])
    got = m.forward(toks).cpu().numpy().copy()
    assert np.all(np.isfinite(got)), "non-finite logits"
    check(got, ref, "bulk 45 after a reset over non-finite rows")
    m.close()
