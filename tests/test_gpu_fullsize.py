"""Parity at the full sizes the benchmark runs, through the C ABI, on
outputs the oracle can compute.

* llama-8B shape, f16, all 32 layers: the KV cache of both sides is restored
  to 4096 synthetic positions, then decode steps at p = 4096.. are compared
  (logits rel-L2 <= 1e-4) -- the bench's decode launch configuration.
* the same shape with 8-bit blocks at contexts 1024 and 8192 (<= 1e-3).
* qwen2-7B shape, f16, all 28 layers (q/k/v biases, 7 query heads per KV
  head), decode at p = 4096 on a restored cache (<= 1e-4).
* gemma3-4B shape, f16, all 34 layers (head_dim 256, sliding windows of
  1024 on the local layers), decode at p = 4096 on a restored cache.
* qwen3-8B shape, all 36 layers, one bulk prefill of 2048 tokens: against
  GPU token-by-token (<= 5e-3, greedy token identical), and layer 0's K / V
  cache rows at sampled positions against the oracle's step functions (a
  layer-0 row depends on its own token only). The oracle checks the same
  kernels at these widths over 2 layers in test_gpu_fullwidth_oracle.py.
* llama-8B shape with 8-bit blocks, all 32 layers, bulk prefill of 1024 and
  2100 tokens against GPU token-by-token.

Weights come from synth's seeded device generator and are copied to host
for the oracle.
"""
import numpy as np
import pytest

import oracle
import synth
from parity import check_steps, first_argmax, rel_l2

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


def host_copy(Wd):
    return {k: v.cpu().numpy() for k, v in Wd.items()}


def restored_decode(dfa, cfg, ctx, n_steps, tol):
    import torch
    Wd = synth.make_weights_device(cfg)
    torch.cuda.synchronize()
    W = host_copy(Wd)
    m = dfa.Model(cfg, Wd, max_ctx=ctx + n_steps + 1)
    del Wd
    torch.cuda.empty_cache()
    om = oracle.Model(cfg, W, max_ctx=ctx + n_steps + 1)
    for layer in range(cfg["n_layers"]):
        K, V = synth.make_kv_rows(cfg, layer, ctx)
        om.kv_write(layer, 0, 0, K)
        om.kv_write(layer, 1, 0, V)
        m.write_kv(layer, 0, 0, K, ctx)
        m.write_kv(layer, 1, 0, V, ctx)
    om.set_kv_len(ctx)
    toks = synth.make_prompt(cfg, n_steps, stream=5)
    ref, got = [], []
    for t in toks:
        ref.append(om.forward([t]))
        got.append(m.forward([t]).cpu().numpy().copy())
    worst, ties = check_steps(got, ref, tol, f"{cfg['name']} ctx {ctx}")
    say(f"  worst rel-L2 {worst:.2e}, near-ties {ties}")
    assert m.kv_len == ctx + n_steps
    # the cache row each step appended (layer 0 and the last layer)
    for layer in (0, cfg["n_layers"] - 1):
        a = m.read_kv(layer, 0, ctx, n_steps)
        b = om.kv_read(layer, 0, ctx, n_steps)
        assert np.linalg.norm(a - b) / np.linalg.norm(b) <= tol
    m.close()
    om.close()


def test_llama_8b_f16_decode_at_4096(dfa):
    say("[llama-8B shape, 32 layers, f16] decode at p = 4096, 4097 on a restored cache")
    restored_decode(dfa, synth.config("llama_8b"), 4096, 2, 1e-4)


def test_qwen2_7b_f16_decode_at_4096(dfa):
    say("[qwen2-7B shape, 28 layers, f16, q/k/v biases, 7 heads per KV head] "
        "decode at p = 4096, 4097 on a restored cache")
    restored_decode(dfa, synth.config("qwen2_7b"), 4096, 2, 1e-4)


def test_gemma3_4b_f16_decode_at_4096(dfa):
    say("[gemma3-4B shape, 34 layers, f16, head_dim 256, windows of 1024 on 5 of 6 layers] "
        "decode at p = 4096, 4097 on a restored cache")
    restored_decode(dfa, synth.config("gemma3_4b"), 4096, 2, 1e-4)


@pytest.mark.parametrize("ctx", [1024, 8192])
def test_llama_8b_q8_decode(dfa, ctx):
    say(f"[llama-8B shape, 32 layers, 8-bit blocks] decode at p = {ctx} on a restored cache")
    restored_decode(dfa, synth.config("llama_8b_q8"), ctx, 2, 1e-3)


def test_qwen3_8b_bulk_2048(dfa):
    import torch
    cfg = synth.config("qwen3_8b")
    S = cfg["prompt_len"]
    say(f"[qwen3-8B shape, 36 layers] bulk prefill of {S} vs token-by-token; layer-0 KV vs oracle")
    Wd = synth.make_weights_device(cfg)
    torch.cuda.synchronize()
    toks = synth.make_prompt(cfg, S)
    a = dfa.Model(cfg, Wd, max_ctx=S + 16)
    la = a.forward(toks).cpu().numpy()
    b = dfa.Model(cfg, Wd, max_ctx=S + 16)
    keep = {k: Wd[k].cpu().numpy() for k in ("token_embd.weight", "blk.0.attn_norm.weight",
                                            "blk.0.attn_k.weight", "blk.0.attn_v.weight",
                                            "blk.0.attn_k_norm.weight")}
    del Wd
    torch.cuda.empty_cache()
    for t in toks[:-1]:
        b.forward([t], logits=False)
    lb = b.forward([toks[-1]]).cpu().numpy()
    e = rel_l2(la, lb)
    say(f"  bulk vs token-by-token: rel-L2 {e:.2e}")
    assert e <= 5e-3
    assert first_argmax(la) == first_argmax(lb)
    # layer 0 rows at sampled positions: rope(norm_heads(W_k rmsnorm(E[t])))
    hd, nkv = cfg["head_dim"], cfg["n_kv_heads"]
    c, s = oracle.rope_table(S, hd, cfg["rope_theta"])
    for p in (0, 1, 127, 128, 1000, S - 1):
        x = oracle.embed(keep["token_embd.weight"], int(toks[p]))
        h = oracle.rmsnorm(x, keep["blk.0.attn_norm.weight"], cfg["rms_eps"])
        k = oracle.matvec(keep["blk.0.attn_k.weight"], h).reshape(nkv, hd)
        k = np.stack([oracle.rmsnorm(k[g], keep["blk.0.attn_k_norm.weight"], cfg["rms_eps"])
                      for g in range(nkv)])
        k = oracle.rope(k.reshape(-1), hd, c[p], s[p]).reshape(nkv, hd)
        v = oracle.matvec(keep["blk.0.attn_v.weight"], h).reshape(nkv, hd)
        for m_, tol in ((a, 5e-3), (b, 1e-5)):
            gk = m_.read_kv(0, 0, p, 1)[:, 0, :]
            gv = m_.read_kv(0, 1, p, 1)[:, 0, :]
            assert np.linalg.norm(gk - k) / np.linalg.norm(k) <= tol, p
            assert np.linalg.norm(gv - v) / np.linalg.norm(v) <= tol, p
    # 8 decode steps after the bulk prefill: both models agree
    t = first_argmax(lb)
    for i in range(8):
        ga = a.forward([t]).cpu().numpy()
        gb = b.forward([t]).cpu().numpy()
        assert rel_l2(ga, gb) <= 5e-3, i
        t = first_argmax(gb)
    a.close()
    b.close()


# Rows from which bulk prefill dequantises 8-bit matrices to f16 before the
# GEMMs (the library's PF_DEQUANT_MIN_ROWS).
DEQUANT_FIRST_ROWS = 1024


@pytest.mark.parametrize("S", [1000, 2100])
def test_llama_8b_q8_bulk(dfa, S):
    """8-bit blocks, all 32 layers: one bulk prefill of S tokens against
    GPU token-by-token (5e-3, greedy token identical), and the cache rows of
    the first and last layer. 1000 rows dequantise inside the GEMMs; 2100
    rows convert each matrix to f16 first and run the direct-to-LDS tiles
    over K = 4096 and 14336."""
    import torch
    cfg = synth.config("llama_8b_q8")
    say(f"[llama-8B shape, 32 layers, 8-bit blocks] bulk prefill of {S} vs token-by-token")
    Wd = synth.make_weights_device(cfg)
    torch.cuda.synchronize()
    toks = synth.make_prompt(cfg, S, stream=6)
    a = dfa.Model(cfg, Wd, max_ctx=S + 16)
    la = a.forward(toks).cpu().numpy()
    b = dfa.Model(cfg, Wd, max_ctx=S + 16)
    del Wd
    torch.cuda.empty_cache()
    for t in toks[:-1]:
        b.forward([t], logits=False)
    lb = b.forward([toks[-1]]).cpu().numpy()
    e = rel_l2(la, lb)
    say(f"  bulk vs token-by-token: rel-L2 {e:.2e}")
    assert e <= 5e-3
    assert first_argmax(la) == first_argmax(lb)
    plan = dfa.df_prefill_plan(a.h, S)
    say(f"  GEMM plan: {plan}")
    first = S >= DEQUANT_FIRST_ROWS
    assert all(v[2] == first and v[1] == (not first) for v in plan.values()), plan
    for layer in (0, cfg["n_layers"] - 1):
        for which in (0, 1):
            ka = a.read_kv(layer, which, 0, S)
            kb = b.read_kv(layer, which, 0, S)
            assert np.linalg.norm(ka - kb) / np.linalg.norm(kb) <= 5e-3, (layer, which)
    a.close()
    b.close()
