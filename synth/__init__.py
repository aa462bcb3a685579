"""Seeded synthetic inputs for the decoder forward pass.

This module is the only code shared by the GPU library's callers and the CPU
oracle. It draws numbers and lays them out in the tensor-table format; it
holds none of the forward pass's arithmetic (no norm, no matmul, no
dequantisation, no RoPE).

Tensor names follow the GGUF naming that the architecture-definition format
uses (page "Local inference and architectures", section "The format"):
``token_embd.weight``, ``blk.{i}.attn_norm.weight`` ... ``output.weight``.
Matrices are ``[rows = N_out][cols = K_in]`` row-major, so ``y = W h``.

Value recipe (all seeded, chunked so that generation runs on many threads):

* every tensor draws from ``numpy.random.Generator(PCG64(SeedSequence(
  [base_seed, tensor_id, stream, chunk])))`` with ``chunk`` numbering
  consecutive blocks of ``CHUNK`` elements of the flattened tensor;
  ``tensor_id`` depends only on the name, so a model with fewer layers has
  exactly the first layers of the full model;
* matrices and embeddings: ``standard_normal`` in f32 times 0.02, rounded to
  the storage dtype (RNE);
* norm weights: ``1 + 0.02 * standard_normal`` in f32, rounded likewise;
* q/k/v biases (qwen2): ``BIAS_SCALE * standard_normal``, kept in f32;
* 8-bit blocks: 32 consecutive int8 along K drawn uniformly from
  [-127, 127] (stream 0) plus one f16 scale ``|N(0, 0.02)| / 127`` per block
  (stream 1); host bytes per block are the scale (little-endian f16) then the
  32 values, 34 bytes;
* prompt ids: uniform on [0, vocab) from ``SeedSequence([base_seed, 10**6 +
  stream])``;
* synthetic KV-cache rows: ``standard_normal`` f32 from ``SeedSequence(
  [base_seed, 2 * 10**6 + layer, which, chunk])``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22
# q/k/v biases (qwen2): f32 vectors, N(0, BIAS_SCALE^2); large enough that a
# dropped bias shows in the logits far above the decode tolerance.
BIAS_SCALE = 0.5
Q8_BLOCK = 32
Q8_BLOCK_BYTES = 34

# Model shapes. ``seed`` is the base seed of each workload.
CONFIGS = {
    # 2 layers, d 64, 4/2 heads of 16, ffn 128, vocab 256, tied, all f32
    "tiny": dict(arch="qwen3", n_layers=2, d_model=64, n_heads=4, n_kv_heads=2,
                 head_dim=16, ffn_dim=128, vocab=256, rope_theta=10000.0,
                 rms_eps=1e-6, tied=True, wdtype="f32", seed=1, max_ctx=48,
                 prompt_len=32, decode_steps=16),
    # qwen3-0.6B shape: 28 layers, d 1024, 16/8 heads of 128, ffn 3072,
    # vocab 151936, tied, f16
    "qwen3_0p6b": dict(arch="qwen3", n_layers=28, d_model=1024, n_heads=16,
                       n_kv_heads=8, head_dim=128, ffn_dim=3072, vocab=151936,
                       rope_theta=10000.0, rms_eps=1e-6, tied=True,
                       wdtype="f16", seed=2, max_ctx=768, prompt_len=512,
                       decode_steps=256),
    # llama-8B shape: 32 layers, d 4096, 32/8 heads of 128, ffn 14336,
    # vocab 128256, untied, no Q/K norm, f16
    "llama_8b": dict(arch="llama", n_layers=32, d_model=4096, n_heads=32,
                     n_kv_heads=8, head_dim=128, ffn_dim=14336, vocab=128256,
                     rope_theta=10000.0, rms_eps=1e-6, tied=False,
                     wdtype="f16", seed=3, max_ctx=4224, prompt_len=4096,
                     decode_steps=128),
    # the same llama-8B shape with every matmul weight in 8-bit blocks
    "llama_8b_q8": dict(arch="llama", n_layers=32, d_model=4096, n_heads=32,
                        n_kv_heads=8, head_dim=128, ffn_dim=14336,
                        vocab=128256, rope_theta=10000.0, rms_eps=1e-6,
                        tied=False, wdtype="q8", seed=4, max_ctx=8320,
                        prompt_len=8192, decode_steps=128,
                        contexts=(1024, 8192)),
    # qwen2-7B shape: 28 layers, d 3584, 28/4 heads of 128 (7 query heads
    # per KV head), ffn 18944, vocab 152064, untied, q/k/v biases, f16
    "qwen2_7b": dict(arch="qwen2", n_layers=28, d_model=3584, n_heads=28,
                     n_kv_heads=4, head_dim=128, ffn_dim=18944, vocab=152064,
                     rope_theta=1000000.0, rms_eps=1e-6, tied=False,
                     wdtype="f16", seed=6, max_ctx=4224, prompt_len=4096,
                     decode_steps=64),
    # gemma3-style tiny model: 2 layers (a local layer with a window of 8
    # positions, then a global one), d 64, 4/2 heads of 16, ffn 128, vocab
    # 256, tied, f32
    "tiny_gemma3": dict(arch="gemma3", n_layers=2, d_model=64, n_heads=4, n_kv_heads=2,
                        head_dim=16, ffn_dim=128, vocab=256, rope_theta=1000000.0,
                        rope_theta_local=10000.0, sliding_window=8, window_pattern=2,
                        rms_eps=1e-6, tied=True, wdtype="f32", seed=7, max_ctx=48,
                        prompt_len=32, decode_steps=16),
    # gemma3-4B shape: 34 layers, d 2560, 8/4 heads of 256, ffn 10240, vocab
    # 262208, tied; five local layers (window 1024, theta 1e4) per global
    # one (theta 1e6); post-attention and post-FFN norms, gelu_tanh; f16
    "gemma3_4b": dict(arch="gemma3", n_layers=34, d_model=2560, n_heads=8, n_kv_heads=4,
                      head_dim=256, ffn_dim=10240, vocab=262208, rope_theta=1000000.0,
                      rope_theta_local=10000.0, sliding_window=1024, window_pattern=6,
                      rms_eps=1e-6, tied=True, wdtype="f16", seed=8, max_ctx=4224,
                      prompt_len=4096, decode_steps=64),
    # qwen3-8B shape: 36 layers, d 4096, 32/8 heads of 128, ffn 12288,
    # vocab 151936, untied, per-head Q/K norm, f16
    "qwen3_8b": dict(arch="qwen3", n_layers=36, d_model=4096, n_heads=32,
                     n_kv_heads=8, head_dim=128, ffn_dim=12288, vocab=151936,
                     rope_theta=10000.0, rms_eps=1e-6, tied=False,
                     wdtype="f16", seed=5, max_ctx=2112, prompt_len=2048,
                     decode_steps=64),
}

LAYER_SLOTS = ("attn_norm", "attn_q", "attn_k", "attn_v", "attn_q_norm",
               "attn_k_norm", "attn_output", "ffn_norm", "ffn_gate",
               "ffn_up", "ffn_down", "attn_q.bias", "attn_k.bias",
               "attn_v.bias", "post_attention_norm", "post_ffw_norm")


def config(name: str, **overrides) -> dict:
    """A copy of a named shape with fields overridden (e.g. n_layers=2)."""
    cfg = dict(CONFIGS[name])
    cfg["name"] = name
    cfg.update(overrides)
    return cfg


def tensor_id(name: str) -> int:
    """A stable stream id per tensor name, independent of the layer count."""
    if name == "token_embd.weight":
        return 0
    if name == "output_norm.weight":
        return 1
    if name == "output.weight":
        return 2
    _, i, slot, kind = name.split(".")
    key = slot + ".bias" if kind == "bias" else slot
    return 100 + 16 * int(i) + LAYER_SLOTS.index(key)


def tensor_specs(cfg: dict) -> list[tuple[str, str, int, int]]:
    """(name, kind, rows, cols) for every tensor of the model.

    kind is "embed", "norm" or "matmul"; norms are vectors with rows = 1.
    """
    d, F, V = cfg["d_model"], cfg["ffn_dim"], cfg["vocab"]
    hd = cfg["head_dim"]
    qd, kvd = cfg["n_heads"] * hd, cfg["n_kv_heads"] * hd
    specs = [("token_embd.weight", "embed", V, d)]
    for i in range(cfg["n_layers"]):
        b = f"blk.{i}."
        specs += [(b + "attn_norm.weight", "norm", 1, d),
                  (b + "attn_q.weight", "matmul", qd, d),
                  (b + "attn_k.weight", "matmul", kvd, d),
                  (b + "attn_v.weight", "matmul", kvd, d)]
        if cfg["arch"] == "qwen2":
            specs += [(b + "attn_q.bias", "bias", 1, qd),
                      (b + "attn_k.bias", "bias", 1, kvd),
                      (b + "attn_v.bias", "bias", 1, kvd)]
        if cfg["arch"] in ("qwen3", "gemma3"):
            specs += [(b + "attn_q_norm.weight", "norm", 1, hd),
                      (b + "attn_k_norm.weight", "norm", 1, hd)]
        specs += [(b + "attn_output.weight", "matmul", d, qd),
                  (b + "ffn_norm.weight", "norm", 1, d),
                  (b + "ffn_gate.weight", "matmul", F, d),
                  (b + "ffn_up.weight", "matmul", F, d),
                  (b + "ffn_down.weight", "matmul", d, F)]
        if cfg["arch"] == "gemma3":
            specs += [(b + "post_attention_norm.weight", "norm", 1, d),
                      (b + "post_ffw_norm.weight", "norm", 1, d)]
    specs.append(("output_norm.weight", "norm", 1, d))
    if not cfg["tied"]:
        specs.append(("output.weight", "matmul", V, d))
    return specs


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _threads(threads):
    if threads:
        return threads
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _fill_chunks(out_flat: np.ndarray, key: tuple, draw, pool) -> None:
    """out_flat[c*CHUNK:(c+1)*CHUNK] = draw(rng(key + (c,)), n) for every c."""
    n = out_flat.size
    nchunk = (n + CHUNK - 1) // CHUNK

    def one(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        out_flat[lo:hi] = draw(_rng(*key, c), hi - lo)

    list(pool.map(one, range(nchunk)))


def _normal(scale: float, offset: float, dtype):
    def draw(rng, n):
        z = rng.standard_normal(n, dtype=np.float32)
        z *= np.float32(scale)
        if offset:
            z += np.float32(offset)
        return z.astype(dtype)
    return draw


def _q8_values(rng, n):
    return rng.integers(-127, 128, size=n, dtype=np.int8)


def _q8_scales(rng, n):
    z = rng.standard_normal(n, dtype=np.float32)
    return (np.abs(z) * np.float32(0.02) / np.float32(127.0)).astype(np.float16)


def make_tensor(cfg: dict, name: str, kind: str, rows: int, cols: int,
                pool=None) -> np.ndarray:
    """Draw one tensor. Returns float32 / float16 [rows, cols], or for 8-bit
    blocks a uint8 array [rows, cols/32*34] of packed blocks."""
    own = pool is None
    if own:
        pool = ThreadPoolExecutor(_threads(None))
    try:
        base, tid = cfg["seed"], tensor_id(name)
        wd = cfg["wdtype"]
        if kind == "matmul" and wd == "q8":
            if cols % Q8_BLOCK:
                raise ValueError(f"{name}: cols {cols} not a multiple of 32")
            nblk = cols // Q8_BLOCK
            q = np.empty(rows * cols, np.int8)
            _fill_chunks(q, (base, tid, 0), _q8_values, pool)
            s = np.empty(rows * nblk, np.float16)
            _fill_chunks(s, (base, tid, 1), _q8_scales, pool)
            out = np.empty((rows, nblk, Q8_BLOCK_BYTES), np.uint8)
            out[:, :, 0:2] = s.view(np.uint8).reshape(rows, nblk, 2)
            out[:, :, 2:] = q.view(np.uint8).reshape(rows, nblk, Q8_BLOCK)
            return out.reshape(rows, nblk * Q8_BLOCK_BYTES)
        dtype = np.float32 if wd == "f32" or kind == "bias" else np.float16
        out = np.empty(rows * cols, dtype)
        if kind == "norm":
            _fill_chunks(out, (base, tid, 0), _normal(0.02, 1.0, dtype), pool)
        elif kind == "bias":
            _fill_chunks(out, (base, tid, 0), _normal(BIAS_SCALE, 0.0, np.float32), pool)
        else:
            _fill_chunks(out, (base, tid, 0), _normal(0.02, 0.0, dtype), pool)
        return out.reshape(rows, cols)
    finally:
        if own:
            pool.shutdown()


def make_weights(cfg: dict, threads: int | None = None) -> dict[str, np.ndarray]:
    """All tensors of the model, keyed by GGUF name."""
    out = {}
    with ThreadPoolExecutor(_threads(threads)) as pool:
        for name, kind, rows, cols in tensor_specs(cfg):
            out[name] = make_tensor(cfg, name, kind, rows, cols, pool)
    return out


def make_prompt(cfg: dict, n: int, stream: int = 0) -> np.ndarray:
    """n token ids uniform on [0, vocab), int32."""
    rng = _rng(cfg["seed"], 10**6 + stream)
    return rng.integers(0, cfg["vocab"], size=n, dtype=np.int64).astype(np.int32)


def make_kv_rows(cfg: dict, layer: int, n_pos: int, pool=None):
    """Synthetic cache rows for one layer: (K, V), each f32 [n_kv, n_pos, hd]
    drawn N(0, 1). Used to stand a long context up without prefilling it."""
    shape = (cfg["n_kv_heads"], n_pos, cfg["head_dim"])
    own = pool is None
    if own:
        pool = ThreadPoolExecutor(_threads(None))
    try:
        res = []
        for which in (0, 1):
            a = np.empty(int(np.prod(shape)), np.float32)
            _fill_chunks(a, (cfg["seed"], 2 * 10**6 + layer, which),
                         _normal(1.0, 0.0, np.float32), pool)
            res.append(a.reshape(shape))
        return tuple(res)
    finally:
        if own:
            pool.shutdown()


def weight_bytes(cfg: dict) -> int:
    """Bytes of every matmul weight, embedding and norm as stored on the host."""
    total = 0
    for name, kind, rows, cols in tensor_specs(cfg):
        if kind == "matmul" and cfg["wdtype"] == "q8":
            total += rows * cols // Q8_BLOCK * Q8_BLOCK_BYTES
        elif kind == "bias":
            total += rows * cols * 4
        else:
            total += rows * cols * (4 if cfg["wdtype"] == "f32" else 2)
    return total


def make_weights_device(cfg: dict, device="cuda") -> dict:
    """The same distributions drawn on the GPU with torch's generator (one
    seeded stream per tensor: seed = base * 1000003 + tensor_id). Used where
    a run needs full-size random weights fast and does not compare with the
    oracle (benchmarks); parity tests use make_weights."""
    import torch
    out = {}
    g = torch.Generator(device=device)
    for name, kind, rows, cols in tensor_specs(cfg):
        g.manual_seed(cfg["seed"] * 1000003 + tensor_id(name))
        wd = cfg["wdtype"]
        if kind == "matmul" and wd == "q8":
            nblk = cols // Q8_BLOCK
            q = torch.randint(-127, 128, (rows, nblk, Q8_BLOCK), device=device,
                              generator=g, dtype=torch.int8)
            s = (torch.randn(rows, nblk, 1, device=device, generator=g).abs()
                 * 0.02 / 127.0).half()
            blk = torch.empty(rows, nblk, Q8_BLOCK_BYTES, dtype=torch.uint8, device=device)
            blk[:, :, 0:2] = s.view(torch.uint8)
            blk[:, :, 2:] = q.view(torch.uint8)
            out[name] = blk.reshape(rows, nblk * Q8_BLOCK_BYTES)
            continue
        dtype = torch.float32 if wd == "f32" else torch.float16
        z = torch.randn(rows, cols, device=device, generator=g) * 0.02
        if kind == "norm":
            z += 1.0
        if kind == "bias":
            z = z * (BIAS_SCALE / 0.02)
            out[name] = z.to(torch.float32)
            continue
        out[name] = z.to(dtype)
    return out


def make_kv_rows_device(cfg: dict, layer: int, n_pos: int, device="cuda"):
    """Synthetic cache rows (K, V) f32 [n_kv, n_pos, hd] ~ N(0, 1) on the GPU."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(cfg["seed"] * 1000003 + 2 * 10**6 + layer)
    shape = (cfg["n_kv_heads"], n_pos, cfg["head_dim"])
    return (torch.randn(shape, device=device, generator=g),
            torch.randn(shape, device=device, generator=g))
