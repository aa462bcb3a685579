"""Independent float64 brute force of the decoder, for pinning the oracle.

A different formulation from the oracle on purpose: the whole sequence at
once as matrices, an explicit causal mask instead of a KV cache, RoPE as a
complex multiplication, softmax over a masked score matrix, everything in
float64 with no intermediate rounding. Tiny shapes only.

Follows the step list of page "Local inference and architectures", section
"The format"; readings of the open points are the same as the oracle's
(rotate-half RoPE pairs unless the config asks for adjacent ones, eps inside
the root, scale 1/sqrt(hd), GQA head j on KV head j // group, qwen2's biases
added right after their matmuls; gemma3: embedding times f32(sqrt(d)),
q/k head norms, an rms_norm on the o and down outputs before each residual
add, gelu_tanh, and on the pattern's local layers a window of W positions
with the local RoPE theta).
"""
from __future__ import annotations

import numpy as np


def dequant(W: np.ndarray, K: int) -> np.ndarray:
    """float64 [N, K] from f32 / f16 [N, K] or 8-bit blocks [N, K/32*34]."""
    if W.dtype != np.uint8:
        return W.astype(np.float64)
    N = W.shape[0]
    blocks = W.reshape(N, K // 32, 34)
    scale = np.ascontiguousarray(blocks[:, :, 0:2]).view(np.float16)[..., 0]
    q = np.ascontiguousarray(blocks[:, :, 2:]).view(np.int8)
    return (scale.astype(np.float64)[:, :, None] * q.astype(np.float64)).reshape(N, K)


def rms(X: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    w = w.reshape(-1).astype(np.float64)
    return X / np.sqrt(np.mean(X * X, axis=-1, keepdims=True) + eps) * w


def rope_complex(T: np.ndarray, pos: np.ndarray, theta: float,
                 pairing: str = "halves") -> np.ndarray:
    """T [S, heads, hd]; pair i as the complex a + i b, with (a, b) =
    (t[i], t[i + hd/2]) for "halves" or (t[2i], t[2i+1]) for "adjacent"."""
    hd = T.shape[-1]
    half = hd // 2
    inv = theta ** (-2.0 * np.arange(half) / hd)
    ang = pos[:, None].astype(np.float64) * inv[None, :]
    if pairing == "adjacent":
        z = T[..., 0::2] + 1j * T[..., 1::2]
    else:
        z = T[..., :half] + 1j * T[..., half:]
    z = z * np.exp(1j * ang)[:, None, :]
    if pairing == "adjacent":
        out = np.empty(T.shape)
        out[..., 0::2] = z.real
        out[..., 1::2] = z.imag
        return out
    return np.concatenate([z.real, z.imag], axis=-1)


def forward_all(cfg: dict, W: dict, tokens) -> np.ndarray:
    """Logits [S, vocab] for every prefix of `tokens` (positions 0..S-1)."""
    tokens = np.asarray(tokens)
    S = tokens.size
    d, hd = cfg["d_model"], cfg["head_dim"]
    nh, nkv, F = cfg["n_heads"], cfg["n_kv_heads"], cfg["ffn_dim"]
    eps, theta = cfg["rms_eps"], cfg["rope_theta"]
    group = nh // nkv
    pos = np.arange(S)
    E = W["token_embd.weight"].astype(np.float64)
    X = E[tokens]
    gemma = cfg["arch"] == "gemma3"
    if gemma:
        X = X * float(np.float32(np.sqrt(d)))
    mask = np.triu(np.ones((S, S), bool), k=1)  # True where t > s
    Wn = cfg.get("sliding_window", 0)
    far = (pos[:, None] - pos[None, :]) >= Wn if Wn else np.zeros((S, S), bool)
    for i in range(cfg["n_layers"]):
        b = f"blk.{i}."
        local = Wn > 0 and (i + 1) % cfg["window_pattern"] != 0
        th = cfg.get("rope_theta_local") or theta if local else theta
        lmask = mask | far if local else mask
        H = rms(X, W[b + "attn_norm.weight"], eps)
        Q = H @ dequant(W[b + "attn_q.weight"], d).T
        Kx = H @ dequant(W[b + "attn_k.weight"], d).T
        Vx = H @ dequant(W[b + "attn_v.weight"], d).T
        if cfg["arch"] == "qwen2":
            Q = Q + W[b + "attn_q.bias"].reshape(-1).astype(np.float64)
            Kx = Kx + W[b + "attn_k.bias"].reshape(-1).astype(np.float64)
            Vx = Vx + W[b + "attn_v.bias"].reshape(-1).astype(np.float64)
        Q = Q.reshape(S, nh, hd)
        Kx = Kx.reshape(S, nkv, hd)
        Vx = Vx.reshape(S, nkv, hd)
        if cfg["arch"] in ("qwen3", "gemma3"):
            Q = rms(Q, W[b + "attn_q_norm.weight"], eps)
            Kx = rms(Kx, W[b + "attn_k_norm.weight"], eps)
        pairing = cfg.get("rope_pairing", "halves")
        Q = rope_complex(Q, pos, th, pairing)
        Kx = rope_complex(Kx, pos, th, pairing)
        A = np.empty((S, nh, hd))
        for j in range(nh):
            g = j // group
            sc = Q[:, j, :] @ Kx[:, g, :].T / np.sqrt(hd)
            sc[lmask] = -np.inf
            sc = sc - sc.max(axis=1, keepdims=True)
            P = np.exp(sc)
            P /= P.sum(axis=1, keepdims=True)
            A[:, j, :] = P @ Vx[:, g, :]
        O = A.reshape(S, nh * hd) @ dequant(W[b + "attn_output.weight"], nh * hd).T
        if gemma:
            O = rms(O, W[b + "post_attention_norm.weight"], eps)
        X = X + O
        H = rms(X, W[b + "ffn_norm.weight"], eps)
        G = H @ dequant(W[b + "ffn_gate.weight"], d).T
        U = H @ dequant(W[b + "ffn_up.weight"], d).T
        if gemma:
            c = np.sqrt(2.0 / np.pi)
            M = 0.5 * G * (1.0 + np.tanh(c * (G + 0.044715 * G ** 3))) * U
        else:
            M = G / (1.0 + np.exp(-G)) * U
        Dn = M @ dequant(W[b + "ffn_down.weight"], F).T
        if gemma:
            Dn = rms(Dn, W[b + "post_ffw_norm.weight"], eps)
        X = X + Dn
    Y = rms(X, W["output_norm.weight"], eps)
    Wout = W["output.weight"] if "output.weight" in W else W["token_embd.weight"]
    return Y @ dequant(Wout, d).T


def rel_l2(a: np.ndarray, ref: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(a - ref) / np.linalg.norm(ref))
