"""Python face of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg; never by the GPU library or its binding.
It shares no code with the GPU path; only the seeded inputs (``synth``) are
common to both.

Parity status of each function (how it is pinned) is listed in the tests
under tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, F16, Q8 = 0, 1, 2
LLAMA, QWEN3, QWEN2, GEMMA3 = 0, 1, 2, 3
ARCHS = {"llama": LLAMA, "qwen3": QWEN3, "qwen2": QWEN2, "gemma3": GEMMA3}
ROPE_PAIRINGS = {"halves": 0, "adjacent": 1}
# Per-layer tensors in the oracle's slot order (GGUF names after "blk.{i}.").
SLOTS = ("attn_norm.weight", "attn_q.weight", "attn_k.weight",
         "attn_v.weight", "attn_q_norm.weight", "attn_k_norm.weight",
         "attn_output.weight", "ffn_norm.weight", "ffn_gate.weight",
         "ffn_up.weight", "ffn_down.weight", "attn_q.bias", "attn_k.bias",
         "attn_v.bias", "post_attention_norm.weight", "post_ffw_norm.weight")

MUTATIONS = {
    "none": 0, "norm_after_rope": 1, "rope_interleaved": 2,
    "no_attn_residual": 3, "scale_1_over_hd": 4, "gqa_modulo": 5,
    "eps_outside": 6, "exclude_self": 7, "silu_on_up": 8,
    "rope_pos_plus1": 9, "matvec_transpose": 10, "k_bias_after_rope": 11,
    "gelu_erf": 12, "window_plus1": 13, "no_post_attn_norm": 14,
    "global_theta": 15,
}


class Config(C.Structure):
    _fields_ = [("arch", C.c_int32), ("n_layers", C.c_int32),
                ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn_dim", C.c_int32), ("vocab", C.c_int32),
                ("max_ctx", C.c_int32), ("rope_pairing", C.c_int32),
                ("rope_theta", C.c_double), ("rms_eps", C.c_double),
                ("sliding_window", C.c_int32), ("window_pattern", C.c_int32),
                ("rope_theta_local", C.c_double)]


class Tensor(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("pad_", C.c_int32),
                ("data", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        fp, i32, i64, dbl, vp = (C.POINTER(C.c_float), C.c_int32, C.c_int64,
                                 C.c_double, C.c_void_p)
        T = C.POINTER(Tensor)
        L.orc_f16_to_f32.argtypes = [vp, fp, i64]
        L.orc_rmsnorm.argtypes = [fp, T, i32, dbl, fp]
        L.orc_matvec.argtypes = [T, i64, i64, fp, fp]
        L.orc_embed.argtypes = [T, i64, i64, fp]
        L.orc_rope_table.argtypes = [i32, i32, dbl, fp, fp]
        L.orc_rope.argtypes = [fp, i32, i32, fp, fp]
        L.orc_rope_pairs.argtypes = [fp, i32, i32, fp, fp, i32]
        L.orc_add_bias.argtypes = [fp, T, i64]
        L.orc_attention.argtypes = [fp, i32, i32, i32, fp, fp, i64, i32, fp]
        L.orc_silu.argtypes = [fp, i64]
        L.orc_gelu_tanh.argtypes = [fp, i64]
        L.orc_scale.argtypes = [fp, i64, C.c_float]
        L.orc_mul.argtypes = [fp, fp, i64]
        L.orc_create.argtypes = [C.POINTER(Config), T, T, T, T]
        L.orc_create.restype = vp
        L.orc_forward.argtypes = [vp, C.POINTER(C.c_int32), i32, fp]
        L.orc_forward.restype = C.c_int
        L.orc_reset.argtypes = [vp]
        L.orc_kv_len.argtypes = [vp]
        L.orc_kv_len.restype = i32
        L.orc_kv_read.argtypes = [vp, i32, i32, i32, i32, fp]
        L.orc_kv_write.argtypes = [vp, i32, i32, i32, i32, fp]
        L.orc_set_kv_len.argtypes = [vp, i32]
        L.orc_trace.argtypes = [vp]
        L.orc_trace.restype = C.c_char_p
        L.orc_destroy.argtypes = [vp]
        L.orc_set_mutation.argtypes = [i32]
        L.orc_set_f32_accumulate.argtypes = [i32]
        L.orc_set_threads.argtypes = [i32]
        L.orc_get_threads.restype = i32
        _lib = L
    return _lib


def _fp(a: np.ndarray):
    assert a.dtype == np.float32 and a.flags.c_contiguous
    return a.ctypes.data_as(C.POINTER(C.c_float))


def dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.uint8:
        return Q8
    raise TypeError(f"unsupported weight dtype {a.dtype}")


def tensor(a: np.ndarray) -> Tensor:
    a = np.ascontiguousarray(a)
    return Tensor(dtype_code(a), 0, a.ctypes.data)


def set_mutation(name: str) -> None:
    lib().orc_set_mutation(MUTATIONS[name])


def set_f32_accumulate(on: bool) -> None:
    lib().orc_set_f32_accumulate(1 if on else 0)


def set_threads(n: int) -> None:
    lib().orc_set_threads(n)


def threads() -> int:
    return lib().orc_get_threads()


# --- single steps ----------------------------------------------------------

def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.float16)
    out = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32(h.ctypes.data, _fp(out), h.size)
    return out


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    w = np.ascontiguousarray(w)
    out = np.empty_like(x)
    t = tensor(w)
    lib().orc_rmsnorm(_fp(x), C.byref(t), x.size, eps, _fp(out))
    return out


def matvec(W: np.ndarray, h: np.ndarray, K: int | None = None) -> np.ndarray:
    """y = W h for f32/f16 [N, K] or packed 8-bit blocks [N, K/32*34]."""
    W = np.ascontiguousarray(W)
    h = np.ascontiguousarray(h, np.float32)
    N = W.shape[0]
    K = h.size if K is None else K
    y = np.empty(N, np.float32)
    t = tensor(W)
    lib().orc_matvec(C.byref(t), N, K, _fp(h), _fp(y))
    return y


def embed(E: np.ndarray, row: int) -> np.ndarray:
    E = np.ascontiguousarray(E)
    x = np.empty(E.shape[1], np.float32)
    t = tensor(E)
    lib().orc_embed(C.byref(t), row, E.shape[1], _fp(x))
    return x


def rope_table(n_pos: int, hd: int, theta: float):
    c = np.empty((n_pos, hd // 2), np.float32)
    s = np.empty((n_pos, hd // 2), np.float32)
    lib().orc_rope_table(n_pos, hd, theta, _fp(c), _fp(s))
    return c, s


def rope(t: np.ndarray, hd: int, cos_row: np.ndarray, sin_row: np.ndarray,
         pairing: str = "halves") -> np.ndarray:
    t = np.array(t, np.float32, copy=True, order="C")
    cr = np.ascontiguousarray(cos_row, np.float32)
    sr = np.ascontiguousarray(sin_row, np.float32)
    lib().orc_rope_pairs(_fp(t), t.size // hd, hd, _fp(cr), _fp(sr), ROPE_PAIRINGS[pairing])
    return t


def add_bias(y: np.ndarray, b: np.ndarray) -> np.ndarray:
    y = np.array(y, np.float32, copy=True, order="C")
    b = np.ascontiguousarray(b)
    t = tensor(b)
    lib().orc_add_bias(_fp(y), C.byref(t), y.size)
    return y


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """q [n_heads, hd]; K, V [n_kv, n_pos, hd] -> [n_heads, hd]."""
    q = np.ascontiguousarray(q, np.float32)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    nh, hd = q.shape
    nkv, npos, _ = K.shape
    out = np.empty((nh, hd), np.float32)
    lib().orc_attention(_fp(q), nh, nkv, hd, _fp(K), _fp(V), npos * hd, npos,
                        _fp(out))
    return out


def silu(g: np.ndarray) -> np.ndarray:
    g = np.array(g, np.float32, copy=True, order="C")
    lib().orc_silu(_fp(g), g.size)
    return g


def gelu_tanh(g: np.ndarray) -> np.ndarray:
    g = np.array(g, np.float32, copy=True, order="C")
    lib().orc_gelu_tanh(_fp(g), g.size)
    return g


def scale(x: np.ndarray, s: float) -> np.ndarray:
    x = np.array(x, np.float32, copy=True, order="C")
    lib().orc_scale(_fp(x), x.size, C.c_float(s))
    return x


def mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.array(g, np.float32, copy=True, order="C")
    u = np.ascontiguousarray(u, np.float32)
    lib().orc_mul(_fp(g), _fp(u), g.size)
    return g


# --- the model ---------------------------------------------------------------

class Model:
    """The oracle's decoder: weights borrowed from a dict of numpy arrays
    keyed by GGUF name (see synth.tensor_specs)."""

    def __init__(self, cfg: dict, weights: dict, max_ctx: int | None = None):
        self.cfg = dict(cfg)
        if max_ctx is not None:
            self.cfg["max_ctx"] = max_ctx
        c = self.cfg
        self._keep = []

        def T(name):
            a = np.ascontiguousarray(weights[name])
            self._keep.append(a)
            return tensor(a)

        self.ccfg = Config(ARCHS[c["arch"]],
                           c["n_layers"], c["d_model"], c["n_heads"],
                           c["n_kv_heads"], c["head_dim"], c["ffn_dim"],
                           c["vocab"], c["max_ctx"],
                           ROPE_PAIRINGS[c.get("rope_pairing", "halves")],
                           float(c["rope_theta"]), float(c["rms_eps"]),
                           int(c.get("sliding_window", 0)), int(c.get("window_pattern", 0)),
                           float(c.get("rope_theta_local", 0.0)))
        nl = c["n_layers"]
        layers = (Tensor * max(1, nl * len(SLOTS)))()
        for i in range(nl):
            for s, slot in enumerate(SLOTS):
                name = f"blk.{i}.{slot}"
                if name in weights:
                    layers[i * len(SLOTS) + s] = T(name)
        self._layers = layers
        te = T("token_embd.weight")
        on = T("output_norm.weight")
        out = T("output.weight") if "output.weight" in weights else Tensor(0, 0, None)
        self._h = lib().orc_create(C.byref(self.ccfg), C.byref(te), C.byref(on),
                                   C.byref(out), layers)
        if not self._h:
            raise ValueError("oracle: invalid config")

    def forward(self, tokens, logits: bool = True):
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        out = np.empty(self.cfg["vocab"], np.float32) if logits else None
        rc = lib().orc_forward(self._h, toks.ctypes.data_as(C.POINTER(C.c_int32)),
                               toks.size, _fp(out) if logits else None)
        if rc != 0:
            raise RuntimeError(f"oracle forward failed: code {rc}")
        return out

    def reset(self):
        lib().orc_reset(self._h)

    @property
    def kv_len(self) -> int:
        return lib().orc_kv_len(self._h)

    def set_kv_len(self, n: int):
        if lib().orc_set_kv_len(self._h, n) != 0:
            raise ValueError("bad kv length")

    def kv_read(self, layer: int, which: int, pos0: int, n: int) -> np.ndarray:
        c = self.cfg
        out = np.empty((c["n_kv_heads"], n, c["head_dim"]), np.float32)
        if lib().orc_kv_read(self._h, layer, which, pos0, n, _fp(out)) != 0:
            raise ValueError("bad kv range")
        return out

    def kv_write(self, layer: int, which: int, pos0: int, rows: np.ndarray):
        rows = np.ascontiguousarray(rows, np.float32)
        if lib().orc_kv_write(self._h, layer, which, pos0, rows.shape[1], _fp(rows)) != 0:
            raise ValueError("bad kv range")

    def trace(self) -> str:
        return lib().orc_trace(self._h).decode()

    def close(self):
        if self._h:
            lib().orc_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
