"""Python binding of libdecfwd.so (include/decfwd.h).

Argument marshalling only: every step of the forward pass runs in the HIP
library. Function names are the C names. Weights are given as a dict keyed
by GGUF tensor name whose values are numpy arrays (host) or torch tensors
(host or device): float32 -> DF_F32, float16 -> DF_F16, uint8 [rows,
cols/32*34] -> DF_Q8_32 blocks. Device outputs are torch tensors; torch is
used for device memory and streams only.

The library must be built (decoder_forward_amd/build.py); importing this
module without it raises, there is no other path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdecfwd.so")

DF_OK = 0
STATUS_NAMES = {
    0: "OK", 1: "UNSUPPORTED_OP", 2: "SHAPE_MISMATCH", 3: "MISSING_TENSOR",
    4: "WEIGHT_FORMAT_MISMATCH", 5: "OUT_OF_MEMORY", 6: "BACKEND_INIT",
    7: "INVALID_CONFIG", 8: "CONTEXT_FULL", 9: "BUSY", 10: "INVALID_ARGUMENT",
    11: "DEVICE",
}
DF_ARCH_LLAMA, DF_ARCH_QWEN3, DF_ARCH_QWEN2, DF_ARCH_GEMMA3 = 0, 1, 2, 3
ARCHS = {"llama": DF_ARCH_LLAMA, "qwen3": DF_ARCH_QWEN3, "qwen2": DF_ARCH_QWEN2,
         "gemma3": DF_ARCH_GEMMA3}
DF_ROPE_HALVES, DF_ROPE_ADJACENT = 0, 1
ROPE_PAIRINGS = {"halves": DF_ROPE_HALVES, "adjacent": DF_ROPE_ADJACENT}
DF_F32, DF_F16, DF_Q8_32 = 0, 1, 2

# Every entry point of include/decfwd.h.
EXPORTS = ("df_load", "df_forward", "df_generate", "df_reset_kv_cache",
           "df_free", "df_last_error", "df_get_timings", "df_kv_length",
           "df_argmax", "df_read_kv", "df_write_kv", "df_stream",
           "df_profile", "df_profile_read", "df_time_kernel", "df_session",
           "df_time_prefill", "df_prefill_plan", "df_forward_noalloc")
KERNELS = {"embed": 0, "qkv": 1, "attn": 2, "o": 3, "gate_up": 4, "down": 5,
           "logits": 6, "argmax": 7, "attn_merge": 8}
PREFILL_KERNELS = {"qkv": 10, "attn": 11, "o": 12, "gate_up": 13, "down": 14, "rows": 15}
# df_prefill_plan tile codes and flags.
GEMM_TILES = {1: "128x128", 2: "128x256", 3: "256x256", 4: "256x256_lds", 5: "256x192_lds"}
DF_GEMM_TILE_MASK, DF_GEMM_Q8_IN_GEMM, DF_GEMM_Q8_DEQUANT_FIRST = 15, 16, 32
DF_GEMM_SPLIT_SHIFT, DF_GEMM_SPLIT_MASK = 8, 0xF00


class DecFwdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        self.code = code
        self.status = STATUS_NAMES.get(code, str(code))
        super().__init__(f"{self.status}: {msg}")


class df_config(C.Structure):
    _fields_ = [("arch", C.c_int32), ("n_layers", C.c_int32),
                ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("ffn_dim", C.c_int32), ("vocab", C.c_int32),
                ("max_ctx", C.c_int32), ("rope_pairing", C.c_int32),
                ("rope_theta", C.c_double), ("rms_eps", C.c_double),
                ("sliding_window", C.c_int32), ("window_pattern", C.c_int32),
                ("rope_theta_local", C.c_double)]


class df_tensor(C.Structure):
    _fields_ = [("name", C.c_char_p), ("dtype", C.c_int32),
                ("on_device", C.c_int32), ("rows", C.c_int64),
                ("cols", C.c_int64), ("data", C.c_void_p),
                ("nbytes", C.c_uint64)]


class df_options(C.Structure):
    _fields_ = [("stream", C.c_void_p), ("device", C.c_int32),
                ("flags", C.c_int32)]


class df_timings(C.Structure):
    _fields_ = [("load_ms", C.c_double), ("last_prefill_ms", C.c_double),
                ("last_step_ms", C.c_double), ("n_forward", C.c_int64),
                ("weight_bytes", C.c_int64), ("kv_bytes", C.c_int64),
                ("pool_bytes", C.c_int64)]


_lib = None


def lib() -> C.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "decoder_forward_amd/build.py (hipcc, gfx950)")
    L = C.CDLL(LIB_PATH)
    vp, i32, P = C.c_void_p, C.c_int32, C.POINTER
    L.df_load.argtypes = [P(df_config), P(df_tensor), C.c_size_t, P(df_options), P(vp)]
    L.df_session.argtypes = [vp, i32, P(df_options), P(vp)]
    L.df_forward.argtypes = [vp, P(i32), i32, vp]
    L.df_forward_noalloc.argtypes = [vp, P(i32), i32, vp]
    L.df_generate.argtypes = [vp, i32, i32, vp, vp]
    L.df_reset_kv_cache.argtypes = [vp]
    L.df_free.argtypes = [P(vp)]
    L.df_free.restype = None
    L.df_last_error.argtypes = [vp]
    L.df_last_error.restype = C.c_char_p
    L.df_get_timings.argtypes = [vp, P(df_timings)]
    L.df_kv_length.argtypes = [vp, P(i32)]
    L.df_argmax.argtypes = [vp, vp, P(i32)]
    L.df_read_kv.argtypes = [vp, i32, i32, i32, i32, P(C.c_float)]
    L.df_write_kv.argtypes = [vp, i32, i32, i32, i32, P(C.c_float), i32]
    L.df_stream.argtypes = [vp]
    L.df_stream.restype = vp
    L.df_profile.argtypes = [vp, i32, i32]
    L.df_profile_read.argtypes = [vp, i32, P(C.c_int64), P(C.c_double)]
    L.df_time_kernel.argtypes = [vp, i32, i32, P(C.c_double)]
    L.df_time_prefill.argtypes = [vp, i32, i32, i32, P(C.c_double)]
    L.df_prefill_plan.argtypes = [vp, i32, P(i32)]
    for name in EXPORTS:
        if name not in ("df_free", "df_last_error", "df_stream"):
            getattr(L, name).restype = i32
    _lib = L
    return L


def _check(rc: int, handle=None):
    if rc != DF_OK:
        msg = lib().df_last_error(handle)
        raise DecFwdError(rc, msg.decode() if msg else "")


def make_config(cfg: dict, max_ctx: int | None = None) -> df_config:
    return df_config(ARCHS[cfg["arch"]],
                     cfg["n_layers"], cfg["d_model"], cfg["n_heads"],
                     cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn_dim"],
                     cfg["vocab"], max_ctx if max_ctx is not None else cfg["max_ctx"],
                     ROPE_PAIRINGS[cfg.get("rope_pairing", "halves")],
                     float(cfg["rope_theta"]), float(cfg["rms_eps"]),
                     int(cfg.get("sliding_window", 0)), int(cfg.get("window_pattern", 0)),
                     float(cfg.get("rope_theta_local", 0.0)))


def _tensor_entry(name: str, a, keep: list) -> df_tensor:
    """df_tensor for a numpy array or a torch tensor."""
    try:
        import torch
        is_torch = isinstance(a, torch.Tensor)
    except ImportError:  # pragma: no cover
        is_torch = False
    if is_torch:
        a = a.contiguous()
        keep.append(a)
        dt = {"torch.float32": DF_F32, "torch.float16": DF_F16,
              "torch.uint8": DF_Q8_32}[str(a.dtype)]
        rows, last = a.shape[0], a.shape[-1]
        ptr, nbytes, on_dev = a.data_ptr(), a.numel() * a.element_size(), int(a.is_cuda)
    else:
        a = np.ascontiguousarray(a)
        keep.append(a)
        dt = {np.dtype(np.float32): DF_F32, np.dtype(np.float16): DF_F16,
              np.dtype(np.uint8): DF_Q8_32}[a.dtype]
        rows, last = (a.shape[0], a.shape[-1]) if a.ndim == 2 else (1, a.shape[0])
        ptr, nbytes, on_dev = a.ctypes.data, a.nbytes, 0
    if a.ndim == 1:
        rows = 1
    cols = last // 34 * 32 if dt == DF_Q8_32 else last
    return df_tensor(name.encode(), dt, on_dev, rows, cols, ptr, nbytes)


def df_load(cfg: dict, weights: dict, stream=None, device: int = 0,
            max_ctx: int | None = None, flags: int = 0):
    """Load a model; returns an opaque handle (c_void_p)."""
    keep: list = []
    names = list(weights)
    arr = (df_tensor * max(1, len(names)))()
    for i, n in enumerate(names):
        arr[i] = _tensor_entry(n, weights[n], keep)
    c = make_config(cfg, max_ctx)
    opt = df_options(stream, device, flags)
    h = C.c_void_p()
    rc = lib().df_load(C.byref(c), arr, len(names), C.byref(opt), C.byref(h))
    _check(rc, None)
    return h


def df_session(h, max_ctx: int, stream=None):
    """Another conversation on the loaded model h: its own KV cache of
    max_ctx positions, the model's weights. Returns a handle."""
    opt = df_options(stream, 0, 0)
    out = C.c_void_p()
    rc = lib().df_session(h, max_ctx, C.byref(opt), C.byref(out))
    _check(rc, None)
    return out


def df_forward(h, tokens, logits=None) -> None:
    """tokens: host ints; logits: torch f32 device tensor [vocab] or None."""
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    ptr = logits.data_ptr() if logits is not None else None
    _check(lib().df_forward(h, toks.ctypes.data_as(C.POINTER(C.c_int32)),
                            toks.size, ptr), h)


def df_forward_noalloc(h, tokens, logits=None) -> None:
    """df_forward through the decode kernels with the step's activations in
    the library's fixed device array: the call allocates nothing."""
    toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    ptr = logits.data_ptr() if logits is not None else None
    _check(lib().df_forward_noalloc(h, toks.ctypes.data_as(C.POINTER(C.c_int32)),
                                    toks.size, ptr), h)


def df_generate(h, first_token: int, n_steps: int, tokens_out, logits=None) -> None:
    """tokens_out: torch int32 device tensor of at least n_steps entries."""
    _check(lib().df_generate(h, int(first_token), int(n_steps),
                             tokens_out.data_ptr(),
                             logits.data_ptr() if logits is not None else None), h)


def df_reset_kv_cache(h) -> None:
    _check(lib().df_reset_kv_cache(h), h)


def df_free(h) -> None:
    lib().df_free(C.byref(h))


def df_last_error(h=None) -> str:
    r = lib().df_last_error(h)
    return r.decode() if r else ""


def df_get_timings(h) -> dict:
    t = df_timings()
    _check(lib().df_get_timings(h, C.byref(t)), h)
    return {f: getattr(t, f) for f, _ in df_timings._fields_}


def df_kv_length(h) -> int:
    n = C.c_int32()
    _check(lib().df_kv_length(h, C.byref(n)), h)
    return n.value


def df_argmax(h, logits) -> int:
    t = C.c_int32()
    _check(lib().df_argmax(h, logits.data_ptr(), C.byref(t)), h)
    return t.value


def df_read_kv(h, cfg: dict, layer: int, which: int, pos0: int, n: int) -> np.ndarray:
    out = np.empty((cfg["n_kv_heads"], n, cfg["head_dim"]), np.float32)
    _check(lib().df_read_kv(h, layer, which, pos0, n,
                            out.ctypes.data_as(C.POINTER(C.c_float))), h)
    return out


def df_write_kv(h, layer: int, which: int, pos0: int, rows: np.ndarray,
                kv_len_after: int) -> None:
    rows = np.ascontiguousarray(rows, np.float32)
    _check(lib().df_write_kv(h, layer, which, pos0, rows.shape[1],
                             rows.ctypes.data_as(C.POINTER(C.c_float)),
                             kv_len_after), h)


def df_stream(h) -> int:
    return lib().df_stream(h) or 0


def df_profile(h, kernel: str, enable: bool = True) -> None:
    _check(lib().df_profile(h, KERNELS[kernel], 1 if enable else 0), h)


def df_time_kernel(h, kernel: str, reps: int = 8) -> float:
    """Mean microseconds of one launch of a kernel class, back-to-back replay."""
    us = C.c_double()
    _check(lib().df_time_kernel(h, KERNELS[kernel], reps, C.byref(us)), h)
    return us.value


def df_time_prefill(h, kernel: str, rows: int, reps: int = 2) -> float:
    """Mean microseconds of one layer's launches of a bulk-prefill class for
    `rows` rows at positions kv_len.. (writes only cache rows past kv_len)."""
    us = C.c_double()
    _check(lib().df_time_prefill(h, PREFILL_KERNELS[kernel], rows, reps, C.byref(us)), h)
    return us.value


def df_prefill_plan(h, rows: int) -> dict:
    """The GEMM kernels a bulk prefill of `rows` rows runs: for each of
    qkv / o / gate_up / down, (tile name, 8-bit in-GEMM dequantisation,
    8-bit dequantised first, work-groups per tile along K)."""
    plan = (C.c_int32 * 4)()
    _check(lib().df_prefill_plan(h, rows, plan), h)
    out = {}
    for k, v in zip(("qkv", "o", "gate_up", "down"), plan):
        out[k] = (GEMM_TILES.get(v & DF_GEMM_TILE_MASK), bool(v & DF_GEMM_Q8_IN_GEMM),
                  bool(v & DF_GEMM_Q8_DEQUANT_FIRST), (v & DF_GEMM_SPLIT_MASK) >> DF_GEMM_SPLIT_SHIFT)
    return out


def df_profile_read(h, kernel: str):
    """(launches, total device ms) since the last read."""
    n, ms = C.c_int64(), C.c_double()
    _check(lib().df_profile_read(h, KERNELS[kernel], C.byref(n), C.byref(ms)), h)
    return n.value, ms.value


class Model:
    """Convenience owner of a handle: Model(cfg, weights).forward(tokens).

    The library orders its work on a torch stream of its own (default
    priority); every call makes that stream wait for torch's current stream
    first and makes torch's current stream wait for it afterwards, so torch
    code before and after sees the results in order."""

    def __init__(self, cfg: dict, weights: dict | None, max_ctx: int | None = None,
                 device: int = 0, _base=None):
        import torch
        self._torch = torch
        self.cfg = dict(cfg)
        if max_ctx is not None:
            self.cfg["max_ctx"] = max_ctx
        self.device = torch.device("cuda", device)
        self.stream = torch.cuda.Stream(self.device)
        self.h = None
        if _base is not None:
            self.h = df_session(_base.h, self.cfg["max_ctx"], stream=self.stream.cuda_stream)
        else:
            self.h = df_load(self.cfg, weights, stream=self.stream.cuda_stream,
                             device=device)
        self.logits = torch.empty(self.cfg["vocab"], dtype=torch.float32,
                                  device=self.device)

    def session(self, max_ctx: int | None = None) -> "Model":
        """A new conversation on these weights with its own KV cache and
        stream (df_session)."""
        return Model(self.cfg, None, max_ctx=max_ctx if max_ctx is not None else self.cfg["max_ctx"],
                     device=self.device.index, _base=self)

    def _enter(self):
        self.stream.wait_stream(self._torch.cuda.current_stream(self.device))

    def _leave(self):
        self._torch.cuda.current_stream(self.device).wait_stream(self.stream)

    def forward(self, tokens, logits: bool = True):
        self._enter()
        df_forward(self.h, tokens, self.logits if logits else None)
        self._leave()
        return self.logits if logits else None

    def argmax(self) -> int:
        self._enter()
        return df_argmax(self.h, self.logits)

    def generate(self, first_token: int, n_steps: int):
        out = self._torch.empty(n_steps, dtype=self._torch.int32, device=self.device)
        self._enter()
        df_generate(self.h, first_token, n_steps, out, self.logits)
        self._leave()
        return out

    def reset(self):
        df_reset_kv_cache(self.h)

    @property
    def kv_len(self) -> int:
        return df_kv_length(self.h)

    def read_kv(self, layer, which, pos0, n):
        return df_read_kv(self.h, self.cfg, layer, which, pos0, n)

    def write_kv(self, layer, which, pos0, rows, kv_len_after):
        df_write_kv(self.h, layer, which, pos0, rows, kv_len_after)

    def timings(self) -> dict:
        return df_get_timings(self.h)

    def close(self):
        if self.h:
            df_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
