"""The C-ABI library without a GPU: it loads, exports every symbol that
include/decfwd.h declares, and validates config and tensor table on the
host before any device call (page "Execution contract", "Load phase" step 3
and "Error semantics": each error names the field / tensor / bytes)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decfwd.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(df_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def dfa():
    import decoder_forward_amd as dfa
    dfa.lib()
    return dfa


def test_library_exports_every_declared_symbol(dfa):
    names = header_functions()
    assert len(names) >= 12
    lib = C.CDLL(dfa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dfa.EXPORTS)


def test_library_links_no_torch():
    import subprocess
    import decoder_forward_amd as dfa
    out = subprocess.run(["ldd", dfa.LIB_PATH], capture_output=True, text=True).stdout
    # library names only (the load addresses are hex and can contain "c10")
    names = [line.split()[0] for line in out.splitlines() if line.strip()]
    assert not any("torch" in n or n.startswith("libc10") for n in names), names
    assert any(n.startswith("libamdhip64") for n in names), names


def tiny_table(**kw):
    cfg = synth.config("tiny", **kw)
    return cfg, synth.make_weights(cfg)


def load_rc(dfa, cfg, W, max_ctx=None):
    try:
        h = dfa.df_load(cfg, W, max_ctx=max_ctx)
    except dfa.DecFwdError as e:
        return e.status, str(e)
    dfa.df_free(h)
    return "OK", ""


@pytest.mark.parametrize("field,value,needle", [
    ("arch", "gemma3", None), ("d_model", 48, "d_model"), ("head_dim", 24, "head_dim"),
    ("n_kv_heads", 3, "n_kv_heads"), ("ffn_dim", 100, "ffn_dim"), ("vocab", 0, "vocab"),
    ("max_ctx", 0, "max_ctx"), ("rope_theta", -1.0, "rope_theta"),
    ("rms_eps", float("nan"), "rms_eps"), ("n_layers", -1, "n_layers"),
])
def test_invalid_config_is_named(dfa, field, value, needle):
    cfg, W = tiny_table()
    if field == "arch":
        c = dfa.make_config(cfg)
        c.arch = 7
        h = C.c_void_p()
        arr = (dfa.df_tensor * 1)()
        rc = dfa.lib().df_load(C.byref(c), arr, 0, None, C.byref(h))
        assert rc == 7 and b"arch" in dfa.lib().df_last_error(None)
        return
    cfg[field] = value
    status, msg = load_rc(dfa, cfg, W)
    assert status == "INVALID_CONFIG", msg
    assert needle in msg


@pytest.mark.parametrize("nh,nkv", [(16, 1), (18, 2)])
def test_unsupported_group_size(dfa, nh, nkv):
    cfg, W = tiny_table(n_heads=nh, n_kv_heads=nkv, head_dim=16, d_model=256)
    status, msg = load_rc(dfa, cfg, synth.make_weights(cfg))
    assert status == "INVALID_CONFIG" and "query heads" in msg


@pytest.mark.parametrize("nh,nkv", [(6, 2), (14, 2), (10, 2)])
def test_any_group_size_up_to_8_passes_validation(dfa, nh, nkv):
    cfg, W = tiny_table(n_heads=nh, n_kv_heads=nkv, head_dim=16, d_model=256)
    status, msg = load_rc(dfa, cfg, synth.make_weights(cfg))
    assert status in ("OK", "BACKEND_INIT"), msg


def test_invalid_rope_pairing_is_named(dfa):
    cfg, W = tiny_table()
    c = dfa.make_config(cfg)
    c.rope_pairing = 2
    h = C.c_void_p()
    arr = (dfa.df_tensor * 1)()
    rc = dfa.lib().df_load(C.byref(c), arr, 0, None, C.byref(h))
    assert dfa.STATUS_NAMES[rc] == "INVALID_CONFIG"
    assert b"rope_pairing" in dfa.lib().df_last_error(None)


def test_qwen2_missing_bias_is_named(dfa):
    cfg, W = tiny_table(arch="qwen2")
    del W["blk.1.attn_v.bias"]
    status, msg = load_rc(dfa, cfg, W)
    assert status == "MISSING_TENSOR"
    assert "blk.1.attn_v.bias" in msg and "add_bias v" in msg


def test_qwen2_bias_shape_and_dtype_checked(dfa):
    cfg, W = tiny_table(arch="qwen2")
    W["blk.0.attn_k.bias"] = W["blk.0.attn_q.bias"]
    status, msg = load_rc(dfa, cfg, W)
    assert status == "SHAPE_MISMATCH" and "blk.0.attn_k.bias" in msg
    cfg, W = tiny_table(arch="qwen2")
    W["blk.0.attn_q.bias"] = np.zeros((1, 2 * 34), np.uint8)
    status, msg = load_rc(dfa, cfg, W)
    assert status == "UNSUPPORTED_OP" and "blk.0.attn_q.bias" in msg


def test_bias_on_llama_rejected(dfa):
    cfg, W = tiny_table(arch="llama")
    W.update({k: v for k, v in synth.make_weights(synth.config("tiny", arch="qwen2")).items()
              if k.endswith(".bias")})
    status, msg = load_rc(dfa, cfg, W)
    assert status == "INVALID_ARGUMENT" and ".bias" in msg and "llama" in msg


def test_valid_qwen2_table_passes_validation(dfa):
    cfg, W = tiny_table(arch="qwen2", rope_pairing="adjacent")
    status, msg = load_rc(dfa, cfg, W)
    assert status in ("OK", "BACKEND_INIT"), msg


def test_missing_tensor_is_named(dfa):
    cfg, W = tiny_table()
    del W["blk.1.ffn_up.weight"]
    status, msg = load_rc(dfa, cfg, W)
    assert status == "MISSING_TENSOR"
    assert "blk.1.ffn_up.weight" in msg and "layer 1" in msg


def test_wrong_shape_is_named(dfa):
    cfg, W = tiny_table()
    W["blk.0.attn_k.weight"] = W["blk.0.attn_q.weight"]
    status, msg = load_rc(dfa, cfg, W)
    assert status == "SHAPE_MISMATCH"
    assert "blk.0.attn_k.weight" in msg and "[32, 64]" in msg and "[64, 64]" in msg


def test_byte_count_mismatch_is_named(dfa):
    cfg, W = tiny_table()
    keep = []
    names = list(W)
    arr = (dfa.df_tensor * len(names))()
    for i, n in enumerate(names):
        arr[i] = dfa._tensor_entry(n, W[n], keep)
    arr[3].nbytes -= 4
    c = dfa.make_config(cfg)
    h = C.c_void_p()
    rc = dfa.lib().df_load(C.byref(c), arr, len(names), None, C.byref(h))
    assert dfa.STATUS_NAMES[rc] == "WEIGHT_FORMAT_MISMATCH"
    msg = dfa.df_last_error(None)
    assert names[3] in msg and "bytes" in msg
    assert not h.value


def test_q8_norm_weight_rejected(dfa):
    cfg, W = tiny_table(wdtype="q8")
    W["output_norm.weight"] = np.zeros((1, 2 * 34), np.uint8)
    status, msg = load_rc(dfa, cfg, W)
    assert status == "UNSUPPORTED_OP" and "output_norm.weight" in msg


def test_mixed_block_dtypes_rejected(dfa):
    cfg, W = tiny_table()
    W["blk.1.ffn_down.weight"] = W["blk.1.ffn_down.weight"].astype(np.float16)
    status, msg = load_rc(dfa, cfg, W)
    assert status == "WEIGHT_FORMAT_MISMATCH" and "blk.1.ffn_down.weight" in msg


def test_unknown_tensor_rejected(dfa):
    cfg, W = tiny_table(arch="llama")
    W.update(synth.make_weights(synth.config("tiny")))  # brings qwen3's q/k norms
    status, msg = load_rc(dfa, cfg, W)
    assert status == "INVALID_ARGUMENT" and "attn_q_norm" in msg


def test_valid_table_reaches_backend_init_or_loads(dfa):
    cfg, W = tiny_table()
    status, msg = load_rc(dfa, cfg, W)
    assert status in ("OK", "BACKEND_INIT"), msg


def test_null_handles(dfa):
    L = dfa.lib()
    assert L.df_forward(None, None, 1, None) == 10
    assert L.df_reset_kv_cache(None) == 10
    L.df_free(None)
    h = C.c_void_p()
    L.df_free(C.byref(h))
    n = C.c_int32()
    assert L.df_kv_length(None, C.byref(n)) == 10
    assert L.df_stream(None) is None


def test_session_argument_checks_before_any_device_call(dfa):
    out = C.c_void_p(1)
    rc = dfa.lib().df_session(None, 16, None, C.byref(out))
    assert dfa.STATUS_NAMES[rc] == "INVALID_ARGUMENT" and not out.value
    assert "model is NULL" in dfa.df_last_error(None)
    rc = dfa.lib().df_session(None, 16, None, None)
    assert dfa.STATUS_NAMES[rc] == "INVALID_ARGUMENT"
