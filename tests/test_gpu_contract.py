"""Runtime contract of page "Execution contract" on the GPU:

* "Concurrency": one forward at a time per KV cache. A second df_forward on
  a handle while another thread's df_forward runs on it returns DF_ERR_BUSY
  and changes nothing; the calls that were let through account for kv_len
  exactly.
* "Error semantics": a KV cache that cannot be allocated gives
  DF_ERR_OUT_OF_MEMORY with the handle left NULL and every device byte the
  failed load took given back.
* "Shutdown": no leaks; free device memory is the same after every one of
  20 load / forward / free cycles.
* positions run up to max_ctx - 1: the cache filled by one bulk call, and
  by a bulk call plus decode steps, matches the oracle; one more token is
  DF_ERR_CONTEXT_FULL with the cache unchanged; an empty call is
  DF_ERR_INVALID_ARGUMENT.
* the greedy token (page "Local inference and architectures", "Choosing the
  engine": temperature 0): df_argmax on crafted vectors takes the lowest
  index among equal maxima wherever they sit in the per-block partition,
  and a NaN never wins.
"""
import ctypes as C
import threading

import numpy as np
import pytest

import synth

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


def free_bytes():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return torch.cuda.mem_get_info()[0]


def test_second_forward_on_one_handle_is_busy(dfa):
    cfg = synth.config("tiny", wdtype="f32", max_ctx=4096)
    W = synth.make_weights(cfg)
    say("[tiny qwen3 f32] df_forward of 3000 tokens on one thread, 1-token forwards on another")
    h = dfa.df_load(cfg, W)
    toks = synth.make_prompt(cfg, 3000)
    started = threading.Event()
    res = {"a": []}

    def long_call():
        started.set()
        for _ in range(1000):  # again while the other thread holds the handle
            try:
                dfa.df_forward(h, toks)
                res["a"].append("OK")
                return
            except dfa.DecFwdError as e:
                res["a"].append(e.status)

    th = threading.Thread(target=long_call)
    th.start()
    started.wait()
    ok = busy = 0
    other = []
    while th.is_alive():
        try:
            dfa.df_forward(h, [int(toks[0])])
            ok += 1
        except dfa.DecFwdError as e:
            if e.status == "BUSY":
                busy += 1
            else:
                other.append(e.status)
    th.join()
    n_long = res["a"].count("OK")
    say(f"  long call: {res['a']}; short calls: {ok} OK, {busy} BUSY, others {other}")
    assert not other
    assert set(res["a"]) <= {"OK", "BUSY"} and n_long == 1 and res["a"][-1] == "OK"
    assert busy > 0
    assert dfa.df_kv_length(h) == 3000 * n_long + ok
    # the handle is usable afterwards
    dfa.df_reset_kv_cache(h)
    dfa.df_forward(h, toks[:4])
    assert dfa.df_kv_length(h) == 4
    dfa.df_free(h)


def test_out_of_memory_leaves_nothing_behind(dfa):
    # K and V of 64 layers x 8 KV heads x 2^20 positions x 256 dims: 512 GiB
    # each, more than the device holds
    cfg = synth.config("tiny", n_layers=64, n_heads=8, n_kv_heads=8, head_dim=256,
                       ffn_dim=64, wdtype="f16", max_ctx=1 << 20)
    W = synth.make_weights(cfg)
    say("[tiny f16, 64 layers, 8 KV heads of 256, max_ctx 2^20] load needs 1 TiB of KV cache")
    before = free_bytes()
    L = dfa.lib()
    keep = []
    names = list(W)
    arr = (dfa.df_tensor * len(names))()
    for i, n in enumerate(names):
        arr[i] = dfa._tensor_entry(n, W[n], keep)
    c = dfa.make_config(cfg, None)
    opt = dfa.df_options(None, 0, 0)
    out = C.c_void_p(0x1234)  # must come back NULL
    rc = L.df_load(C.byref(c), arr, len(names), C.byref(opt), C.byref(out))
    msg = dfa.df_last_error(None)
    say(f"  df_load -> {dfa.STATUS_NAMES.get(rc)}: {msg}")
    assert rc == 5, (rc, msg)  # DF_ERR_OUT_OF_MEMORY
    assert out.value is None
    assert "KV" in msg or "kv" in msg or "bytes" in msg
    after = free_bytes()
    say(f"  free device memory before {before / 2**20:.1f} MiB, after {after / 2**20:.1f} MiB")
    assert abs(after - before) <= 4 << 20
    # the library still loads a model afterwards
    small = synth.config("tiny", wdtype="f16")
    h = dfa.df_load(small, synth.make_weights(small))
    dfa.df_forward(h, [1, 2, 3])
    dfa.df_free(h)


def test_load_free_cycles_do_not_leak(dfa):
    cfg = synth.config("qwen3_0p6b", n_layers=2, max_ctx=256)
    W = synth.make_weights(cfg)
    toks = synth.make_prompt(cfg, 40)
    say("[qwen3-0.6B shape, 2 layers] 20 cycles of load, bulk 40 + decode 2, free")
    free = []
    held = 0
    for i in range(20):
        h = dfa.df_load(cfg, W)
        dfa.df_forward(h, toks)
        dfa.df_forward(h, toks[:1])
        dfa.df_forward(h, toks[1:2])
        if i == 0:
            t = dfa.df_get_timings(h)
            held = t["weight_bytes"] + t["kv_bytes"] + t["pool_bytes"]
        dfa.df_free(h)
        assert h.value is None
        free.append(free_bytes())
    spread = max(free[1:]) - min(free[1:])
    say(f"  a model holds {held / 2**20:.0f} MiB; free memory over cycles 2..20 "
        f"varies by {spread / 2**20:.2f} MiB")
    assert held > 300 << 20
    assert spread <= 4 << 20
    dfa.df_free(h)  # freeing a released handle is a no-op


def test_argmax_ties_and_nans(dfa):
    """Crafted vectors over a vocabulary of 300000 (256 argmax blocks of
    1172 values): equal maxima in different blocks, in one block, at both
    ends; NaN and -inf around them."""
    import torch
    V = 300000
    cfg = synth.config("tiny", vocab=V, max_ctx=8)
    say(f"[tiny, vocab {V}] df_argmax on crafted vectors")
    h = dfa.df_load(cfg, synth.make_weights(cfg))
    nan, inf = float("nan"), float("inf")

    def case(fill, sets, want, what):
        v = np.full(V, fill, np.float32)
        for i, x in sets:
            v[i] = x
        got = dfa.df_argmax(h, torch.from_numpy(v).to("cuda"))
        say(f"  {what}: {got}")
        assert got == want, (what, got, want)

    case(0.0, [(1000, 1.0), (250000, 1.0)], 1000, "equal maxima in blocks 0 and 213")
    case(0.0, [(250000, 1.0), (1000, 1.0), (1001, 1.0)], 1000, "three equal maxima")
    case(0.0, [(299999, 2.0), (298000, 2.0)], 298000, "equal maxima in the last block")
    case(0.0, [(0, 5.0), (299999, 5.0)], 0, "equal maxima at both ends")
    case(0.0, [(299999, 5.0)], 299999, "maximum at the last index")
    case(2.0, [(5, nan), (7, nan), (100000, 3.0)], 100000, "NaNs beside the maximum")
    case(nan, [(123456, -1e30)], 123456, "one finite value among NaNs")
    case(-inf, [(3, nan), (77, 0.0)], 77, "-inf and a NaN around one zero")
    case(-inf, [], 0, "all -inf: the lowest index")
    case(nan, [], 0, "all NaN: index 0")
    case(0.0, [(40000, inf), (20000, inf), (30000, nan)], 20000, "two +inf and a NaN")
    rng = np.random.default_rng(11)
    for k in range(4):
        v = rng.standard_normal(V).astype(np.float32)
        got = dfa.df_argmax(h, torch.from_numpy(v).to("cuda"))
        assert got == int(np.argmax(v)), k
    dfa.df_free(h)


@pytest.mark.parametrize("arch,hd", [("qwen3", 128), ("llama", 64)])
def test_filling_the_cache_to_max_ctx(dfa, arch, hd):
    """Positions up to max_ctx - 1 (reading 6: overflow is an error, nothing
    wraps): a bulk prefill that fills the whole cache in one call, and a
    bulk prefill plus decode steps that reach the last slot, against the
    oracle; one more token is CONTEXT_FULL and leaves the cache as it was;
    an empty call is INVALID_ARGUMENT."""
    import oracle
    from parity import first_argmax, rel_l2
    P = 130  # two 64-key tiles and a ragged third
    cfg = synth.config("tiny", arch=arch, wdtype="f16", head_dim=hd, n_heads=4, n_kv_heads=2, max_ctx=P)
    W = synth.make_weights(cfg)
    toks = synth.make_prompt(cfg, P, stream=5)
    say(f"[tiny {arch} f16, head_dim {hd}, max_ctx {P}] bulk of {P}; bulk of {P - 3} + 3 decode steps")
    om = oracle.Model(cfg, W, max_ctx=P)
    refs = [om.forward([t]) for t in toks]
    m = dfa.Model(cfg, W)
    got = m.forward(toks).cpu().numpy().copy()
    assert m.kv_len == P
    e = rel_l2(got, refs[-1])
    say(f"  bulk of {P}: rel-L2 {e:.2e}")
    assert e <= 5e-3 and first_argmax(got) == first_argmax(refs[-1])
    before = m.read_kv(0, 0, 0, P)
    with pytest.raises(dfa.DecFwdError) as ei:
        m.forward([int(toks[0])])
    assert ei.value.status == "CONTEXT_FULL"
    assert m.kv_len == P and np.array_equal(m.read_kv(0, 0, 0, P), before)
    m.reset()
    got = m.forward(toks[:P - 3]).cpu().numpy().copy()
    assert rel_l2(got, refs[P - 4]) <= 5e-3
    for i in range(P - 3, P):
        got = m.forward([int(toks[i])]).cpu().numpy().copy()
        e = rel_l2(got, refs[i])
        say(f"  decode at position {i}: rel-L2 {e:.2e}")
        assert e <= 5e-3 and first_argmax(got) == first_argmax(refs[i])
    assert m.kv_len == P
    with pytest.raises(dfa.DecFwdError) as ei:
        m.forward(toks[:2])
    assert ei.value.status == "CONTEXT_FULL"
    with pytest.raises(dfa.DecFwdError) as ei:
        m.forward(np.zeros(0, np.int32))
    assert ei.value.status == "INVALID_ARGUMENT"
    assert m.kv_len == P
    m.close()
    om.close()
