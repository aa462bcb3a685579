"""Several conversations on one loaded model (df_session) on the GPU.

Page "Execution contract", "Concurrency": each conversation has its own KV
cache, several share one loaded model, and concurrent forwards on one model
are allowed when each has its own cache. Checks:

* interleaved decode of three prompts on the model and two sessions: each
  matches the oracle run of its own prompt (rel-L2 <= 1e-4) and, bit for
  bit, a model that ran that prompt alone;
* bulk prefill in sessions, the same bit-for-bit check;
* forwards and generate on two sessions from two host threads at once equal
  the sequential results bit for bit;
* a session keeps working after the model it came from is freed;
* a session holds a KV cache, not a second copy of the weights;
* argument errors (max_ctx beyond the model's, option flags).
"""
import threading

import numpy as np
import pytest

import oracle
import synth
from parity import check_steps, oracle_greedy

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


def run_alone(dfa, cfg, W, fed):
    m = dfa.Model(cfg, W)
    out = [m.forward([t]).cpu().numpy().copy() for t in fed]
    m.close()
    return out


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def test_interleaved_conversations_match_their_own_runs(dfa):
    cfg = synth.config("tiny", arch="qwen3", wdtype="f32")
    W = synth.make_weights(cfg)
    say("[tiny qwen3 f32] three prompts interleaved token by token on a model and two sessions")
    prompts = [synth.make_prompt(cfg, 20, stream=s) for s in (0, 1, 2)]
    runs = [oracle_greedy(cfg, W, p, 6) for p in prompts]
    m = dfa.Model(cfg, W)
    handles = [m, m.session(), m.session(40)]
    got = [[] for _ in handles]
    n = len(runs[0][0])
    for i in range(n):
        for k, h in enumerate(handles):
            got[k].append(h.forward([runs[k][0][i]]).cpu().numpy().copy())
    for k, h in enumerate(handles):
        worst, _ = check_steps(got[k], runs[k][1], 1e-4, f"conversation {k}")
        say(f"  conversation {k}: worst rel-L2 {worst:.2e}")
        assert h.kv_len == n
        alone = run_alone(dfa, cfg, W, runs[k][0])
        for a, b in zip(got[k], alone):
            assert np.array_equal(bits(a), bits(b)), f"conversation {k} differs from its lone run"
    # each conversation's cache holds its own rows
    om = oracle.Model(cfg, W)
    om.forward(runs[2][0], logits=False)
    a = handles[2].read_kv(1, 0, 0, n)
    b = om.kv_read(1, 0, 0, n)
    assert np.max(np.abs(a - b)) <= 1e-4 * max(1.0, np.max(np.abs(b)))
    om.close()
    handles[1].reset()
    assert handles[1].kv_len == 0 and handles[0].kv_len == n
    for h in handles[::-1]:
        h.close()


def test_bulk_prefill_in_sessions(dfa):
    cfg = synth.config("tiny", arch="llama", wdtype="f16", max_ctx=64)
    W = synth.make_weights(cfg)
    say("[tiny llama f16] bulk prefill of two prompts in two sessions, then decode")
    m = dfa.Model(cfg, W)
    s1, s2 = m.session(), m.session()
    p1, p2 = synth.make_prompt(cfg, 37, stream=4), synth.make_prompt(cfg, 45, stream=5)
    g1 = s1.forward(p1).cpu().numpy().copy()
    g2 = s2.forward(p2).cpu().numpy().copy()
    d1 = s1.forward([7]).cpu().numpy().copy()
    for p, g, d in ((p1, g1, d1), (p2, g2, None)):
        lone = dfa.Model(cfg, W)
        assert np.array_equal(bits(lone.forward(p).cpu().numpy()), bits(g))
        if d is not None:
            assert np.array_equal(bits(lone.forward([7]).cpu().numpy()), bits(d))
        lone.close()
    assert m.kv_len == 0 and s1.kv_len == 38 and s2.kv_len == 45
    for h in (s2, s1, m):
        h.close()


def test_two_threads_on_two_sessions(dfa):
    cfg = synth.config("tiny", arch="qwen2", wdtype="f16", max_ctx=96)
    W = synth.make_weights(cfg)
    say("[tiny qwen2 f16] two host threads, one session each: prefill + forward + generate")
    m = dfa.Model(cfg, W)
    prompts = [synth.make_prompt(cfg, 30, stream=s) for s in (6, 7)]

    def work(h, p, out):
        h.forward(p, logits=False)
        for t in (3, 9, 27):
            out.append(h.forward([t]).cpu().numpy().copy())
        out.append(h.generate(11, 24).cpu().numpy().copy())

    seq = []
    for p in prompts:
        h = m.session()
        o = []
        work(h, p, o)
        seq.append(o)
        h.close()
    sessions = [m.session(), m.session()]
    par = [[], []]
    errors = []

    def runner(k):
        try:
            for _ in range(3):
                sessions[k].reset()
                par[k].clear()
                work(sessions[k], prompts[k], par[k])
        except Exception as e:  # reported below
            errors.append(e)

    th = [threading.Thread(target=runner, args=(k,)) for k in (0, 1)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in th), "a session thread did not finish"
    assert not errors, errors
    for k in (0, 1):
        for a, b in zip(par[k], seq[k]):
            assert np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))
    for h in sessions + [m]:
        h.close()


def test_session_outlives_its_model(dfa):
    cfg = synth.config("tiny", arch="qwen3", wdtype="f16")
    W = synth.make_weights(cfg)
    say("[tiny qwen3 f16] free the model first, keep decoding in its session")
    m = dfa.Model(cfg, W)
    s = m.session(32)
    toks = synth.make_prompt(cfg, 12, stream=8)
    m.forward(toks[:4], logits=False)
    m.close()
    fed, ref = oracle_greedy(cfg, W, toks, 4)
    got = [s.forward([t]).cpu().numpy().copy() for t in fed]
    check_steps(got, ref, 1e-4, "session after model free")
    s.close()


def test_session_holds_a_cache_not_weights(dfa):
    import torch
    cfg = synth.config("qwen3_0p6b", n_layers=2, max_ctx=256)
    say("[qwen3-0.6B shape, 2 layers] device memory of a session")
    Wd = synth.make_weights_device(cfg)
    m = dfa.Model(cfg, Wd)
    del Wd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    t = m.timings()
    free0 = torch.cuda.mem_get_info()[0]
    s = m.session(128)
    free1 = torch.cuda.mem_get_info()[0]
    ts = s.timings()
    assert ts["weight_bytes"] == t["weight_bytes"] > 300e6
    assert ts["kv_bytes"] * 2 == t["kv_bytes"]
    used = free0 - free1
    say(f"  weights {t['weight_bytes'] / 1e6:.0f} MB, session took {used / 1e6:.1f} MB")
    assert used < 64e6, used
    toks = synth.make_prompt(cfg, 3)
    a = m.forward(toks).cpu().numpy().copy()
    b = s.forward(toks).cpu().numpy().copy()
    assert np.array_equal(bits(a), bits(b))
    s.close()
    m.close()


def test_session_argument_errors(dfa):
    cfg = synth.config("tiny", wdtype="f16", max_ctx=48)
    m = dfa.Model(cfg, synth.make_weights(cfg))
    with pytest.raises(dfa.DecFwdError) as e:
        dfa.df_session(m.h, 49)
    assert e.value.status == "INVALID_ARGUMENT" and "max_ctx" in str(e.value)
    with pytest.raises(dfa.DecFwdError):
        dfa.df_session(m.h, 0)
    import ctypes as C
    opt = dfa.df_options(None, 0, 1)  # no option flags are defined
    out = C.c_void_p()
    rc = dfa.lib().df_session(m.h, 16, C.byref(opt), C.byref(out))
    assert dfa.STATUS_NAMES[rc] == "INVALID_ARGUMENT" and not out.value
    assert "flags" in dfa.df_last_error(None)
    m.close()


def test_load_rejects_option_flags(dfa):
    import ctypes as C
    cfg = synth.config("tiny", wdtype="f16", max_ctx=16)
    W = synth.make_weights(cfg)
    for bit in (1, 2, 1 << 30):
        with pytest.raises(dfa.DecFwdError) as e:
            dfa.df_load(cfg, W, flags=bit)
        assert e.value.status == "INVALID_ARGUMENT" and "flags" in str(e.value)
