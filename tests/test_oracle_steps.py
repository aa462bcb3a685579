"""Pins of the oracle's single steps against closed forms, exact special
cases, invariants and numpy float64 textbook versions (CPU only).

Each op is the one named in the step list of page "Local inference and
architectures", section "The format"; RoPE's position cache follows page
"Execution contract", section "Memory lifecycle" (Position caches).
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(12345)


def ulp_close(a, b, ulps=1):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    sp = np.spacing(np.maximum(np.abs(a), np.abs(b)).astype(np.float32))
    return np.all(np.abs(a.astype(np.float64) - b.astype(np.float64)) <= ulps * sp)


# ---- f16 -> f32 (exact conversion, written from IEEE-754) -----------------

def test_f16_all_bit_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(bits.view(np.float16))
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_subnormals_not_flushed():
    smallest = np.array([1], np.uint16).view(np.float16)
    assert oracle.f16_to_f32(smallest)[0] == np.float32(2.0 ** -24)


# ---- rms_norm ----------------------------------------------------------------

@pytest.mark.parametrize("c", [1e-3, 0.25, 3.0, 1000.0])
def test_rmsnorm_constant_vector_closed_form(c):
    n, eps = 64, 1e-6
    x = np.full(n, c, np.float32)
    w = np.ones(n, np.float32)
    got = oracle.rmsnorm(x, w, eps)
    cc = float(np.float32(c))
    ref = cc / np.sqrt(cc * cc + eps)
    assert ulp_close(got, np.full(n, ref, np.float32), ulps=2)


def test_rmsnorm_weight_multiplies():
    n, eps = 32, 1e-6
    x = np.full(n, 2.0, np.float32)
    w = np.linspace(0.5, 1.5, n).astype(np.float32)
    got = oracle.rmsnorm(x, w, eps)
    ref = w.astype(np.float64) * 2.0 / np.sqrt(4.0 + eps)
    assert ulp_close(got, ref.astype(np.float32), ulps=2)


def test_rmsnorm_power_of_two_scale_invariance_exact():
    x = RNG.standard_normal(1024).astype(np.float32)
    w = (1 + 0.02 * RNG.standard_normal(1024)).astype(np.float16)
    a = oracle.rmsnorm(x, w, 0.0)
    b = oracle.rmsnorm(x * np.float32(2.0 ** 7), w, 0.0)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_rmsnorm_vs_numpy_f64():
    x = RNG.standard_normal(4096).astype(np.float32) * 3
    w = (1 + 0.02 * RNG.standard_normal(4096)).astype(np.float16)
    got = oracle.rmsnorm(x, w, 1e-6)
    xd = x.astype(np.float64)
    ref = w.astype(np.float64) * xd / np.sqrt(np.mean(xd * xd) + 1e-6)
    assert np.max(np.abs(got - ref) / np.abs(ref)) < 3e-7


# ---- matmul ------------------------------------------------------------------

def pack_q8(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    N, K = q.shape
    out = np.empty((N, K // 32, 34), np.uint8)
    out[:, :, 0:2] = s.astype(np.float16).view(np.uint8).reshape(N, K // 32, 2)
    out[:, :, 2:] = q.astype(np.int8).view(np.uint8).reshape(N, K // 32, 32)
    return out.reshape(N, K // 32 * 34)


def q8_dequant_f32(q, s):
    N, K = q.shape
    sf = s.astype(np.float16).astype(np.float32)
    return (np.repeat(sf, 32, axis=1) * q.astype(np.float32)).astype(np.float32)


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_matvec_one_hot_gives_column_exactly(dtype):
    N, K = 48, 96
    W = (0.02 * RNG.standard_normal((N, K))).astype(dtype)
    for k in (0, 17, K - 1):
        h = np.zeros(K, np.float32)
        h[k] = 1.0
        y = oracle.matvec(W, h)
        assert np.array_equal(y, W[:, k].astype(np.float32)), k


def test_matvec_one_hot_q8_column_exactly():
    N, K = 16, 128
    q = RNG.integers(-127, 128, size=(N, K))
    s = (np.abs(RNG.standard_normal((N, K // 32))) * 0.02 / 127)
    W = pack_q8(q, s)
    Wd = q8_dequant_f32(q, s)
    for k in (0, 33, 127):
        h = np.zeros(K, np.float32)
        h[k] = 1.0
        assert np.array_equal(oracle.matvec(W, h, K=K), Wd[:, k])


def test_matvec_non_square_orientation():
    # y has N entries and row n of W meets h: a transposed reading would
    # not even have the right length.
    W = np.arange(6, dtype=np.float32).reshape(2, 3)
    y = oracle.matvec(W, np.array([1, 10, 100], np.float32))
    assert np.array_equal(y, np.array([210, 543], np.float32))


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_matvec_vs_numpy_f64(dtype):
    N, K = 300, 4096
    W = (0.02 * RNG.standard_normal((N, K))).astype(dtype)
    h = RNG.standard_normal(K).astype(np.float32)
    ref = W.astype(np.float64) @ h.astype(np.float64)
    got = oracle.matvec(W, h)
    assert ulp_close(got, ref.astype(np.float32), ulps=1)


def test_matvec_q8_equals_f32_on_dequantised_weights_bitwise():
    N, K = 64, 1024
    q = RNG.integers(-127, 128, size=(N, K))
    s = np.abs(RNG.standard_normal((N, K // 32))) * 0.02 / 127
    s[0, 0] = 3e-8  # an f16 subnormal scale
    h = RNG.standard_normal(K).astype(np.float32)
    a = oracle.matvec(pack_q8(q, s), h, K=K)
    b = oracle.matvec(q8_dequant_f32(q, s), h)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_embed_row_exact():
    E = (0.02 * RNG.standard_normal((10, 64))).astype(np.float16)
    assert np.array_equal(oracle.embed(E, 7), E[7].astype(np.float32))


# ---- rope --------------------------------------------------------------------

def test_rope_table_row0_and_values():
    c, s = oracle.rope_table(64, 128, 10000.0)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    i = np.arange(64)
    ang = np.arange(64)[:, None] * 10000.0 ** (-2.0 * i / 128)[None, :]
    assert ulp_close(c, np.cos(ang).astype(np.float32), ulps=1)
    assert ulp_close(s, np.sin(ang).astype(np.float32), ulps=1)


def test_rope_identity_at_position_zero():
    c, s = oracle.rope_table(4, 128, 10000.0)
    t = RNG.standard_normal(4 * 128).astype(np.float32)
    assert np.array_equal(oracle.rope(t, 128, c[0], s[0]), t)


def test_rope_keeps_each_pair_norm():
    c, s = oracle.rope_table(500, 128, 10000.0)
    t = RNG.standard_normal(2 * 128).astype(np.float32)
    r = oracle.rope(t, 128, c[397], s[397])
    for j in range(2):
        a, b = t[j * 128:(j + 1) * 128], r[j * 128:(j + 1) * 128]
        na = np.hypot(a[:64].astype(np.float64), a[64:])
        nb = np.hypot(b[:64].astype(np.float64), b[64:])
        assert np.max(np.abs(na - nb) / na) < 1e-6


def test_rope_dot_product_depends_only_on_offset():
    c, s = oracle.rope_table(64, 64, 10000.0)
    q = RNG.standard_normal(64).astype(np.float32)
    k = RNG.standard_normal(64).astype(np.float32)

    def score(m, n):
        return np.dot(oracle.rope(q, 64, c[m], s[m]).astype(np.float64),
                      oracle.rope(k, 64, c[n], s[n]))
    assert abs(score(5, 2) - score(45, 42)) < 1e-4
    assert abs(score(7, 7) - np.dot(q.astype(np.float64), k)) < 1e-4
    assert abs(score(5, 2) - score(5, 3)) > 1e-3


def test_rope_vs_complex_multiplication():
    hd, theta, p = 128, 10000.0, 1234
    c, s = oracle.rope_table(p + 1, hd, theta)
    t = RNG.standard_normal(3 * hd).astype(np.float32)
    got = oracle.rope(t, hd, c[p], s[p]).reshape(3, hd)
    tt = t.reshape(3, hd).astype(np.float64)
    z = (tt[:, :64] + 1j * tt[:, 64:]) * np.exp(
        1j * p * theta ** (-2.0 * np.arange(64) / hd))
    ref = np.concatenate([z.real, z.imag], axis=1)
    assert np.max(np.abs(got - ref)) < 2e-6 * np.max(np.abs(ref))


# ---- attention ---------------------------------------------------------------

def test_attention_one_key_returns_v_exactly():
    q = RNG.standard_normal((4, 16)).astype(np.float32)
    K = RNG.standard_normal((2, 1, 16)).astype(np.float32)
    V = RNG.standard_normal((2, 1, 16)).astype(np.float32)
    out = oracle.attention(q, K, V)
    assert np.array_equal(out[:2], np.repeat(V[0], 2, axis=0))
    assert np.array_equal(out[2:], np.repeat(V[1], 2, axis=0))


def test_attention_equal_keys_gives_mean_of_values():
    q = RNG.standard_normal((2, 32)).astype(np.float32)
    K = np.repeat(RNG.standard_normal((1, 1, 32)), 9, axis=1).astype(np.float32)
    V = RNG.standard_normal((1, 9, 32)).astype(np.float32)
    out = oracle.attention(q, K, V)
    ref = V[0].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(out - ref)) < 1e-6


def test_attention_vs_numpy_softmax_and_gqa_groups():
    nh, nkv, hd, T = 8, 2, 64, 37
    q = RNG.standard_normal((nh, hd)).astype(np.float32)
    K = RNG.standard_normal((nkv, T, hd)).astype(np.float32)
    V = RNG.standard_normal((nkv, T, hd)).astype(np.float32)
    out = oracle.attention(q, K, V)
    for j in range(nh):
        g = j // (nh // nkv)
        z = K[g].astype(np.float64) @ q[j] / np.sqrt(hd)
        p = np.exp(z - z.max())
        p /= p.sum()
        assert np.sum(p) == pytest.approx(1.0, abs=1e-12)
        ref = p @ V[g]
        assert np.max(np.abs(out[j] - ref)) < 1e-6


def test_attention_heads_in_one_group_share_kv():
    nh, nkv, hd, T = 4, 2, 16, 5
    q = np.repeat(RNG.standard_normal((1, hd)), nh, axis=0).astype(np.float32)
    K = RNG.standard_normal((nkv, T, hd)).astype(np.float32)
    V = RNG.standard_normal((nkv, T, hd)).astype(np.float32)
    out = oracle.attention(q, K, V)
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[2], out[3])
    assert not np.array_equal(out[1], out[2])


# ---- silu, mul ---------------------------------------------------------------

def test_silu_closed_forms():
    g = np.array([0.0, 40.0, -40.0, 1.0, -1.0], np.float32)
    out = oracle.silu(g)
    assert out[0] == 0.0
    assert out[1] == np.float32(40.0)
    assert abs(out[2]) < 1e-15
    ref = 1.0 / (1.0 + np.exp(-1.0))
    assert out[3] == np.float32(ref)
    assert out[4] == np.float32(-1.0 + ref)


def test_silu_mul_vs_numpy():
    g = RNG.standard_normal(1000).astype(np.float32) * 4
    u = RNG.standard_normal(1000).astype(np.float32)
    s = oracle.silu(g)
    gd = g.astype(np.float64)
    assert ulp_close(s, (gd / (1 + np.exp(-gd))).astype(np.float32), ulps=1)
    m = oracle.mul(s, u)
    assert np.array_equal(m, s * u)
