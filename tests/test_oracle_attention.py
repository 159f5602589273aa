"""Pins for the oracle's attention (CPU).

Scaled dot-product attention per head, the "FlashAttention" row of the
tiled-kernel table in "Tiling Strategies", section 5: s_ij = scale * q_i . k_j
over the allowed keys (j < Skv, and j <= i when causal), p = softmax(s),
O_i = sum_j p_ij v_j.  The oracle is tied to things other than itself:
  * a library routine: torch's float64 scaled_dot_product_attention on the CPU,
    with and without the causal mask, Sq != Skv included;
  * closed forms: one key gives O = V[0] exactly; zero queries give uniform
    weights, so O_i is the mean of the allowed value rows; keys that pick one
    row through a dominant score return that row;
  * invariants: adding one vector to every key adds a per-row constant to the
    scores and leaves O unchanged; permuting keys and values together leaves
    non-causal O unchanged;
  * the magnitude outputs: mag = softmax-weighted |V|, smax = largest
    scale * sum |q||k|, against direct evaluation.
Planted mistakes in a copy of oracle.c must each fail one of these checks.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _real(Q, K, V, H, Sq, Skv, D, scale, causal):
    return oracle.attention_f64(Q, K, V, H, Sq, Skv, D, scale, causal)


def _f32(x):
    return float(np.float32(x))


def _sdpa(Q, K, V, scale, causal):
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(Q), t(K), t(V), scale=scale, is_causal=causal).numpy()


CASES = [(2, 5, 7, 8), (1, 9, 9, 16), (3, 1, 4, 4), (2, 6, 3, 32), (1, 17, 17, 64)]


def check_torch_sdpa(att):
    rng = np.random.default_rng(1)
    for (H, Sq, Skv, D) in CASES:
        Q = rng.standard_normal((H, Sq, D)).astype(np.float32)
        K = rng.standard_normal((H, Skv, D)).astype(np.float32)
        V = rng.standard_normal((H, Skv, D)).astype(np.float32)
        sc = _f32(1.0 / np.sqrt(D))
        for causal in (False, True):
            O, _, _ = att(Q, K, V, H, Sq, Skv, D, sc, causal)
            ref = _sdpa(Q, K, V, sc, causal)
            assert np.allclose(O, ref, rtol=1e-12, atol=1e-12), (H, Sq, Skv, D, causal)


def check_single_key(att):
    rng = np.random.default_rng(2)
    H, Sq, D = 2, 5, 8
    Q = rng.standard_normal((H, Sq, D)).astype(np.float32)
    K = rng.standard_normal((H, 1, D)).astype(np.float32)
    V = rng.standard_normal((H, 1, D)).astype(np.float32)
    for causal in (False, True):
        O, mag, _ = att(Q, K, V, H, Sq, 1, D, 0.7, causal)
        assert np.array_equal(O, np.broadcast_to(V.astype(np.float64), O.shape))
        assert np.array_equal(mag, np.abs(O))


def check_uniform_weights(att):
    rng = np.random.default_rng(3)
    H, S, D = 2, 6, 4
    Q = np.zeros((H, S, D), np.float32)
    K = rng.standard_normal((H, S, D)).astype(np.float32)
    V = rng.standard_normal((H, S, D)).astype(np.float32)
    O, _, _ = att(Q, K, V, H, S, S, D, 0.5, False)
    assert np.allclose(O, np.broadcast_to(V.astype(np.float64).mean(axis=1, keepdims=True),
                                          O.shape), rtol=1e-13, atol=1e-14)
    O, _, _ = att(Q, K, V, H, S, S, D, 0.5, True)
    cum = np.cumsum(V.astype(np.float64), axis=1) / np.arange(1, S + 1)[None, :, None]
    assert np.allclose(O, cum, rtol=1e-13, atol=1e-14)


def check_dominant_key(att):
    rng = np.random.default_rng(4)
    H, Sq, Skv, D = 1, 3, 5, 8
    K = np.zeros((H, Skv, D), np.float32)
    for j in range(Skv):
        K[0, j, j] = 1.0
    V = rng.standard_normal((H, Skv, D)).astype(np.float32)
    picks = [3, 0, 4]
    Q = np.zeros((H, Sq, D), np.float32)
    for i, j in enumerate(picks):
        Q[0, i, j] = 200.0          # score 200 for key j, 0 for the others
    O, _, _ = att(Q, K, V, H, Sq, Skv, D, 1.0, False)
    for i, j in enumerate(picks):
        assert np.allclose(O[0, i], V[0, j], rtol=0, atol=1e-80)


def check_key_shift_invariance(att):
    rng = np.random.default_rng(5)
    H, Sq, Skv, D = 2, 4, 6, 8
    Q = (rng.integers(-3, 4, (H, Sq, D))).astype(np.float32)
    K = (rng.integers(-3, 4, (H, Skv, D))).astype(np.float32)
    V = rng.standard_normal((H, Skv, D)).astype(np.float32)
    c = (rng.integers(-3, 4, (H, 1, D))).astype(np.float32)
    for causal in (False, True):
        O1, _, _ = att(Q, K, V, H, Sq, Skv, D, 0.25, causal)
        O2, _, _ = att(Q, K + c, V, H, Sq, Skv, D, 0.25, causal)
        assert np.allclose(O1, O2, rtol=1e-12, atol=1e-13)


def check_kv_permutation(att):
    rng = np.random.default_rng(6)
    H, Sq, Skv, D = 2, 5, 7, 8
    Q = rng.standard_normal((H, Sq, D)).astype(np.float32)
    K = rng.standard_normal((H, Skv, D)).astype(np.float32)
    V = rng.standard_normal((H, Skv, D)).astype(np.float32)
    perm = rng.permutation(Skv)
    O1, _, _ = att(Q, K, V, H, Sq, Skv, D, 0.3, False)
    O2, _, _ = att(Q, K[:, perm], V[:, perm], H, Sq, Skv, D, 0.3, False)
    assert np.allclose(O1, O2, rtol=1e-12, atol=1e-13)


def check_magnitudes(att):
    rng = np.random.default_rng(7)
    H, Sq, Skv, D = 1, 4, 6, 5
    Q = rng.standard_normal((H, Sq, D)).astype(np.float32)
    K = rng.standard_normal((H, Skv, D)).astype(np.float32)
    V = rng.standard_normal((H, Skv, D)).astype(np.float32)
    sc = 0.4
    for causal in (False, True):
        _, mag, smax = att(Q, K, V, H, Sq, Skv, D, sc, causal)
        q, k, v = (a.astype(np.float64)[0] for a in (Q, K, V))
        s = _f32(sc) * q @ k.T
        allowed = np.tril(np.ones((Sq, Skv), bool)) if causal else np.ones((Sq, Skv), bool)
        s = np.where(allowed, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        assert np.allclose(mag[0], p @ np.abs(v), rtol=1e-12, atol=1e-14)
        sabs = _f32(sc) * np.abs(q) @ np.abs(k).T
        assert np.allclose(smax[0], np.where(allowed, sabs, 0.0).max(axis=1), rtol=1e-13)


def check_magnitude_closed_forms(att):
    """mag and smax against values written out by hand, not by restating the
    oracle's formula: one key (every weight is 1, so mag is |v| of that key
    and smax is scale * sum_d |q_d||k_d|); zero queries (uniform weights over
    the allowed keys, so mag is the mean |v| over them, and smax is 0); keys
    that grow with their index (the largest allowed key gives smax)."""
    H, D = 1, 4
    # One key: q = (1, -2, 3, 0), k = (2, 1, -1, 5), scale 1/4.
    Q = np.array([[[1, -2, 3, 0], [0, 0, 0, 0]]], np.float32)
    K = np.array([[[2, 1, -1, 5]]], np.float32)
    V = np.array([[[-1.5, 2.0, 0.25, -3.0]]], np.float32)
    _, mag, smax = att(Q, K, V, H, 2, 1, D, 0.25, False)
    assert np.array_equal(mag[0], np.abs(V[0, [0, 0]]).astype(np.float64))
    assert smax[0, 0] == 0.25 * (2 + 2 + 3 + 0) and smax[0, 1] == 0.0
    # Zero queries, five keys: uniform weights.
    Sq, Skv = 3, 5
    Q = np.zeros((H, Sq, D), np.float32)
    K = np.arange(H * Skv * D, dtype=np.float32).reshape(H, Skv, D) - 7
    V = np.array([[[1, -2, 0, 4], [3, 0, -1, 1], [-5, 2, 2, 0], [0, 1, 1, -1],
                   [2, 2, -3, 3]]], np.float32)
    _, mag, smax = att(Q, K, V, H, Sq, Skv, D, 0.5, False)
    want = np.array([11, 7, 7, 9], np.float64) / 5      # column sums of |V| over 5 keys
    for i in range(Sq):
        assert np.allclose(mag[0, i], want, rtol=1e-15, atol=0)
    assert np.all(smax == 0.0)
    # Causal: query i sees keys 0..i, uniform weights over them.
    _, mag, smax = att(Q, K, V, H, Sq, Skv, D, 0.5, True)
    want_rows = [np.array([1, 2, 0, 4]) / 1, np.array([4, 2, 1, 5]) / 2,
                 np.array([9, 4, 3, 5]) / 3]
    for i in range(Sq):
        assert np.allclose(mag[0, i], want_rows[i], rtol=1e-15, atol=0)
    # Keys k_j = (j, j, j, j) and q = (1, 1, 1, 1): scale * sum_d |q||k_j| = 4 j / 8.
    Sq, Skv = 4, 6
    Q = np.ones((H, Sq, D), np.float32)
    K = np.repeat(np.arange(Skv, dtype=np.float32)[None, :, None], D, axis=2)
    V = np.ones((H, Skv, D), np.float32)
    _, _, smax = att(Q, K, V, H, Sq, Skv, D, 0.125, False)
    assert np.all(smax[0] == 0.125 * 4 * (Skv - 1))
    _, _, smax = att(Q, K, V, H, Sq, Skv, D, 0.125, True)
    assert np.array_equal(smax[0], 0.125 * 4 * np.arange(Sq, dtype=np.float64))


PIN_CHECKS = [check_torch_sdpa, check_single_key, check_uniform_weights, check_dominant_key,
              check_key_shift_invariance, check_kv_permutation, check_magnitudes,
              check_magnitude_closed_forms]


@pytest.mark.parametrize("chk", PIN_CHECKS, ids=lambda c: c.__name__)
def test_attention_oracle_pin(chk):
    chk(_real)


def test_attention_rows_match_full_and_empty_keys():
    rng = np.random.default_rng(8)
    H, Sq, Skv, D = 3, 7, 9, 16
    Q = rng.standard_normal((H, Sq, D)).astype(np.float32)
    K = rng.standard_normal((H, Skv, D)).astype(np.float32)
    V = rng.standard_normal((H, Skv, D)).astype(np.float32)
    for causal in (False, True):
        O, mag, smax = oracle.attention_f64(Q, K, V, H, Sq, Skv, D, 0.25, causal)
        rows = [0, 5, 8, 20, 13]
        o, m, sm = oracle.attention_rows_f64(Q, K, V, H, Sq, Skv, D, 0.25, rows, causal)
        assert np.array_equal(o, O.reshape(-1, D)[rows])
        assert np.array_equal(m, mag.reshape(-1, D)[rows])
        assert np.array_equal(sm, smax.reshape(-1)[rows])
    O, mag, smax = oracle.attention_f64(Q, K[:, :0], V[:, :0], H, Sq, 0, D, 0.25)
    assert np.all(O == 0.0) and np.all(mag == 0.0)


# ------------------------------------------------------------- planted mistakes

ATT_MUTATIONS = {
    "scale_ignored": ("s[j] = scale * dot;", "s[j] = dot;"),
    "causal_off_by_one": ("const int64_t nj = causal ? (i + 1 < Skv ? i + 1 : Skv) : Skv;",
                          "const int64_t nj = causal ? (i < Skv ? i : Skv) : Skv;"),
    "key_index_transposed": ("dot += (double)q[d] * (double)K[j * D + d];",
                             "dot += (double)q[d] * (double)K[(d % Skv) * D + (j % D)];"),
    "value_column_reversed": ("acc += s[j] * (double)V[j * D + d];",
                              "acc += s[j] * (double)V[j * D + (D - 1 - d)];"),
    "normaliser_dropped": ("o[d] = nj > 0 ? acc / l : 0.0;", "o[d] = nj > 0 ? acc : 0.0;"),
    "abs_dropped": ("accabs += s[j] * fabs((double)V[j * D + d]);",
                    "accabs += s[j] * (double)V[j * D + d];"),
    "fp32_scores": ("s[j] = scale * dot;", "s[j] = (float)(scale * (float)dot);"),
    "exp_without_max": ("s[j] = exp(s[j] - m);  /* p_ij */", "s[j] = exp(s[j] - 1.0);  /* p_ij */"),
}


def _build_mutant(tmp_path, name):
    old, new = ATT_MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor missing: %s" % name
    src = tmp_path / ("oracle_a_%s.c" % name)
    src.write_text(text.replace(old, new))
    so = tmp_path / ("liboracle_a_%s.so" % name)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", str(src), "-o", str(so), "-lm"], check=True)
    lib = ctypes.CDLL(str(so))
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_attention_f64.argtypes = [i64, i64, i64, i64, p, p, p, ctypes.c_float,
                                         ctypes.c_int, p, p, p]
    lib.oracle_attention_f64.restype = ctypes.c_int

    def att(Q, K, V, H, Sq, Skv, D, scale, causal):
        q, k, v = (np.ascontiguousarray(np.asarray(a, np.float32).ravel()) for a in (Q, K, V))
        O = np.empty((H, Sq, D))
        mag = np.empty((H, Sq, D))
        smax = np.empty((H, Sq))
        assert lib.oracle_attention_f64(H, Sq, Skv, D, q.ctypes.data, k.ctypes.data,
                                        v.ctypes.data, scale, int(causal), O.ctypes.data,
                                        mag.ctypes.data, smax.ctypes.data) == 0
        return O, mag, smax

    return att


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(ATT_MUTATIONS))
def test_planted_mistake_in_attention_fails_a_pin(tmp_path, name):
    att = _build_mutant(tmp_path, name)
    failed = []
    for chk in PIN_CHECKS:
        try:
            with np.errstate(all="ignore"):
                chk(att)
        except AssertionError:
            failed.append(chk.__name__)
    assert failed, "mutation %s passed every pin" % name


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_unmutated_attention_copy_passes(tmp_path):
    ATT_MUTATIONS["_noop"] = ("s[j] = scale * dot;", "s[j] = scale * dot;")
    try:
        att = _build_mutant(tmp_path, "_noop")
        for chk in PIN_CHECKS:
            chk(att)
    finally:
        del ATT_MUTATIONS["_noop"]
