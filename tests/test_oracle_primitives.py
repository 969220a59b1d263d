"""Pins for the oracle's primitives (CPU only).

Each primitive is checked against something other than itself: textbook
values stored under tests/golden, closed forms, invariants, or a library
routine (torch CPU in float64) that computes the same definition.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import photon_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------- bf16 rounding ----------------
def test_bf16_textbook_points():
    for x, want in _gold("textbook.json")["bf16"]["points"]:
        got = O.round_bf16(np.array([x]))[0]
        want = math.inf if want == "inf" else want
        assert got == want, (x, got, want)


def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * s for s in
                        (1e-3, 1.0, 1e3, 1e30)])
    x32 = x.astype(np.float32).astype(np.float64)   # torch goes via the value
    want = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.round_bf16(x32), want)


def test_bf16_ties_go_to_even():
    # exactly halfway between neighbours 1 and 1+2^-7 -> 1 (even significand)
    one = 1.0 + 2.0 ** -8
    assert O.round_bf16(np.array([one]))[0] == 1.0
    # halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> 1+2^-6
    assert O.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # just above the tie rounds up
    assert O.round_bf16(np.array([one + 1e-9]))[0] == 1.0 + 2.0 ** -7


def test_precision_f32_is_identity():
    x = np.random.default_rng(0).standard_normal(100)
    np.testing.assert_array_equal(O.Precision("f32").r(x), x)


# ---------------- RMSNorm ----------------
def test_rmsnorm_closed_form():
    x = np.array([[3.0, 4.0]])                 # mean(x^2) = 12.5
    g = np.array([1.0, 2.0])
    want = np.array([[3.0, 8.0]]) / math.sqrt(12.5 + 1e-5)
    np.testing.assert_allclose(O.rmsnorm(x, g, 1e-5), want, rtol=1e-15)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    g = rng.standard_normal(64)
    want = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g),
                      eps=1e-5).numpy()
    np.testing.assert_allclose(O.rmsnorm(x, g, 1e-5), want, rtol=1e-13)


# ---------------- GELU ----------------
def test_gelu_textbook_points():
    for z, want in _gold("textbook.json")["gelu"]["points"]:
        assert abs(O.gelu(np.array([z]))[0] - want) < 1e-15


def test_gelu_matches_torch_exact():
    z = np.linspace(-8, 8, 1001)
    want = F.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(O.gelu(z), want, rtol=1e-12, atol=1e-18)


# ---------------- RoPE ----------------
def test_rope_hd2_is_rotation_by_pos_radians():
    x = np.array([[[[1.0, 0.0]]], [[[0.3, -0.7]]]])   # [2 rows, T=1, H=1, hd=2]
    for pos in (0, 1, 5):
        y = O.rope(x, np.array([pos]), 1e4)
        c, s = math.cos(pos), math.sin(pos)
        R = np.array([[c, -s], [s, c]])
        for r in range(2):
            np.testing.assert_allclose(y[r, 0, 0], R @ x[r, 0, 0], rtol=1e-15,
                                       atol=1e-15)


def test_rope_second_pair_frequency():
    # hd = 4: pair (x1, x3) turns at theta^(-2/4) = 1/100 rad per position
    x = np.zeros((1, 1, 1, 4))
    x[..., 1] = 1.0
    y = O.rope(x, np.array([7]), 1e4)[0, 0, 0]
    np.testing.assert_allclose(y, [0.0, math.cos(0.07), 0.0, math.sin(0.07)],
                               atol=1e-15)


def test_rope_invariants():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 1, 3, 32))
    k = rng.standard_normal((1, 1, 3, 32))
    # norm preserving
    y = O.rope(q, np.array([11]), 1e4)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1),
                               np.linalg.norm(q, axis=-1), rtol=1e-13)
    # q.k depends only on the position difference
    dots = []
    for base in (0, 3, 40):
        qa = O.rope(q, np.array([base + 5]), 1e4)
        ka = O.rope(k, np.array([base + 2]), 1e4)
        dots.append((qa * ka).sum(-1))
    np.testing.assert_allclose(dots[0], dots[1], rtol=1e-12)
    np.testing.assert_allclose(dots[0], dots[2], rtol=1e-12)
    # position 0 is the identity
    np.testing.assert_array_equal(O.rope(q, np.array([0]), 1e4), q)


# ---------------- attention ----------------
def test_attention_matches_torch_sdpa_causal():
    rng = np.random.default_rng(3)
    B, T, H, hd = 2, 9, 3, 8
    q, k, v = (rng.standard_normal((B, T, H, hd)) for _ in range(3))
    got = O.attention(q, k, v, 0)
    tt = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3)
    want = F.scaled_dot_product_attention(tt(q), tt(k), tt(v), is_causal=True)
    np.testing.assert_allclose(got, want.permute(0, 2, 1, 3).numpy(),
                               rtol=1e-12, atol=1e-14)


def test_attention_with_cache_prefix_matches_brute_force():
    rng = np.random.default_rng(4)
    B, n_prev, Tq, H, hd = 1, 5, 3, 2, 4
    Tk = n_prev + Tq
    q = rng.standard_normal((B, Tq, H, hd))
    k = rng.standard_normal((B, Tk, H, hd))
    v = rng.standard_normal((B, Tk, H, hd))
    got = O.attention(q, k, v, n_prev)
    for t in range(Tq):
        for h in range(H):
            s = [sum(q[0, t, h, e] * k[0, j, h, e] for e in range(hd)) / 2.0
                 for j in range(n_prev + t + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = sum(w)
            o = [sum(w[j] * v[0, j, h, e] for j in range(len(w))) / z
                 for e in range(hd)]
            np.testing.assert_allclose(got[0, t, h], o, rtol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((1, 4, 1, 3))
    k = np.zeros((1, 4, 1, 3))
    q = rng.standard_normal((1, 1, 1, 3))
    # one visible key -> its value; equal scores -> mean of the values
    np.testing.assert_allclose(O.attention(q, k[:, :1], v[:, :1], 0)[0, 0, 0],
                               v[0, 0, 0], rtol=1e-15)
    np.testing.assert_allclose(O.attention(q, k, v, 3)[0, 0, 0],
                               v[0, :, 0].mean(0), rtol=1e-14)


# ---------------- chunker / converter ----------------
class _Cfg:
    dtype = "f32"


def _model_with(weights):
    m = O.Model.__new__(O.Model)
    m.cfg = _Cfg()
    m.pr = O.Precision("f32")
    m.w = weights
    return m


def test_chunker_is_concat_in_time_order_then_linear():
    rng = np.random.default_rng(6)
    B, T, d, C = 2, 8, 3, 4
    z = rng.standard_normal((B, T, d))
    W = rng.standard_normal((d, C * d))
    got = _model_with({"W": W}).chunker("W", z)
    for b in range(B):
        for g in range(T // C):
            cat = []
            for j in range(C):               # explicit concatenation
                cat.extend(z[b, g * C + j])
            want = [sum(W[o, i] * cat[i] for i in range(C * d)) for o in range(d)]
            np.testing.assert_allclose(got[b, g], want, rtol=1e-12)


def test_converter_is_conv_transpose_kernel_eq_stride():
    rng = np.random.default_rng(8)
    B, d, C = 3, 5, 4
    h = rng.standard_normal((B, d))
    W = rng.standard_normal((C * d, d))
    got = _model_with({"W": W}).converter("W", h)          # [B, C, d]
    # torch conv_transpose1d: weight [in_ch, out_ch, kernel]; input [B, in, 1]
    wt = torch.from_numpy(W.reshape(C, d, d).transpose(2, 1, 0).copy())
    y = F.conv_transpose1d(torch.from_numpy(h)[:, :, None], wt, stride=C)
    np.testing.assert_allclose(got, y.permute(0, 2, 1).numpy(), rtol=1e-12)


# ---------------- TPM arithmetic ----------------
def test_tpm_formula_reproduces_printed_table():
    g = _gold("tpm_table.json")
    for row in g["rows"]:
        got = O.tpm(row["throughput"], row["memory"])
        assert round(got, row["digits"]) == pytest.approx(row["tpm"], abs=0.011 + (
            0.5 if row["digits"] == 0 else 0)), row
    for r in g["ratios"]:
        got = r["num"] / r["den"]
        assert abs(got - r["printed"]) / r["printed"] < 0.01, r
