"""Pins for the oracle with more than two levels (CPU only, tiny shapes).

The pages describe the hierarchy for any number of levels (PHOTON explainer,
module table and the hierarchy-shape paragraph under it: a chunker and an
encoder per level on the way up, a converter and a decoder per level on the
way down; recursive-generation section: RecGen feeds the reconstruction of
the level under the top to the top encoder, HierGen re-encodes bottom-up).
Checked here, for L = 3 and 4 with unequal chunk sizes (so that a swapped
level or a transposed index changes a shape or a value):
  * the decoders below the top equal a brute-force loop that expands every
    vector of every level on its own with explicit per-tap converters;
  * HierGen's incremental logits equal a cache-free forward over the whole
    sequence (every encoder level over its whole stream at once), also for
    a ragged prompt;
  * RecGen's cached top outputs equal a cache-free top forward over its
    inputs; its top stream never reads a token;
  * Theorem A.6 (forced feedback, and the zero top chunker) at L = 3;
  * groups of the chunk are independent below the level they share;
  * the kept caches have the lengths and sizes the memory formula states.
"""
import numpy as np
import pytest

import photon_inputs as pi
from oracle import photon_oracle as O

TINY = pi.CONFIGS["tiny"]
L3 = TINY.with_(chunk=(2, 3, 2), n_enc_hi=(1,), n_dec_hi=(1,))            # S = 12
L3B = TINY.with_(chunk=(3, 2, 2), n_enc1=2, n_enc_hi=(1,), n_dec1=1, n_dec_hi=(2,))   # S = 12
L4 = TINY.with_(chunk=(2, 2, 3, 2), n_enc_hi=(1, 1), n_dec_hi=(1, 1))      # S = 24


def make(cfg, seed=0, zero=()):
    return O.Model(cfg, pi.gen_weights(cfg, seed, zero=zero))


def prompts(cfg, B, P, seed=0):
    return pi.gen_prompts(cfg, B, P, seed)


def test_config_levels_and_weight_order():
    assert (L3.L, L3.S, L3.span(1), L3.span(2)) == (3, 12, 2, 6)
    assert [L3.enc_layers(l) for l in (1, 2)] == [1, 1]
    assert [L3B.dec_layers(l) for l in (0, 1, 2)] == [1, 1, 2]
    names = [n for n in pi.weight_names(L3) if "." not in n or n.endswith(".gf")]
    assert names == ["E", "W_ch1", "enc1.gf", "W_ch2", "enc2.gf", "W_ch3", "top.gf",
                     "W_cv3", "dec2.gf", "W_cv2", "dec1.gf", "W_cv1", "dec0.gf", "W_out"]
    shapes = dict(pi.weight_shapes(L3))
    d = L3.d_model
    assert shapes["W_ch2"] == (d, 3 * d) and shapes["W_cv2"] == (3 * d, d)
    assert shapes["W_ch3"] == (d, 2 * d) and shapes["W_cv3"] == (2 * d, d)
    with pytest.raises(ValueError):
        TINY.with_(chunk=(2, 2, 2))            # level-2 layer counts missing
    # the matched flat baseline counts every stack
    assert pi.vanilla_of(L4).n_layers == 1 + 3 + 4


def _conv_taps(m, name, v):
    """Converter by its definition: tap j is W[j*d:(j+1)*d, :] times the
    rounded input vector."""
    W = m.w[name]
    d = v.shape[-1]
    x = m.pr.r(v)
    return np.stack([W[j * d:(j + 1) * d] @ x for j in range(W.shape[0] // d)])


def _down_by_loops(m, h):
    """Every vector of every level expanded on its own, one sequence and one
    group at a time, level by level from the top; returns the level-1
    vectors of each sequence in time order."""
    cfg = m.cfg
    out = []
    for b in range(h.shape[0]):
        level = [h[b]]                                  # vectors of level L, in time order
        for l in range(cfg.L, 1, -1):
            nxt = []
            for v in level:
                c = _conv_taps(m, f"W_cv{l}", v)        # [C_l, d]
                z = m.stack(f"dec{l - 1}", cfg.dec_layers(l - 1), c[None], np.arange(c.shape[0]), None)[0]
                nxt.extend(z)
            level = nxt
        out.append(np.stack(level))
    return np.stack(out)


@pytest.mark.parametrize("cfg", [L3, L3B, L4], ids=["2x3x2", "3x2x2", "2x2x3x2"])
def test_decoders_below_the_top_equal_per_group_loops(cfg):
    m = make(cfg, seed=21)
    h = np.random.default_rng(0).standard_normal((2, cfg.d_model))
    top_hat, z1 = O.decode_down(m, h)
    assert top_hat.shape == (2, cfg.chunk[-1], cfg.d_model)
    assert z1.shape == (2, cfg.S // cfg.C1, cfg.d_model)
    np.testing.assert_allclose(z1, _down_by_loops(m, h), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("cfg,P,N", [(L3, 12, 24), (L3B, 24, 24), (L4, 24, 48)],
                         ids=["2x3x2", "3x2x2", "2x2x3x2"])
def test_hiergen_incremental_equals_teacher_forced_full(cfg, P, N):
    m = make(cfg, seed=22)
    pr = prompts(cfg, 2, P, seed=22)
    toks, lg, st, _ = O.generate(m, pr, N, mode="hiergen")
    full = O.hier_full_logits(m, np.concatenate([pr, toks], 1), P // cfg.S)
    np.testing.assert_allclose(lg, full, rtol=1e-10, atol=1e-12)
    # every lower encoder kept its K/V over the whole sequence
    T = P + N
    for l in range(1, cfg.L):
        assert st.lower[l][0]["k"].shape[1] == T // cfg.span(l)


def test_hiergen_ragged_prompt_equals_teacher_forced_full():
    cfg = L3
    m = make(cfg, seed=23)
    P, N = 12 + 7, 24 - 7
    pr = prompts(cfg, 2, P, seed=23)
    toks, lg, st, recs = O.generate(m, pr, N, mode="hiergen")
    full = O.hier_full_logits(m, np.concatenate([pr, toks], 1), P // cfg.S)
    np.testing.assert_allclose(lg, full[:, 7:], rtol=1e-10, atol=1e-12)
    assert np.array_equal(recs[0]["tokens"][:, :7], pr[:, P - 7:])


def _bottom_up_inputs(m, tokens):
    """Top inputs of a token sequence by the cache-free encoder chain."""
    cfg = m.cfg
    z = m.embed(tokens)
    for l in range(1, cfg.L):
        z = m.stack(f"enc{l}", cfg.enc_layers(l), m.chunker(f"W_ch{l}", z),
                    np.arange(tokens.shape[1] // cfg.span(l)), None)
    return m.chunker(f"W_ch{cfg.L}", z)


@pytest.mark.parametrize("cfg", [L3, L4], ids=["2x3x2", "2x2x3x2"])
def test_recgen_top_incremental_equals_full(cfg):
    m = make(cfg, seed=24)
    P, N = 2 * cfg.S, 2 * cfg.S
    pr = prompts(cfg, 2, P, seed=24)
    _, _, st, recs = O.generate(m, pr, N)
    u = np.concatenate([_bottom_up_inputs(m, pr)] + [r["u"][:, None] for r in recs], 1)
    h = O.top_full(m, u)
    for c, r in enumerate(recs):
        np.testing.assert_allclose(r["h"], h[:, 2 + c], rtol=1e-10, atol=1e-12)
        # RecGen's top input is the top chunker over the reconstruction
        np.testing.assert_allclose(r["u"], m.chunker(f"W_ch{cfg.L}", r["A_hat"])[:, 0], rtol=0, atol=0)
    assert st.lower is None and st.top_len == (P + N) // cfg.S


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_thm_a6_forced_feedback_gives_hiergen_l3(dtype):
    cfg = L3.with_(dtype=dtype)
    m = make(cfg, seed=25)
    pr = prompts(cfg, 2, 24, seed=25)
    th, _, sh, rh = O.generate(m, pr, 36, mode="hiergen")
    st = O.prefill(m, pr, "recgen")
    toks = []
    for r in rh:
        o = O.decode_chunk(m, st, "recgen", forced_u=r["u"])
        toks.append(o["tokens"])
        np.testing.assert_array_equal(o["h"], r["h"])
    np.testing.assert_array_equal(np.concatenate(toks, 1), th)
    for a, b in zip(st.top, sh.top):
        np.testing.assert_array_equal(a["k"], b["k"])
        np.testing.assert_array_equal(a["v"], b["v"])


def test_thm_a6_zero_top_chunker_makes_modes_equal_l3():
    cfg = L3.with_(dtype="bf16")
    m = make(cfg, seed=26, zero=("W_ch3",))
    pr = prompts(cfg, 2, 24, seed=26)
    tr, lr, sr, _ = O.generate(m, pr, 36, mode="recgen")
    th, lh, sh, _ = O.generate(m, pr, 36, mode="hiergen")
    np.testing.assert_array_equal(tr, th)
    np.testing.assert_array_equal(lr, lh)
    for a, b in zip(sr.top, sh.top):
        np.testing.assert_array_equal(a["k"], b["k"])
    # and it is not vacuous: with the chunker in place the modes part
    m2 = make(cfg, seed=26)
    _, _, s2r, _ = O.generate(m2, pr, 36, mode="recgen")
    _, _, s2h, _ = O.generate(m2, pr, 36, mode="hiergen")
    assert np.abs(s2r.top[0]["k"][:, 2:] - s2h.top[0]["k"][:, 2:]).max() > 1e-4


def test_recgen_top_stream_independent_of_tokens_l3():
    cfg = L3.with_(dtype="bf16")
    m = make(cfg, seed=27)
    pr = prompts(cfg, 2, 24, seed=27)
    _, _, s1, _ = O.generate(m, pr, 36)
    junk = np.random.default_rng(1).integers(0, cfg.vocab, (2, 36))
    _, _, s2, _ = O.generate(m, pr, 36, forced_tokens=junk)
    for a, b in zip(s1.top, s2.top):
        np.testing.assert_array_equal(a["k"], b["k"])
    np.testing.assert_array_equal(s1.h, s2.h)


def test_groups_are_independent_below_their_level():
    # changing a token of level-1 group k (C1 tokens) moves only the later
    # logits of group k; the level-2 groups (C1*C2 tokens) around it keep
    # every logit, since nothing but the top stream crosses a group
    cfg = L3
    m = make(cfg, seed=28)
    pr = prompts(cfg, 1, 12, seed=28)
    toks, lg, _, _ = O.generate(m, pr, 12)
    forced = toks.copy()
    forced[0, 6] = (forced[0, 6] + 1) % cfg.vocab      # level-2 group 1, level-1 group 3, position 0
    _, lg2, _, _ = O.generate(m, pr, 12, forced_tokens=forced)
    np.testing.assert_array_equal(lg[0, :7], lg2[0, :7])
    np.testing.assert_array_equal(lg[0, 8:], lg2[0, 8:])
    assert np.abs(lg[0, 7] - lg2[0, 7]).max() > 1e-6


def test_memory_formula_matches_the_kept_caches():
    for cfg in (L3, L4):
        m = make(cfg, seed=29)
        P, N = 2 * cfg.S, cfg.S
        _, _, st, _ = O.generate(m, prompts(cfg, 2, P, seed=29), N, mode="hiergen")
        kv = O.kv_bytes(cfg, 2, P + N, "hiergen")
        eb = 4
        kept = sum(e["k"].size + e["v"].size for l in st.lower for e in st.lower[l]) * eb
        assert kv["lower"] == kept
        assert kv["top"] == sum(e["k"].size + e["v"].size for e in st.top) * eb
        # the token decoder's cache: C1 slots for every level-1 group
        assert kv["dec"] == cfg.n_dec0 * 2 * 2 * (cfg.S // cfg.C1) * cfg.C1 * cfg.d_model * eb
        assert O.kv_bytes(cfg, 2, P + N)["lower"] == 0


def test_consistency_at_the_level_under_the_top():
    m = make(L3, seed=30)
    st = O.prefill(m, prompts(L3, 2, 24, seed=30), "hiergen")
    o = O.decode_chunk(m, st, "hiergen")
    assert o["A_hat"].shape == o["A"].shape == (2, L3.chunk[-1], L3.d_model)
    d = O.consistency(o["A_hat"], o["A"])
    assert d.shape == (2, 2) and (d >= 0).all() and (d <= 2).all()
