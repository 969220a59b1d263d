"""Model-level pins for the oracle (CPU only, tiny configurations).

What the pages fix for the generation procedure, checked here:
  * Theorem A.6 (PHOTON explainer, recursive-generation section): with the
    bottleneck reconstruction forced equal to the encoder summary, RecGen and
    HierGen make the same top-level updates and emit the same tokens; the
    special case W_ch2 = 0 makes the premise hold with no forcing.
  * the top-level KV holds ceil(T / (C1*C2)) states; the decoder cache does
    not grow with the context; RecGen keeps no level-1 cache after prefill
    (same section, cache-drop paragraph; module table, Decoder row);
  * incremental decoding equals a full recompute without caches;
  * RecGen's top stream never sees the tokens, sub-chunks are independent
    and sequences are independent (top-down expansion runs in parallel,
    abstract and module table).
A Transformer block is also checked against torch library routines.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import photon_inputs as pi
from oracle import photon_oracle as O


def tiny(dtype="f32", **kw):
    cfg = pi.CONFIGS["tiny"].with_(dtype=dtype, **kw)
    return cfg


def make(cfg, seed=0, zero=()):
    return O.Model(cfg, pi.gen_weights(cfg, seed, zero=zero))


def prompts(cfg, B, P, seed=0):
    return pi.gen_prompts(cfg, B, P, seed)


# ---------------- block vs library routines ----------------
def test_stack_matches_torch_library_block():
    cfg = tiny(n_dec1=2)
    m = make(cfg, seed=11)
    rng = np.random.default_rng(0)
    B, T, d, H = 2, 5, cfg.d_model, cfg.n_heads
    x = rng.standard_normal((B, T, d))
    # positions all 0 make the rotary embedding the identity, so every step
    # is a plain library call
    got = m.stack("dec1", 2, x, np.zeros(T, dtype=np.int64), None)
    t = torch.from_numpy(x)
    W = {k: torch.from_numpy(v) for k, v in m.w.items()}
    for l in range(2):
        p = f"dec1.{l}."
        a = F.rms_norm(t, (d,), W[p + "g1"], eps=1e-5)
        heads = lambda y: y.reshape(B, T, H, d // H).transpose(1, 2)
        q, k, v = (heads(F.linear(a, W[p + n])) for n in ("Wq", "Wk", "Wv"))
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        t = t + F.linear(o.transpose(1, 2).reshape(B, T, d), W[p + "Wo"])
        a = F.rms_norm(t, (d,), W[p + "g2"], eps=1e-5)
        t = t + F.linear(F.gelu(F.linear(a, W[p + "W1"])), W[p + "W2"])
    want = F.rms_norm(t, (d,), W["dec1.gf"], eps=1e-5).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13)


def test_rope_positions_enter_only_through_q_and_k():
    # shifting every rotary position by a constant leaves a causal stack's
    # output unchanged (scores depend on position differences only)
    cfg = tiny()
    m = make(cfg, seed=12)
    x = np.random.default_rng(1).standard_normal((1, 6, cfg.d_model))
    a = m.stack("top", 1, x, np.arange(6), None)
    b = m.stack("top", 1, x, np.arange(6) + 37, None)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)
    c = m.stack("top", 1, x, np.arange(6) * 2, None)
    assert np.abs(a - c).max() > 1e-6


# ---------------- cache invariants ----------------
@pytest.mark.parametrize("T", [1, 15, 16, 17, 64, 96, 100])
def test_top_length_is_ceil_T_over_S(T):
    cfg = tiny()
    assert O.top_states(cfg, T) == -(-T // 16)


def test_top_length_after_generation():
    cfg = tiny()
    m = make(cfg)
    toks, lg, st, _ = O.generate(m, prompts(cfg, 2, 64), 32)
    T = 64 + 32
    assert st.top_len == O.top_states(cfg, T) == 6
    for e in st.top:
        assert e["k"].shape[1] == e["v"].shape[1] == 6
    assert st.lvl1 is None                      # RecGen dropped level 1


def test_hiergen_keeps_level1_cache():
    cfg = tiny()
    m = make(cfg)
    _, _, st, _ = O.generate(m, prompts(cfg, 2, 32), 32, mode="hiergen")
    assert st.lvl1 is not None
    assert st.lvl1[0]["k"].shape[1] == (32 + 32) // cfg.C1


def test_decoder_cache_independent_of_context():
    for cfg in (tiny(), pi.CONFIGS["m600"], pi.CONFIGS["m600_2x2"]):
        a = O.kv_bytes(cfg, 4, 1024)
        b = O.kv_bytes(cfg, 4, 65536)
        assert a["dec"] == b["dec"] > 0
        assert b["top"] > a["top"]
        assert a["lower"] == 0
        assert O.kv_bytes(cfg, 4, 1024, "hiergen")["lower"] > 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layers", [(1, 2), (3, 1)], ids=["dec1<dec0", "dec1>dec0"])
def test_dec_bytes_equal_the_cache_the_token_decoder_builds(dtype, layers):
    # the TPM denominator's decoder term against the in-chunk caches the
    # token decoder really fills (every empty_cache the chunk creates for it,
    # measured after the chunk), with n_dec1 != n_dec0 so that counting the
    # wrong decoder's layers fails
    n_dec1, n_dec0 = layers
    cfg = tiny(dtype, n_dec1=n_dec1, n_dec0=n_dec0)
    m = make(cfg)
    st = O.prefill(m, prompts(cfg, 3, 32))
    made = []
    orig = m.empty_cache

    def spy(n_layers, B):
        c = orig(n_layers, B)
        made.append(c)
        return c

    m.empty_cache = spy
    O.decode_chunk(m, st)
    b = 2 if dtype == "bf16" else 4
    dec_caches = [c for c in made if len(c) == cfg.n_dec0 and c[0]["k"].shape[0] == 3 * cfg.S // cfg.C1]
    assert len(dec_caches) == 1
    built = sum(e["k"].size + e["v"].size for e in dec_caches[0]) * b
    assert built == O.kv_bytes(cfg, 3, 32 + cfg.S)["dec"] == O.kv_bytes(cfg, 3, 4096)["dec"]


def test_state_from_arrays_decodes_like_the_prefilled_state():
    # an injected state laid out as photon_inputs.gen_decode_state lays it
    # out ([layers, n, H, hd] per sequence) and filled with a real
    # prefill's caches decodes exactly like that prefill's own state
    for mode in ("recgen", "hiergen"):
        cfg = tiny()
        m = make(cfg)
        st = O.prefill(m, prompts(cfg, 2, 48), mode)
        seqs = []
        for b in range(2):
            e = {"top_k": np.stack([c["k"][b] for c in st.top]), "top_v": np.stack([c["v"][b] for c in st.top]),
                 "h": st.h[b]}
            if mode == "hiergen":
                e["low_k"] = {1: np.stack([c["k"][b] for c in st.lower[1]])}
                e["low_v"] = {1: np.stack([c["v"][b] for c in st.lower[1]])}
            seqs.append(e)
        inj = O.state_from_arrays(m, seqs)
        assert inj.top_len == st.top_len == 48 // cfg.S
        for _ in range(2):
            a, b_ = O.decode_chunk(m, st, mode), O.decode_chunk(m, inj, mode)
            np.testing.assert_array_equal(a["tokens"], b_["tokens"])
            np.testing.assert_array_equal(a["logits"], b_["logits"])
            np.testing.assert_array_equal(a["h"], b_["h"])


def test_injected_state_shapes_and_spread():
    # the seeded stand-in has the shapes of a prefilled state, bf16-exact
    # values for bf16 models and the stated spreads
    cfg = pi.CONFIGS["m150"]
    st = pi.gen_decode_state(cfg, 3, 64, "hiergen", seed=1)
    assert st["top_k"].shape == (cfg.n_top, 64, cfg.n_heads, cfg.head_dim)
    assert st["low_v"][1].shape == (cfg.n_enc1, 64 * cfg.C2, cfg.n_heads, cfg.head_dim)
    for a in (st["top_k"], st["h"], st["low_k"][1]):
        assert (O.round_bf16(a.astype(np.float64)) == a).all()
    assert abs(st["top_v"].std() / (0.02 * np.sqrt(cfg.d_model)) - 1) < 0.01
    assert abs(st["h"].std() - 1) < 0.1
    again = pi.gen_decode_state(cfg, 3, 64, "recgen", seed=1)
    np.testing.assert_array_equal(again["top_k"], st["top_k"])


# ---------------- incremental == full recompute ----------------
@pytest.mark.parametrize("P,N", [(16, 16), (32, 48), (64, 32)])
def test_recgen_top_incremental_equals_full(P, N):
    cfg = tiny()
    m = make(cfg, seed=3)
    pr = prompts(cfg, 2, P, seed=3)
    _, _, st, recs = O.generate(m, pr, N)
    # prefill's top inputs, then the fed-back u_i of each chunk
    e = m.embed(pr)
    A1 = m.stack("enc1", 1, m.chunker("W_ch1", e), np.arange(P // 4), None)
    u = np.concatenate([m.chunker("W_ch2", A1)] +
                       [r["u"][:, None] for r in recs], 1)
    h = O.top_full(m, u)
    for c, r in enumerate(recs):
        np.testing.assert_allclose(r["h"], h[:, P // 16 + c], rtol=1e-10,
                                   atol=1e-12)


def test_recgen_token_decoder_incremental_equals_full():
    cfg = tiny()
    m = make(cfg, seed=4)
    _, _, st, recs = O.generate(m, prompts(cfg, 2, 32, seed=4), 32)
    for r in recs:
        B = r["A_hat"].shape[0]
        c0 = m.converter("W_cv1", r["A_hat"]).reshape(B * 4, 4, -1)
        y = r["tokens"].reshape(B * 4, 4)
        x = c0.copy()
        x[:, 1:] += m.embed(y[:, :-1])
        z = m.stack("dec0", 1, x, np.arange(4), None)
        lg = m.logits(z).reshape(B, 16, -1)
        np.testing.assert_allclose(r["logits"], lg, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("P,N", [(16, 32), (64, 32)])
def test_hiergen_incremental_equals_teacher_forced_full(P, N):
    cfg = tiny()
    m = make(cfg, seed=5)
    pr = prompts(cfg, 2, P, seed=5)
    toks, lg, _, _ = O.generate(m, pr, N, mode="hiergen")
    full = O.hier_full_logits(m, np.concatenate([pr, toks], 1), P // 16)
    np.testing.assert_allclose(lg, full, rtol=1e-10, atol=1e-12)


# ---------------- Theorem A.6 ----------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_thm_a6_forced_feedback_gives_hiergen(dtype):
    cfg = tiny(dtype)
    m = make(cfg, seed=6)
    pr = prompts(cfg, 2, 32, seed=6)
    th, lh, sh, rh = O.generate(m, pr, 48, mode="hiergen")
    st = O.prefill(m, pr, "recgen")
    toks = []
    for r in rh:                                  # force u_i := Ch2(A_i)
        o = O.decode_chunk(m, st, "recgen", forced_u=r["u"])
        toks.append(o["tokens"])
        np.testing.assert_array_equal(o["h"], r["h"])
    np.testing.assert_array_equal(np.concatenate(toks, 1), th)
    for a, b in zip(st.top, sh.top):
        np.testing.assert_array_equal(a["k"], b["k"])
        np.testing.assert_array_equal(a["v"], b["v"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_thm_a6_zero_chunker_makes_modes_equal(dtype):
    cfg = tiny(dtype)
    m = make(cfg, seed=7, zero=("W_ch2",))
    pr = prompts(cfg, 2, 32, seed=7)
    tr, lr, sr, _ = O.generate(m, pr, 48, mode="recgen")
    th, lh, sh, _ = O.generate(m, pr, 48, mode="hiergen")
    np.testing.assert_array_equal(tr, th)
    np.testing.assert_array_equal(lr, lh)
    for a, b in zip(sr.top, sh.top):
        np.testing.assert_array_equal(a["k"], b["k"])


def test_thm_a6_is_not_vacuous():
    cfg = tiny()
    m = make(cfg, seed=8)
    pr = prompts(cfg, 2, 32, seed=8)
    _, _, sr, _ = O.generate(m, pr, 32, mode="recgen")
    _, _, sh, _ = O.generate(m, pr, 32, mode="hiergen")
    np.testing.assert_array_equal(sr.top[0]["k"][:, :2], sh.top[0]["k"][:, :2])
    assert np.abs(sr.top[0]["k"][:, 2:] - sh.top[0]["k"][:, 2:]).max() > 1e-4


# ---------------- RecGen structure ----------------
def test_recgen_top_stream_independent_of_tokens():
    cfg = tiny("bf16")
    m = make(cfg, seed=9)
    pr = prompts(cfg, 2, 32, seed=9)
    _, _, s1, r1 = O.generate(m, pr, 48)
    junk = np.random.default_rng(0).integers(0, cfg.vocab, (2, 48))
    _, _, s2, r2 = O.generate(m, pr, 48, forced_tokens=junk)
    for a, b in zip(s1.top, s2.top):
        np.testing.assert_array_equal(a["k"], b["k"])
        np.testing.assert_array_equal(a["v"], b["v"])
    np.testing.assert_array_equal(s1.h, s2.h)


def test_subchunks_are_independent():
    cfg = tiny()
    m = make(cfg, seed=10)
    pr = prompts(cfg, 1, 16, seed=10)
    toks, lg, _, _ = O.generate(m, pr, 16)
    forced = toks.copy()
    forced[0, 4:8] = (forced[0, 4:8] + 1) % cfg.vocab   # alter sub-chunk 1
    _, lg2, _, _ = O.generate(m, pr, 16, forced_tokens=forced)
    np.testing.assert_array_equal(lg[0, :4], lg2[0, :4])
    np.testing.assert_array_equal(lg[0, 8:], lg2[0, 8:])
    # inside sub-chunk 1 the first position is unchanged, the rest move
    np.testing.assert_array_equal(lg[0, 4], lg2[0, 4])
    assert np.abs(lg[0, 5:8] - lg2[0, 5:8]).max() > 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batch_independence(dtype):
    cfg = tiny(dtype)
    m = make(cfg, seed=13)
    pr = prompts(cfg, 3, 32, seed=13)
    t_all, l_all, _, _ = O.generate(m, pr, 32)
    for b in range(3):
        t1, l1, _, _ = O.generate(m, pr[b:b + 1], 32)
        np.testing.assert_array_equal(t1[0], t_all[b])
        np.testing.assert_allclose(l1[0], l_all[b], rtol=1e-12, atol=1e-13)


def test_greedy_picks_lowest_index_on_ties():
    assert int(np.argmax(np.array([0.5, 2.0, 1.0, 2.0]))) == 1


def test_bf16_contract_values_are_bf16():
    cfg = tiny("bf16")
    m = make(cfg, seed=14)
    _, _, st, recs = O.generate(m, prompts(cfg, 2, 32, seed=14), 16)
    for a in (st.top[0]["k"], st.top[0]["v"], st.h, recs[0]["A_hat"]):
        np.testing.assert_array_equal(O.round_bf16(a), a)


def test_prefill_needs_one_whole_chunk():
    cfg = tiny()
    m = make(cfg)
    with pytest.raises(ValueError):
        O.prefill(m, prompts(cfg, 1, 8))
    st = O.prefill(m, prompts(cfg, 1, 24))         # one whole chunk + an 8-token tail
    assert st.top_len == 1 and st.tail.shape == (1, 8)


def test_consistency_is_the_cosine_distance():
    from scipy.spatial.distance import cosine
    rng = np.random.default_rng(12)
    a = rng.standard_normal((3, 4, 64))
    e = rng.standard_normal((3, 4, 64))
    d = O.consistency(a, e)
    ref = np.array([[cosine(a[i, k], e[i, k]) for k in range(4)] for i in range(3)])
    assert np.allclose(d, ref, rtol=0, atol=1e-12)
    assert np.allclose(O.consistency(a, a), 0, atol=1e-12)           # identical
    assert np.allclose(O.consistency(a, -a), 2, atol=1e-12)          # opposite
    assert np.allclose(O.consistency(a, 3.5 * a), 0, atol=1e-12)     # scale free
    x = np.zeros((1, 1, 8)); y = np.zeros((1, 1, 8))
    x[..., 0] = 1; y[..., 1] = 2
    assert O.consistency(x, y)[0, 0] == 1.0                          # orthogonal


def test_consistency_in_hiergen_decoding():
    # HierGen computes both A-hat_i and A_i every chunk; the distance is a
    # proper cosine distance of them, and it is not identically zero (the
    # decoder's reconstruction is not the encoder's summary)
    wl = pi.get(1)
    m = O.Model(wl.cfg, pi.gen_weights(wl.cfg, wl.seed))
    st = O.prefill(m, pi.gen_prompts(wl.cfg, 2, wl.prompt, wl.seed), "hiergen")
    o = O.decode_chunk(m, st, "hiergen")
    d = O.consistency(o["A_hat"], o["A"])
    assert d.shape == (2, wl.cfg.C2)
    assert (d >= 0).all() and (d <= 2).all() and d.max() > 1e-3


# ---------------- ragged prompts (P mod S != 0) ----------------
@pytest.mark.parametrize("P,N", [(21, 27), (31, 17), (17, 47)])
def test_ragged_prompt_hiergen_equals_teacher_forced_full(P, N):
    # the tail tokens open the next chunk as given tokens: HierGen's
    # incremental logits at the new positions equal the cache-free forward
    # over the whole sequence (which sees the chunks in full)
    cfg = tiny()
    m = make(cfg, seed=15)
    pr = prompts(cfg, 2, P, seed=15)
    toks, lg, st, recs = O.generate(m, pr, N, mode="hiergen")
    assert toks.shape == (2, N) and lg.shape == (2, N, cfg.vocab)
    seq = np.concatenate([pr, toks], 1)
    full = O.hier_full_logits(m, seq, P // 16)        # positions (P // 16) * 16 onwards
    r = P % 16
    np.testing.assert_allclose(lg, full[:, r:], rtol=1e-10, atol=1e-12)
    # the first chunk reports the tail as its leading tokens
    assert np.array_equal(recs[0]["tokens"][:, :r], pr[:, P - r:])
    assert st.top_len == (P + N) // 16


def test_ragged_prompt_recgen_top_stream_ignores_the_tail():
    # RecGen's top stream reads no token, so a ragged prompt gives the top
    # stream of its whole-chunk part, bit for bit; the tokens differ
    cfg = tiny()
    m = make(cfg, seed=16)
    pr = prompts(cfg, 2, 16 * 3 + 5, seed=16)
    _, _, st_r, recs_r = O.generate(m, pr, 16 * 2 - 5, mode="recgen")
    _, _, st_w, recs_w = O.generate(m, pr[:, :48], 32, mode="recgen")
    assert np.array_equal(st_r.h, st_w.h)
    for a, b in zip(st_r.top, st_w.top):
        assert np.array_equal(a["k"], b["k"]) and np.array_equal(a["v"], b["v"])
    assert not np.array_equal(recs_r[0]["tokens"], recs_w[0]["tokens"])


def test_ragged_prompt_limits():
    cfg = tiny()
    m = make(cfg, seed=17)
    with pytest.raises(ValueError):
        O.prefill(m, prompts(cfg, 1, 15, seed=17))          # shorter than a chunk
    with pytest.raises(ValueError):
        O.generate(m, prompts(cfg, 1, 20, seed=17), 16)     # does not end on a chunk boundary
