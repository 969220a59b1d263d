"""CPU pins of the oracle's flat (vanilla) Transformer baseline.

The baseline is the comparison model of the pages' decode-heavy table: one
causal stack over the tokens whose K/V cache holds every token.  It reuses
the oracle's pinned block (Model.stack); what is pinned here is the decode
loop: incremental decoding with the cache equals the cache-free causal
forward over the same tokens (every position, every step), the greedy rule,
the cache size growing with every token, and the matched shape.
"""
import numpy as np
import pytest

import photon_inputs as pi
from oracle import photon_oracle as O


def tiny_vanilla(dtype="f32", layers=2):
    return pi.VanillaConfig(d_model=64, n_heads=2, vocab=256, n_layers=layers, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_incremental_equals_full_recompute(dtype):
    v = tiny_vanilla(dtype)
    m = O.Model(v, pi.gen_weights(v, 3))
    pr = pi.gen_prompts(v, 3, 20, 3)
    toks, lg, st = O.vanilla_generate(m, pr, 9)
    full = O.vanilla_full_logits(m, np.concatenate([pr, toks], 1))
    # step j's logits are the full forward's at position P - 1 + j
    err = np.abs(full[:, pr.shape[1] - 1: pr.shape[1] - 1 + 9] - lg).max()
    # fp64 arithmetic in both; bf16 roundings sit at the same points, so only
    # summation order differs
    assert err < 1e-9, err
    assert st.n == 29 and all(e["k"].shape[1] == 29 for e in st.cache)


def test_greedy_is_the_first_argmax_and_forcing_replays():
    v = tiny_vanilla()
    m = O.Model(v, pi.gen_weights(v, 4))
    pr = pi.gen_prompts(v, 2, 12, 4)
    toks, lg, _ = O.vanilla_generate(m, pr, 6)
    assert (toks == np.argmax(lg, -1)).all()
    t2, lg2, _ = O.vanilla_generate(m, pr, 6, forced_tokens=toks)
    assert (t2 == toks).all() and np.array_equal(lg2, lg)
    # forcing other tokens changes the later logits but not the first step's;
    # the reported ids stay the argmax of the forced trajectory's logits
    other = (toks + 1) % v.vocab
    t3, lg3, _ = O.vanilla_generate(m, pr, 6, forced_tokens=other)
    assert np.array_equal(lg3[:, 0], lg[:, 0]) and not np.allclose(lg3[:, 1:], lg[:, 1:])
    assert (t3 == np.argmax(lg3, -1)).all()


def test_off_by_one_position_is_caught():
    # a planted mistake (decode step at the wrong rotary position) breaks the
    # incremental == full equality
    v = tiny_vanilla()
    m = O.Model(v, pi.gen_weights(v, 5))
    pr = pi.gen_prompts(v, 2, 10, 5)
    st = O.vanilla_prefill(m, pr)
    st.n += 1                                  # the mistake
    toks, lg = O.vanilla_decode(m, st, 4)
    full = O.vanilla_full_logits(m, np.concatenate([pr, toks], 1))
    assert np.abs(full[:, 9:13] - lg)[:, 1:].max() > 1e-6


def test_cache_grows_with_every_token_and_matches_photon_layers():
    for idx in (2, 3, 4, 5):
        wl = pi.get(idx)
        v = pi.vanilla_of(wl.cfg)
        assert v.n_layers == wl.cfg.n_top + wl.cfg.n_enc1 + wl.cfg.n_dec1 + wl.cfg.n_dec0
        assert (v.d_model, v.n_heads, v.vocab, v.dtype) == (wl.cfg.d_model, wl.cfg.n_heads, wl.cfg.vocab, wl.cfg.dtype)
        b1 = O.vanilla_kv_bytes(v, wl.batch, wl.max_tokens)
        assert b1 == v.n_layers * 2 * wl.batch * wl.max_tokens * v.d_model * 2
        assert O.vanilla_kv_bytes(v, wl.batch, 2 * wl.max_tokens) == 2 * b1
        # PHOTON's top K/V holds one state per S tokens, for n_top layers
        top = wl.cfg.n_top * 2 * wl.batch * (wl.max_tokens // wl.cfg.S) * wl.cfg.d_model * 2
        assert b1 / top == pytest.approx(v.n_layers / wl.cfg.n_top * wl.cfg.S)
