"""CPU pins of the oracle's sampling decode and multi-query aggregation.

Pinned against what does not depend on the oracle: the Philox-4x32-10
known-answer vectors published with the generator (tests/golden), the
exactness and uniformity of the float32 uniform grid, the distribution that
the Gumbel-max rule must produce (softmax of logit / temperature over the
kept ids: a chi-square test at a fixed seed), scipy's log-softmax, the
limits that reduce sampling to greedy decoding, and aggregation answers
worked out by hand.  The sampled decode loop is pinned by its reduction to
greedy decoding (top_k = 1) and by RecGen's top stream not depending on the
tokens.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats
from scipy.special import log_softmax, softmax

import photon_inputs as pi
from oracle import photon_oracle as O
from oracle import photon_sampling as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    kat = json.load(open(os.path.join(GOLD, "philox_kat.json")))
    for v in kat["vectors"]:
        ctr = np.array([int(x, 16) for x in v["counter"]], dtype=np.uint64)
        key = [int(x, 16) for x in v["key"]]
        out = S.philox4x32_10(ctr, key)
        assert [f"{int(x):08x}" for x in out] == v["out"]


def test_philox_is_a_function_of_each_counter_word_and_the_key():
    base = np.zeros(4, dtype=np.uint64)
    ref = S.philox4x32_10(base, (1, 2))
    for w in range(4):
        c = base.copy()
        c[w] = 1
        assert not np.array_equal(S.philox4x32_10(c, (1, 2)), ref)
    assert not np.array_equal(S.philox4x32_10(base, (1, 3)), ref)
    assert not np.array_equal(S.philox4x32_10(base, (2, 2)), ref)
    # 2^16 consecutive counters: no repeated output block
    ctr = np.zeros((1 << 16, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(1 << 16)
    out = S.philox4x32_10(ctr, (7, 9)).astype(np.uint64)
    packed = (out[:, 0] << np.uint64(32)) | out[:, 1]
    assert len(np.unique(packed)) == 1 << 16


def test_uniforms_are_exact_float32_and_uniform():
    ids = np.arange(200000)
    u = S.uniforms(0x1234_5678_9ABC_DEF0, 3, 77, ids)
    grid = u * (1 << 23) - 0.5
    assert np.array_equal(grid, np.round(grid)) and grid.min() >= 0 and grid.max() < (1 << 23)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)
    assert 0.0 < u.min() and u.max() < 1.0
    counts = np.histogram(u, bins=64, range=(0, 1))[0]
    assert stats.chisquare(counts).pvalue > 1e-4
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / len(u))
    # the seed's two words, the sequence and the position each change the stream
    for args in [(0x1234_5678_9ABC_DEF1, 3, 77), (0x1234_5679_9ABC_DEF0, 3, 77), (0x1234_5678_9ABC_DEF0, 4, 77),
                 (0x1234_5678_9ABC_DEF0, 3, 78)]:
        assert not np.array_equal(S.uniforms(*args, ids[:64]), u[:64])


def test_uniform_word_layout():
    # id v takes word v % 4 of the block v // 4 (position in counter word 1,
    # sequence in word 2)
    seed, seq, pos = 99, 5, 1234
    words = S.philox4x32_10(np.array([2, pos, seq, 0], dtype=np.uint64), S.seed_key(seed))
    u = S.uniforms(seed, seq, pos, np.arange(8, 12))
    assert np.array_equal(u, ((words >> 9).astype(np.float64) + 0.5) / 2 ** 23)


def draw(logits, temperature, top_k, n, seed=2024):
    return np.array([S.sample(logits, temperature, top_k, seed, 0, p) for p in range(n)])


@pytest.mark.parametrize("temperature,top_k", [(1.0, 0), (0.7, 0), (1.6, 3)])
def test_gumbel_max_draws_follow_the_tempered_softmax(temperature, top_k):
    lg = np.array([0.3, -1.0, 1.2, 0.0, 0.9, -0.4])
    n = 30000
    got = np.bincount(draw(lg, temperature, top_k, n), minlength=len(lg))
    keep = S.kept_ids(lg, top_k)
    p = np.zeros(len(lg))
    p[keep] = softmax(lg[keep] / temperature)
    assert (got[p == 0] == 0).all()
    assert stats.chisquare(got[p > 0], n * p[p > 0]).pvalue > 1e-4


def test_top_k_keeps_ties_at_the_cut():
    lg = np.array([1.0, 3.0, 3.0, 2.0, -5.0])
    assert list(S.kept_ids(lg, 1)) == [1, 2]
    assert list(S.kept_ids(lg, 2)) == [1, 2]
    assert list(S.kept_ids(lg, 3)) == [1, 2, 3]
    assert list(S.kept_ids(lg, 0)) == [0, 1, 2, 3, 4]
    assert list(S.kept_ids(lg, 5)) == [0, 1, 2, 3, 4]
    assert list(S.kept_ids(lg, 9)) == [0, 1, 2, 3, 4]
    # only kept ids are ever drawn, and both tied ones are
    got = set(draw(lg, 1.0, 1, 400).tolist())
    assert got == {1, 2}


def test_limits_reduce_to_greedy():
    rng = np.random.default_rng(3)
    for r in range(50):
        lg = rng.standard_normal(300)
        am = int(np.argmax(lg))
        assert S.sample(lg, 1.0, 1, 11, r, r) == am          # top-1, no ties
        assert S.sample(lg, 1e-9, 0, 11, r, r) == am         # temperature -> 0


def test_loglik_is_log_softmax():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((3, 7, 50)) * 3
    ids = rng.integers(0, 50, (3, 7))
    ref = np.take_along_axis(log_softmax(lg, axis=-1), ids[..., None], -1)[..., 0]
    assert np.allclose(S.loglik(lg, ids), ref, rtol=0, atol=1e-12)
    every = S.loglik(np.broadcast_to(lg[0, 0], (50, 50)), np.arange(50))
    assert np.exp(every).sum() == pytest.approx(1.0, abs=1e-12)


def test_aggregate_worked_examples():
    toks = np.array([[1, 2, 3], [1, 2, 3], [4, 5, 6],      # group 0
                     [7, 7, 7], [8, 8, 8], [9, 9, 9],      # group 1: all differ
                     [1, 1, 5], [1, 1, 6]])                # group 2 (short): differ in the last token
    lp = np.array([[-1, -1, -1], [-2, -2, -2], [-0.5, -0.5, -0.5],
                   [-3, -3, -3], [-1, -1, -1], [-1, -1, -1],
                   [-1, -1, -1], [-1, -1, -2]], dtype=float)
    best, major, votes, scores = S.aggregate(toks, lp, 3)
    assert list(scores) == [-3, -6, -1.5, -9, -3, -3, -3, -4]
    assert list(best) == [2, 1, 0]             # group 1: members 1 and 2 tie, lower index
    assert list(major) == [0, 1, 0]            # group 0: the shared answer's higher score (member 0)
    assert list(votes) == [2, 1, 1]
    # answer = the first two tokens: group 2's members now agree
    best, major, votes, _ = S.aggregate(toks, lp, 3, span=(0, 2))
    assert list(major) == [0, 1, 0] and list(votes) == [2, 1, 2]
    # answer = the last token only: group 0 unchanged, group 2 splits again
    _, major, votes, _ = S.aggregate(toks, lp, 3, span=(2, 3))
    assert list(votes) == [2, 1, 1]


def tiny():
    return pi.get(1)


def test_sampled_decode_with_top_1_is_greedy():
    wl = tiny()
    m = O.Model(wl.cfg, pi.gen_weights(wl.cfg, wl.seed))
    pr = pi.gen_prompts(wl.cfg, 2, wl.prompt, wl.seed)
    g, glg, gst, _ = O.generate(m, pr, 32)
    s, slg, sst, _ = O.generate(m, pr, 32, sampling=dict(temperature=0.8, top_k=1, seed=5))
    assert np.array_equal(g, s) and np.array_equal(glg, slg)


def test_sampled_decode_is_seeded_and_leaves_the_top_stream_alone():
    wl = tiny()
    m = O.Model(wl.cfg, pi.gen_weights(wl.cfg, wl.seed))
    pr = pi.gen_prompts(wl.cfg, 2, wl.prompt, wl.seed)
    sp = dict(temperature=1.0, top_k=0, seed=77)
    a, alg, ast, arecs = O.generate(m, pr, 32, sampling=sp)
    b, blg, bst, _ = O.generate(m, pr, 32, sampling=sp)
    assert np.array_equal(a, b)
    c, clg, cst, crecs = O.generate(m, pr, 32, sampling=dict(sp, seed=78))
    assert not np.array_equal(a, c)
    g, _, gst, grecs = O.generate(m, pr, 32)
    assert not np.array_equal(a, g)
    # RecGen's top stream does not read the tokens
    assert np.array_equal(ast.h, gst.h) and np.array_equal(cst.h, gst.h)
    # each reported token is the sampler's choice on the logits it saw, at
    # its absolute position (prompt end + index within the generation)
    P = wl.prompt
    for r in range(2):
        for t in range(32):
            assert a[r, t] == S.sample(alg[r, t], 1.0, 0, 77, r, P + t)
