"""GPU parity for hierarchies deeper than two levels: the HIP path (through
the C ABI) against the CPU oracle, same rules as tests/parity.py.

Shapes: tiny fp32 models with unequal chunk sizes (a swapped level or a
transposed group index changes the result), bf16 models at d = 256 / 384.
HierGen runs S/span(l) queries per sequence in each encoder step, which the
global attention takes for 1, 2 or 4: its cases use (4, 2, 2) and
(2, 2, 2, 1); RecGen also takes (2, 3, 2) and (2, 2, 3, 2).
"""
import numpy as np
import pytest

import photon_inputs as pi
from oracle import photon_oracle as O
from parity import check_against_oracle, check_sampled, gpu_generate, oracle_reference, small_cfg

pytestmark = pytest.mark.gpu

TINY = pi.CONFIGS["tiny"]


def tiny_levels(chunk, **kw):
    k = len(chunk) - 2
    return TINY.with_(chunk=chunk, n_enc_hi=kw.pop("n_enc_hi", (1,) * k), n_dec_hi=kw.pop("n_dec_hi", (1,) * k), **kw)


def _report(name, r):
    print(f"[levels] {name}: max_err={r['max_err']:.3g} noise_max={r['noise_max']:.3g} "
          f"near_ties={r['near_ties']}/{r['tokens']}", flush=True)


CASES = [
    ((2, 3, 2), "recgen", dict(n_dec_hi=(2,))),
    ((4, 2, 2), "recgen", {}),
    ((4, 2, 2), "hiergen", dict(n_enc1=2)),
    ((2, 2, 3, 2), "recgen", {}),
    ((2, 2, 2, 1), "hiergen", {}),
    ((2, 2, 2, 1), "recgen", {}),
]


@pytest.mark.parametrize("chunk,mode,kw", CASES, ids=[f"{'x'.join(map(str, c))}-{m}" for c, m, _ in CASES])
def test_tiny_f32_exact_ids(chunk, mode, kw):
    cfg = tiny_levels(chunk, **kw)
    S = cfg.S
    W, pr = pi.gen_weights(cfg, 31), pi.gen_prompts(cfg, 2, 3 * S, 31)
    model, toks, lg = gpu_generate(cfg, W, pr, 4 * S, mode)
    r = check_against_oracle(cfg, W, pr, toks, lg, mode)
    _report(f"tiny-f32 {chunk} {mode}", r)
    assert r["near_ties"] == 0


@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
def test_tiny_f32_ragged_prompt(mode):
    cfg = tiny_levels((4, 2, 2))
    P = 16 * 2 + 11
    W, pr = pi.gen_weights(cfg, 32), pi.gen_prompts(cfg, 3, P, 32)
    model, toks, lg = gpu_generate(cfg, W, pr, 16 * 3 - 11, mode)
    r = check_against_oracle(cfg, W, pr, toks, lg, mode)
    _report(f"tiny-f32 ragged {mode}", r)


@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
def test_small_bf16_three_levels(mode):
    cfg = small_cfg(chunk=(4, 2, 2), n_enc_hi=(1,), n_dec_hi=(2,))
    W, pr = pi.gen_weights(cfg, 33), pi.gen_prompts(cfg, 3, 64, 33)
    model, toks, lg = gpu_generate(cfg, W, pr, 48, mode)
    r = check_against_oracle(cfg, W, pr, toks, lg, mode)
    _report(f"small-bf16 4x2x2 {mode}", r)


def test_bf16_hd96_four_levels_recgen():
    cfg = small_cfg(d_model=384, n_heads=4, chunk=(2, 3, 2, 2), vocab=2000, n_enc_hi=(1, 1), n_dec_hi=(1, 2))
    W, pr = pi.gen_weights(cfg, 34), pi.gen_prompts(cfg, 5, 48, 34)
    model, toks, lg = gpu_generate(cfg, W, pr, 48)
    r = check_against_oracle(cfg, W, pr, toks, lg)
    _report("bf16 hd96 2x3x2x2 recgen", r)


def test_zero_top_chunker_recgen_equals_hiergen_three_levels():
    cfg = small_cfg(chunk=(4, 2, 2), n_enc_hi=(1,), n_dec_hi=(1,))
    W, pr = pi.gen_weights(cfg, 35, zero=("W_ch3",)), pi.gen_prompts(cfg, 2, 32, 35)
    m1, t1, l1 = gpu_generate(cfg, W, pr, 32, "recgen")
    kv1 = m1.top_kv().float().cpu().numpy()
    m2, t2, l2 = gpu_generate(cfg, W, pr, 32, "hiergen")
    kv2 = m2.top_kv().float().cpu().numpy()
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(kv1, kv2)


def test_sampled_decode_three_levels():
    cfg = small_cfg(chunk=(2, 3, 2), n_enc_hi=(1,), n_dec_hi=(1,))
    W, pr = pi.gen_weights(cfg, 36), pi.gen_prompts(cfg, 3, 24, 36)
    sp = dict(temperature=0.9, top_k=20, seed=77)
    model, toks, lg, lp = gpu_generate(cfg, W, pr, 36, sampling=sp)
    ot, ol, nl, _ = oracle_reference(cfg, W, pr, toks, sampling=sp)
    r = check_sampled(cfg, toks, lg, lp, ot, ol, nl, sp, 24)
    print(f"[levels] sampled 2x3x2: max_err={r['max_err']:.3g} near_ties={r['near_ties']}/{r['tokens']}", flush=True)


def test_consistency_at_the_level_under_the_top():
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon
    cfg = tiny_levels((4, 2, 2))
    W, pr = pi.gen_weights(cfg, 37), pi.gen_prompts(cfg, 2, 32, 37)
    m = Photon(cfg, W)
    m.prefill(torch.from_numpy(pr).cuda(), 32 + 16, mode="hiergen")
    toks = torch.empty((2, cfg.S), dtype=torch.int32, device="cuda")
    m.decode_chunk(toks)
    dist, ah, a = m.consistency(copies=True)
    torch.cuda.synchronize()
    om = O.Model(cfg, W)
    st = O.prefill(om, pr, "hiergen")
    o = O.decode_chunk(om, st, "hiergen")
    assert dist.shape == (2, cfg.chunk[-1])
    np.testing.assert_allclose(ah.cpu().numpy(), o["A_hat"], rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(a.cpu().numpy(), o["A"], rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(dist.cpu().numpy(), O.consistency(o["A_hat"], o["A"]), atol=1e-5)


def test_graph_direct_and_rewind_three_levels():
    # RecGen's top branch prepares the next chunk's decoders; after a rewind
    # (or with direct launches) the first chunk prepares them itself: every
    # order gives the same tokens and the same top K/V, bit for bit
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon
    cfg = small_cfg(chunk=(2, 3, 2), n_enc_hi=(1,), n_dec_hi=(1,))
    W, pr = pi.gen_weights(cfg, 38), pi.gen_prompts(cfg, 3, 24, 38)
    m = Photon(cfg, W)
    prompt = torch.from_numpy(pr).cuda()
    tg, _ = m.generate(prompt, 48)                        # graph replay
    kv_g = m.top_kv().clone()
    m.use_graphs(False)
    td, _ = m.generate(prompt, 48)                        # direct launches
    assert torch.equal(tg, td) and torch.equal(kv_g, m.top_kv())
    m.use_graphs(True)
    m.prefill(prompt, 24 + 48)
    snap = m.state_snapshot()
    a = torch.empty((3, cfg.S), dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    m.decode_chunk(a)
    m.decode_chunk(b)
    m.state_restore(snap, 24)                             # back to the prompt end
    c = torch.empty_like(a)
    m.decode_chunk(c)
    torch.cuda.synchronize()
    assert torch.equal(a, c) and torch.equal(a, tg[:, :cfg.S]) and torch.equal(b, tg[:, cfg.S:2 * cfg.S])
