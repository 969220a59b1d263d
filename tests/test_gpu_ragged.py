"""Ragged prompts (prompt length not a multiple of S = C1*C2) on the GPU
against the oracle: prefill encodes the whole chunks; the tail opens the
next chunk as given tokens.  Same bar as tests/parity.py."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import photon_inputs as pi  # noqa: E402
from parity import check_against_oracle, check_sampled, gpu_generate, oracle_reference, small_cfg  # noqa: E402


@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
@pytest.mark.parametrize("P,N", [(53, 43), (17, 15), (31, 33)])
def test_tiny_f32_ragged(mode, P, N):
    cfg = pi.CONFIGS["tiny"]
    W, pr = pi.gen_weights(cfg, 3), pi.gen_prompts(cfg, 2, P, 3)
    model, toks, lg = gpu_generate(cfg, W, pr, N, mode)
    assert toks.shape == (2, N)
    r = check_against_oracle(cfg, W, pr, toks, lg, mode)
    print(f"[ragged] tiny-f32 {mode} P={P}: max_err={r['max_err']:.3g}", flush=True)


@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
def test_small_bf16_ragged(mode):
    cfg = small_cfg()
    W, pr = pi.gen_weights(cfg, 11), pi.gen_prompts(cfg, 3, 37, 11)
    model, toks, lg = gpu_generate(cfg, W, pr, 43, mode)
    r = check_against_oracle(cfg, W, pr, toks, lg, mode)
    print(f"[ragged] small-bf16 {mode}: max_err={r['max_err']:.3g} near_ties={r['near_ties']}/{r['tokens']}",
          flush=True)


def test_tiny_f32_ragged_sampled():
    cfg = pi.CONFIGS["tiny"]
    W, pr = pi.gen_weights(cfg, 4), pi.gen_prompts(cfg, 2, 45, 4)
    sp = dict(temperature=0.9, top_k=7, seed=99)
    model, toks, lg, lp = gpu_generate(cfg, W, pr, 35, sampling=sp)
    ot, ol, nl, _ = oracle_reference(cfg, W, pr, toks, sampling=sp)
    r = check_sampled(cfg, toks, lg, lp, ot, ol, nl, sp, 45)
    assert r["near_ties"] == 0


def test_ragged_tail_is_given_and_replays_after_a_rewind():
    from hierarchical_autoregressive_lm_amd.photon import Photon
    cfg = small_cfg()
    W, pr = pi.gen_weights(cfg, 12), pi.gen_prompts(cfg, 4, 40, 12)   # 2 chunks + 8 tail tokens
    m = Photon(cfg, W)
    m.prefill(torch.from_numpy(pr).cuda(), 96)
    assert m.position() == (2, 40)
    snaps = [m.state_snapshot()]
    a = [torch.empty((4, cfg.S), dtype=torch.int32, device="cuda") for _ in range(3)]
    for t in a:
        m.decode_chunk(t)                  # the first directly, the rest from the graph
        snaps.append(m.state_snapshot())
    assert m.position() == (5, 80)
    torch.cuda.synchronize()
    assert np.array_equal(a[0][:, :8].cpu().numpy(), pr[:, 32:40])
    m.state_restore(snaps[0], 40)          # back to the ragged prompt end
    b = [torch.empty_like(t) for t in a]
    for t in b:
        m.decode_chunk(t)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    m.state_restore(snaps[1], 48)          # a chunk boundary
    c = torch.empty_like(a[0])
    m.decode_chunk(c)
    assert torch.equal(c, a[1])
