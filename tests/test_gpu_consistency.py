"""The Eq. 1 consistency diagnostic (photon_consistency) on the GPU.

Two checks per decoded HierGen chunk: the kernel alone -- the oracle's
cosine distance on the GPU's own A-hat_i and A_i (copied out by the same
call) agrees to float32 accuracy; and end to end -- the distance on the
oracle's own A-hat_i and A_i (teacher-forced with the GPU's tokens) agrees
to the model tolerance: 1e-4 for float32 models, for bf16 models
max(2e-2, 1.5 x the oracle's own float32-vs-float64 spread of the same
distance), the rounding contract's noise as for the logits.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import photon_inputs as pi  # noqa: E402
from oracle import photon_oracle as O  # noqa: E402
from parity import small_cfg  # noqa: E402


def run(cfg, B, P, N, seed):
    from hierarchical_autoregressive_lm_amd.photon import Photon
    W, pr = pi.gen_weights(cfg, seed), pi.gen_prompts(cfg, B, P, seed)
    m = Photon(cfg, W)
    m.prefill(torch.from_numpy(pr).cuda(), P + N, "hiergen")
    toks, dists, ahs, aas = [], [], [], []
    t = torch.empty((B, cfg.S), dtype=torch.int32, device="cuda")
    for _ in range(N // cfg.S):
        m.decode_chunk(t)
        d, ah, a = m.consistency(copies=True)
        torch.cuda.synchronize()
        toks.append(t.cpu().numpy().copy())
        dists.append(d.cpu().numpy())
        ahs.append(ah.float().cpu().numpy())
        aas.append(a.float().cpu().numpy())
    return W, pr, np.concatenate(toks, 1), dists, ahs, aas


def oracle_dists(cfg, W, pr, toks, compute="f64"):
    m = O.Model(cfg, W, compute=compute)
    _, _, _, recs = O.generate(m, pr, toks.shape[1], mode="hiergen", forced_tokens=toks)
    return [O.consistency(r["A_hat"], r["A"]) for r in recs]


@pytest.mark.parametrize("which", ["tiny-f32", "small-bf16"])
def test_consistency_matches_oracle(which):
    if which == "tiny-f32":
        wl = pi.get(1)
        cfg, B, P, N, seed = wl.cfg, 2, wl.prompt, wl.new_tokens, wl.seed
    else:
        cfg, B, P, N, seed = small_cfg(), 3, 64, 48, 4
    W, pr, toks, dists, ahs, aas = run(cfg, B, P, N, seed)
    ref = oracle_dists(cfg, W, pr, toks)
    if cfg.dtype == "f32":
        tol = 1e-4
    else:
        noise = max(np.abs(a - b).max() for a, b in zip(oracle_dists(cfg, W, pr, toks, "f32"), ref))
        tol = max(2e-2, 1.5 * noise)
    for c, (d, ah, a, r) in enumerate(zip(dists, ahs, aas, ref)):
        assert d.shape == (B, cfg.C2) and np.isfinite(d).all()
        own = O.consistency(ah, a)
        assert np.abs(d - own).max() <= 1e-5, f"chunk {c}: kernel vs its own inputs {np.abs(d - own).max():.3g}"
        err = np.abs(d - r).max()
        assert err <= tol, f"chunk {c}: {err:.3g} > {tol:.3g}"
    print(f"[consistency] {which}: mean distance {np.mean(dists):.4f}, max err vs oracle "
          f"{max(np.abs(d - r).max() for d, r in zip(dists, ref)):.3g} (tol {tol:.3g})", flush=True)


def test_consistency_needs_a_hiergen_chunk():
    from hierarchical_autoregressive_lm_amd.photon import Photon, PhotonError, ESTATE
    cfg = small_cfg()
    W, pr = pi.gen_weights(cfg, 5), pi.gen_prompts(cfg, 2, 32, 5)
    m = Photon(cfg, W)
    m.prefill(torch.from_numpy(pr).cuda(), 64, "recgen")
    t = torch.empty((2, cfg.S), dtype=torch.int32, device="cuda")
    m.decode_chunk(t)
    with pytest.raises(PhotonError) as e:
        m.consistency()
    assert e.value.status == ESTATE
    m.prefill(torch.from_numpy(pr).cuda(), 64, "hiergen")
    with pytest.raises(PhotonError):
        m.consistency()           # nothing decoded yet
    m.decode_chunk(t)
    assert m.consistency().shape == (2, cfg.C2)
