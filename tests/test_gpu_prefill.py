"""GPU parity of a prompt's caches: the prompt-sized QKV projections rotate q
and k and append K and V to the caches from their own epilogue (bf16, head
sizes 64, 96 and 128).  The caches and the kept top output after prefill are
compared with the oracle's prefill state [explainer, recursive generation:
prefill keeps the top-level K/V and the last top output; HierGen also keeps
the level-1 encoder's K/V]."""
import numpy as np
import pytest

import photon_inputs as pi
from oracle import photon_oracle as O
from parity import small_cfg

pytestmark = pytest.mark.gpu


def _prefill_both(cfg, B, P, N, seed, mode):
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon
    W, pr = pi.gen_weights(cfg, seed), pi.gen_prompts(cfg, B, P, seed)
    model = Photon(cfg, W)
    model.prefill(torch.from_numpy(pr).cuda(), P + N, mode)
    torch.cuda.synchronize()
    st = O.prefill(O.Model(cfg, W), pr, mode)
    return model, st


def _check_cache(gpu, ref, n, name):
    # gpu: [layers, 2, B, H, cap, hd]; ref: per layer {"k", "v"} [B, T, H, hd]
    for l, e in enumerate(ref):
        for i, kv in enumerate(("k", "v")):
            g = gpu[l, i][:, :, :n].transpose(0, 2, 1, 3)
            err = float(np.abs(g - e[kv]).max())
            print(f"[prefill] {name} layer {l} {kv}: max err {err:.3g} (max |ref| {np.abs(e[kv]).max():.3g})",
                  flush=True)
            np.testing.assert_allclose(g, e[kv], atol=3e-2)


@pytest.mark.parametrize("d, heads", [(384, 4), (384, 6), (512, 4)])
@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
def test_prompt_caches_match_oracle(d, heads, mode):
    # 3 sequences of 4000 prompt tokens at chunk 2 x 2: 6000 level-1 rows and
    # 3000 top rows, neither a multiple of the 256-row tile, and tiles that
    # straddle two sequences (2000 and 1000 rows per sequence); head sizes
    # 96 (two ring stages), 64 and 128
    cfg = small_cfg(d_model=d, n_heads=heads, chunk=(2, 2), vocab=2000, n_top=2)
    P, N = 4000, 16
    model, st = _prefill_both(cfg, 3, P, N, 31, mode)
    n = P // cfg.S
    assert model.position() == (n, P)
    _check_cache(model.top_kv().float().cpu().numpy(), st.top, n, f"d{d} H{heads} {mode} top")
    if mode == "hiergen":
        _check_cache(model.lower_kv().float().cpu().numpy(), st.lvl1, P // cfg.chunk[0], f"d{d} H{heads} level-1")
    h = model.h_state().float().cpu().numpy().reshape(st.h.shape)
    np.testing.assert_allclose(h, st.h, atol=3e-2)
