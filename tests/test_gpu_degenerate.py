"""Degenerate hierarchy shapes on the GPU against the oracle (tiny fp32
models, exact ids): chunks of one state at either level (the chunker and
converter become square d x d maps), one-chunk prompts and generations, a
batch of one, and a three-level model whose middle level has chunks of one.
Also a head whose logits are all NaN: the greedy ids stay inside the
vocabulary (there is no ordered maximum; the kernel takes id 0).
"""
import numpy as np
import pytest

import photon_inputs as pi
from parity import check_against_oracle, gpu_generate, small_cfg

pytestmark = pytest.mark.gpu

TINY = pi.CONFIGS["tiny"]

CASES = [
    # chunk, batch, prompt chunks, new chunks, mode
    ((1, 4), 2, 3, 4, "recgen"),
    ((4, 1), 2, 3, 4, "recgen"),
    ((1, 1), 2, 5, 6, "recgen"),
    ((1, 4), 2, 3, 4, "hiergen"),
    ((4, 1), 2, 3, 4, "hiergen"),
    ((1, 1), 1, 4, 4, "hiergen"),
    ((4, 4), 1, 1, 1, "recgen"),        # one-chunk prompt and generation, batch of one
    ((4, 4), 1, 1, 1, "hiergen"),
    ((2, 1, 2), 2, 2, 3, "recgen"),     # a middle level with chunks of one
    ((2, 1, 2), 2, 2, 3, "hiergen"),
]


@pytest.mark.parametrize("chunk,B,pc,nc,mode", CASES,
                         ids=[f"{'x'.join(map(str, c))}-B{b}-{m}" for c, b, _, _, m in CASES])
def test_degenerate_shapes_exact_ids(chunk, B, pc, nc, mode):
    k = len(chunk) - 2
    cfg = TINY.with_(chunk=chunk, n_enc_hi=(1,) * k, n_dec_hi=(1,) * k)
    S = cfg.S
    W, pr = pi.gen_weights(cfg, 41), pi.gen_prompts(cfg, B, pc * S, 41)
    model, toks, lg = gpu_generate(cfg, W, pr, nc * S, mode)
    r = check_against_oracle(cfg, W, pr, toks, lg, mode)
    print(f"[degenerate] {chunk} B{B} {mode}: max_err={r['max_err']:.3g}", flush=True)
    assert r["near_ties"] == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flat", [False, True], ids=["photon", "flat"])
def test_nan_head_gives_in_range_ids(dtype, flat):
    # every logit NaN: no id is an ordered maximum, so the first-maximum
    # reduction keeps its initial value; the kernel maps it to id 0, whose
    # embedding row the next step reads
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon, Vanilla
    cfg = TINY if dtype == "f32" else small_cfg()
    S = cfg.S
    mcfg = pi.vanilla_of(cfg) if flat else cfg
    W = pi.gen_weights(mcfg, 43)
    W["W_out"] = np.full_like(W["W_out"], np.nan)
    pr = torch.from_numpy(pi.gen_prompts(cfg, 2, 2 * S, 43)).cuda()
    model = Vanilla(mcfg, W, S) if flat else Photon(cfg, W)
    toks, lg = model.generate(pr, 2 * S, logits=True)
    torch.cuda.synchronize()
    t = toks.cpu().numpy()
    assert np.isnan(lg.cpu().numpy()).all()
    assert (t == 0).all(), f"ids {np.unique(t)}"
