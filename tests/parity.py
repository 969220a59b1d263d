"""Shared helpers of the GPU parity tests: run the HIP path through the C
ABI, run the oracle teacher-forced with the GPU's tokens, compare.

Tolerances (logits): fp32 models |dlogit| <= 1e-4 * max(1, max|oracle row|)
and identical greedy ids.

bf16 models: the rounding contract (bf16 operands and K/V, fp32 accumulate)
has an intrinsic noise: two valid implementations that differ only in
accumulation precision flip some bf16 roundings by one ulp, and RecGen's top
stream, a recurrence over chunks, carries those flips forward.  The noise is
measured by running the oracle's own code in float32 beside the float64
reference.  The bar is |dlogit| <= max(3e-2, 1.5 x that noise), both for the
largest and (with 1.5x) the mean deviation.  Greedy ids must be identical,
except where the reference's margin between its argmax and the GPU's id is
within twice the tolerance (near ties: both ids are correct under rounding
differences); those positions are counted and reported.
"""
import numpy as np

import photon_inputs as pi
from oracle import photon_oracle as O

TOL_F32 = 1e-4
TOL_BF16 = 3e-2


def gpu_generate(cfg, W, prompt, N, mode="recgen", logits=True, rows=None):
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon
    model = Photon(cfg, W)
    toks, lg = model.generate(torch.from_numpy(prompt).cuda(), N, mode=mode, logits=logits)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else list(rows)
    toks_np = toks.cpu().numpy()[sel]
    lg_np = lg[sel].cpu().numpy() if logits else None
    return model, toks_np, lg_np


def oracle_reference(cfg, W, prompt, toks, mode="recgen", log=None):
    """The oracle teacher-forced with ``toks``: its ids and float64 logits,
    and for bf16 models the same run in float32 (the noise probe)."""
    m = O.Model(cfg, W)
    N = toks.shape[1]
    ot, ol, st, _ = O.generate(m, prompt, N, mode=mode, forced_tokens=toks, log=log)
    nl = None
    if cfg.dtype != "f32":
        _, nl, _, _ = O.generate(O.Model(cfg, W, compute="f32"), prompt, N, mode=mode,
                                 forced_tokens=toks, log=log)
    return ot, ol, nl, st


def compare(cfg, toks, lg, ot, ol, nl):
    """Apply the bar of the module docstring; returns a small report dict."""
    if cfg.dtype == "f32":
        scale = np.maximum(1.0, np.abs(ol).max(-1))
        err = (np.abs(lg - ol).max(-1) / scale).max()
        assert err <= TOL_F32, f"fp32 logits differ: {err:.3g}"
        assert (ot == toks).all(), "fp32 greedy ids differ"
        ties = 0
        noise = (0.0, 0.0)
    else:
        dev = np.abs(lg - ol)
        nz = np.abs(nl.astype(np.float64) - ol)
        noise = (float(nz.max()), float(nz.mean()))
        tol = max(TOL_BF16, 1.5 * noise[0])
        err = dev.max()
        assert err <= tol, f"bf16 logits differ: {err:.3g} (tol {tol:.3g}, noise {noise[0]:.3g})"
        assert dev.mean() <= 1.5 * noise[1] + 1e-4, \
            f"bf16 mean deviation {dev.mean():.3g} vs noise {noise[1]:.3g}"
        diff = ot != toks
        gap = np.take_along_axis(ol, ot[..., None], -1)[..., 0] - \
            np.take_along_axis(ol, toks[..., None].astype(np.int64), -1)[..., 0]
        assert (gap[diff] <= 2 * tol).all(), \
            f"ids differ beyond a near-tie: gaps {gap[diff].max():.3g}"
        ties = int(diff.sum())
    return {"max_err": float(err), "near_ties": ties, "tokens": int(toks.size),
            "noise_max": noise[0], "noise_mean": noise[1], "mean_err": float(np.abs(lg - ol).mean())}


def check_against_oracle(cfg, W, prompt, toks, lg, mode="recgen", log=None):
    """prompt/toks/lg for the same rows; returns a small report dict.  ``log``
    passes the oracle's own progress lines through (long runs)."""
    ot, ol, nl, st = oracle_reference(cfg, W, prompt, toks, mode, log)
    r = compare(cfg, toks, lg, ot, ol, nl)
    r["state"] = st
    return r


def small_cfg(**kw):
    base = dict(d_model=256, n_heads=4, chunk=(4, 4), vocab=4096, n_top=2,
                n_enc1=1, n_dec1=2, n_dec0=2, dtype="bf16")
    base.update(kw)
    return pi.PhotonConfig(**base)
