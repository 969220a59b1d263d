"""The decode kernels give the same results whatever runs beside them.

RecGen's chunk runs its token branch and its top branch on two streams at
once, and a caller may run several contexts side by side; kernels then share
CUs with other kernels, which changes their timing.  Every kernel must stay
bit-exact under that.  (A ring-buffered GEMM once let a quickly landing
refill overwrite an LDS slot before a wave slowed down by a neighbour had
read it: tokens changed from run to run whenever the branches overlapped.)
"""
import numpy as np
import pytest

import photon_inputs as pi

pytestmark = pytest.mark.gpu

CHUNKS = 8


def _model(torch, Photon, wl, W):
    m = Photon(wl.cfg, W)
    m.prefill(torch.from_numpy(pi.gen_prompts(wl.cfg, wl.batch, wl.prompt, wl.seed)).cuda(), wl.max_tokens)
    m.release_prefill_weights()
    return m, m.state_snapshot()


def _decode(torch, m, snap, wl, graphs):
    m.use_graphs(graphs)
    m.state_restore(snap, wl.prompt)
    t = torch.empty((CHUNKS, wl.batch, wl.cfg.S), dtype=torch.int32, device="cuda")
    for c in range(CHUNKS):
        m.decode_chunk(t[c])
    return t


def test_branches_and_contexts_side_by_side_are_bit_exact():
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon
    wl = pi.get(2)          # photon-150m: short kernels, the branches overlap the most
    W = pi.gen_weights(wl.cfg, wl.seed)
    m0, s0 = _model(torch, Photon, wl, W)
    m1, s1 = _model(torch, Photon, wl, W)
    ref = _decode(torch, m0, s0, wl, graphs=False)       # direct launches, one stream: the order of record
    torch.cuda.synchronize()
    ref = ref.cpu().numpy()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for graphs in (True, False):
        for rep in range(3):
            outs = []
            for k, (m, s) in enumerate(((m0, s0), (m1, s1))):
                with torch.cuda.stream(streams[k]):
                    outs.append(_decode(torch, m, s, wl, graphs))
            torch.cuda.synchronize()
            for k in range(2):
                diff = int((outs[k].cpu().numpy() != ref).sum())
                assert diff == 0, f"graphs={graphs} rep {rep} context {k}: {diff} tokens differ"
        # and one context alone, both branches forked (graph replay)
        alone = _decode(torch, m0, s0, wl, graphs)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(alone.cpu().numpy(), ref)
