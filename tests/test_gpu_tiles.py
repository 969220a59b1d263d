"""Parity at the decode GEMM shapes of the benchmark workloads.

The tuned GEMM tiles are keyed by the exact (rows, features, k) shape of a
launch, so the small test models never reach them.  These models keep the
workloads' width, heads, chunk shape, vocabulary and batch -- hence every
decode GEMM shape: projections, MLP, converters, chunker and head at B and
B*C2 rows -- with one layer per stack and a one-chunk prompt, so that the
oracle stays cheap.  Same bar as tests/parity.py."""
import pytest

import photon_inputs as pi
from parity import check_against_oracle, gpu_generate

pytestmark = pytest.mark.gpu

SHAPES = [
    # name, d, heads, chunk, batch, new tokens
    ("photon-150m shape B32", 768, 12, (4, 4), 32, 32),
    ("photon-600m shape B64", 1536, 16, (4, 4), 64, 16),
    ("photon-600m-long shape B16", 1536, 16, (4, 4), 16, 32),
    ("photon-600m-2x2 shape B256", 1536, 16, (2, 2), 256, 8),
]


@pytest.mark.parametrize("name,d,H,chunk,B,N", SHAPES)
def test_decode_gemm_shapes(name, d, H, chunk, B, N):
    cfg = pi.PhotonConfig(d_model=d, n_heads=H, chunk=chunk, vocab=32000, n_top=1, n_enc1=1, n_dec1=1, n_dec0=1,
                          dtype="bf16")
    W, pr = pi.gen_weights(cfg, 31), pi.gen_prompts(cfg, B, cfg.S, 31)
    model, toks, lg = gpu_generate(cfg, W, pr, N)
    r = check_against_oracle(cfg, W, pr, toks, lg)
    print(f"[tiles] {name}: max_err={r['max_err']:.3g} noise_max={r['noise_max']:.3g} "
          f"near_ties={r['near_ties']}/{r['tokens']}", flush=True)
