"""photon_attention_noalloc (split partials in the library's built-in
device array) against photon_attention (the caller's scratch): the same
kernels, so the outputs must be identical bit for bit.  Two calls in a row,
the second with a smaller input, for the one-query and the four-query
global kernel, each at a shape whose keys are split (so the array is really
used)."""
import pytest

pytestmark = pytest.mark.gpu

# (groups, heads, head_dim, queries, cap, keys): the second of each pair is
# smaller than the first
PAIRS = [((2, 4, 96, 1, 4096, 4000), (1, 2, 64, 1, 1024, 900)),
         ((2, 4, 128, 4, 2048, 2048), (1, 3, 32, 2, 640, 517))]


def _inputs(torch, G, H, hd, Q, cap, dt, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    K = torch.randn((G, H, cap, hd), generator=gen, device="cuda").to(dt)
    V = torch.randn((G, H, cap, hd), generator=gen, device="cuda").to(dt)
    q = torch.randn((G * Q, H * hd), generator=gen, device="cuda")
    return q, K, V


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_attention_equals_caller_scratch(pair, dtype):
    import torch
    from hierarchical_autoregressive_lm_amd import photon as P
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for i, (G, H, hd, Q, cap, keys) in enumerate(PAIRS[pair]):
        assert 0 < P.attention_scratch_bytes("global", G, H, hd, Q, cap) <= P.NOALLOC_SCRATCH_BYTES
        q, K, V = _inputs(torch, G, H, hd, Q, cap, dt, 11 + i)
        ref = torch.empty((G * Q, H * hd), dtype=dt, device="cuda")
        got = torch.full_like(ref, float("nan"))
        P.Attention("global", G, H, hd, Q, cap)(q, K, V, ref, keys)
        P.attention_noalloc("global", q, K, V, got, keys, Q)
        torch.cuda.synchronize()
        assert torch.equal(ref, got), f"call {i}: max |diff| {(ref.float() - got.float()).abs().max().item()}"
