"""Stand-alone decode attention (photon_attention) against the oracle.

Both kernels the decode path runs over a cache -- the top encoder's global
attention (split over keys when there are few (group, head) pairs) and the
decoders' chunk-confined attention -- are called through the C ABI on
seeded random inputs and compared element by element with the oracle's
float64 causal attention (oracle.photon_oracle.attention) on the same
values: K and V as stored (bf16-rounded for bf16), q in float32.

Bar, from the arithmetic: the kernels accumulate sum_j p_j v_j in float32
(online softmax: a few roundings per key), whose error is at most a small
multiple of sqrt(L) * 2^-24 * sum_j p_j |v_j| for L keys in practice (random
rounding errors add like a random walk; 4x that is the allowance, delta).
float32 outputs: |gpu - ref| <= 1e-4 * max(1, |ref|) + delta.  bf16 outputs
are that float32 value rounded to nearest: |gpu - ref| <= 1 bf16 ulp of ref
+ delta (half an ulp for the rounding, half for a float32 error that moves
the value across a rounding boundary).  delta matters only where the output
is a small average of many values of both signs.

Prompt (prefill) attention on bf16 caches runs on MFMA with q and the
probabilities entering each product as hi + lo bf16 terms; each operand is
then off by at most 2^-18 relative (hi = bf16(x) is within 2^-9|x|, lo
rounds the remainder to within 2^-9 of itself).  A score moves by at most
eps_s = 2^-18 * max_j sum_i |q_i k_ji|, so each weight p_j by a factor within
exp(+-2 eps_s), and the P V product adds 2^-18 * sum_j p_j |v_j|: the
allowance adds (4 eps_s + 2^-18) * sum_j p_j |v_j| (its first-order bound,
doubled).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from oracle import photon_oracle as O  # noqa: E402


@pytest.fixture(scope="module")
def P():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from hierarchical_autoregressive_lm_amd import photon
    return photon


def bf16_ulp(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def make_inputs(seed, G, H, hd, Q, cap, dtype):
    rng = np.random.default_rng([seed, 7])
    q = rng.standard_normal((G * Q, H * hd), dtype=np.float32)
    K = rng.standard_normal((G, H, cap, hd), dtype=np.float32)
    V = rng.standard_normal((G, H, cap, hd), dtype=np.float32)
    if dtype == "bf16":
        K, V = O.round_bf16(K).astype(np.float32), O.round_bf16(V).astype(np.float32)
    return q, K, V


def oracle_out(q, K, V, groups, H, hd, Q, L, split=False):
    """Reference for the given groups, [len(groups)*Q, H*hd] float64, and
    the allowance delta of the same shape (float32 accumulation; plus the
    hi + lo operand split when ``split``)."""
    qq = q.reshape(-1, Q, H, hd)[groups].astype(np.float64)           # [g, Q, H, hd]
    kk = K[groups][:, :, :L].transpose(0, 2, 1, 3).astype(np.float64)  # [g, L, H, hd]
    vv = V[groups][:, :, :L].transpose(0, 2, 1, 3).astype(np.float64)
    out = O.attention(qq, kk, vv, L - Q)                               # [g, Q, H, hd]
    mag = O.attention(qq, kk, np.abs(vv), L - Q)                       # sum_j p_j |v_j|
    delta = 4.0 * math.sqrt(L + 16) * 2.0 ** -24 * mag
    if split:
        # max over keys of sum_i |q_i k_ji| / sqrt(hd), per (g, query, head)
        qk = np.einsum("gthe,gshe->gths", np.abs(qq), np.abs(kk)).max(axis=-1) / math.sqrt(hd)
        eps_s = 2.0 ** -18 * qk                                        # [g, Q, H]
        delta = delta + (4.0 * eps_s[..., None] + 2.0 ** -18) * mag
    n = len(groups) * Q
    return out.reshape(n, H * hd), delta.reshape(n, H * hd)


def run(P, kind, dtype, q, K, V, G, H, hd, Q, L, cap):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dq = torch.from_numpy(q).cuda()
    dK = torch.from_numpy(K).to(tdt).cuda().contiguous()
    dV = torch.from_numpy(V).to(tdt).cuda().contiguous()
    out = torch.full((G * Q, H * hd), float("nan"), dtype=tdt, device="cuda")
    P.Attention(kind, G, H, hd, Q, cap)(dq, dK, dV, out, L)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check(got, ref_delta, dtype):
    ref, delta = ref_delta
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    if dtype == "f32":
        bound = 1e-4 * np.maximum(1.0, np.abs(ref)) + delta
    else:
        bound = bf16_ulp(ref) + delta
    worst = float((err / bound).max())
    assert worst <= 1.0, f"max error / bound = {worst:.3f}"


GLOBAL_CASES = [
    # G, H, hd, Q, L, cap, dtype
    (1, 1, 32, 1, 1, 1, "f32"),         # a single key
    (2, 3, 64, 1, 17, 20, "bf16"),      # ragged, few pairs: split over keys
    (3, 2, 96, 2, 300, 333, "bf16"),    # two queries per group
    (2, 2, 128, 4, 257, 300, "bf16"),   # four queries, ragged tail
    (1, 1, 64, 4, 4, 4, "f32"),         # as many queries as keys
    (2, 4, 32, 1, 700, 700, "f32"),
    (4, 4, 96, 1, 2100, 2176, "bf16"),  # long cache: wide workgroups, splits
    (64, 16, 96, 1, 272, 288, "bf16"),  # 600M, B64 top step: no split
    (16, 16, 96, 1, 2056, 2064, "bf16"),  # 600M, B16 long context top step
]


@pytest.mark.parametrize("G,H,hd,Q,L,cap,dtype", GLOBAL_CASES)
def test_global_attention_matches_oracle(P, G, H, hd, Q, L, cap, dtype):
    q, K, V = make_inputs(G * 1000 + L, G, H, hd, Q, cap, dtype)
    got = run(P, "global", dtype, q, K, V, G, H, hd, Q, L, cap)
    groups = np.arange(G) if G <= 16 else np.array([0, 1, G // 2, G - 1])
    rows = (groups[:, None] * Q + np.arange(Q)[None, :]).reshape(-1)
    check(got[rows], oracle_out(q, K, V, groups, H, hd, Q, L), dtype)


CHUNK_CASES = [
    # G, H, hd, Q, L, cap, dtype
    (5, 3, 64, 1, 1, 4, "bf16"),        # first token-decoder step: one key
    (5, 3, 64, 1, 4, 4, "bf16"),
    (7, 2, 96, 4, 4, 4, "bf16"),        # level-1 decoder: causal over the chunk
    (3, 5, 32, 2, 3, 4, "f32"),
    (2, 2, 128, 1, 16, 16, "bf16"),     # the largest chunk
    (9, 3, 96, 8, 8, 8, "f32"),
    (33, 12, 64, 1, 2, 2, "bf16"),      # pairs not a multiple of a wave's 4
]


@pytest.mark.parametrize("G,H,hd,Q,L,cap,dtype", CHUNK_CASES)
def test_chunk_attention_matches_oracle(P, G, H, hd, Q, L, cap, dtype):
    q, K, V = make_inputs(G * 100 + L, G, H, hd, Q, cap, dtype)
    got = run(P, "chunk", dtype, q, K, V, G, H, hd, Q, L, cap)
    check(got, oracle_out(q, K, V, np.arange(G), H, hd, Q, L), dtype)


PREFILL_CASES = [
    # G, H, hd, T, cap, dtype
    (1, 1, 64, 1, 1, "bf16"),           # a one-row prompt
    (2, 3, 64, 37, 40, "bf16"),         # shorter than one key tile, ragged
    (2, 2, 96, 300, 300, "bf16"),       # several query blocks and key tiles
    (1, 2, 128, 129, 130, "bf16"),      # one row past a query block
    (3, 2, 32, 200, 200, "bf16"),
    (2, 2, 64, 150, 150, "f32"),        # float32 caches: FMA kernel
]


@pytest.mark.parametrize("G,H,hd,T,cap,dtype", PREFILL_CASES)
def test_prefill_attention_matches_oracle(P, G, H, hd, T, cap, dtype):
    q, K, V = make_inputs(G * 10000 + T, G, H, hd, T, cap, dtype)
    got = run(P, "prefill", dtype, q, K, V, G, H, hd, T, T, cap)
    check(got, oracle_out(q, K, V, np.arange(G), H, hd, T, T, split=dtype == "bf16"), dtype)


def test_prefill_attention_long_prompt_sampled(P):
    """A level-1 encoder's prompt at the 600M 2x2 shape: 4096 rows, 16
    heads, hd 96; sampled query rows against the oracle."""
    G, H, hd, T = 2, 16, 96, 4096
    q, K, V = make_inputs(77, G, H, hd, T, T, "bf16")
    got = run(P, "prefill", "bf16", q, K, V, G, H, hd, T, T, T)
    rows = np.array([0, 1, 63, 64, 127, 128, 2049, 4094, 4095])
    for g in range(G):
        for t in rows:
            # the oracle's attention for one query row t: a cache of t keys
            qq = q.reshape(G, T, H * hd)[g:g + 1, t:t + 1]
            ref = oracle_out(qq.reshape(1, H * hd), K[g:g + 1], V[g:g + 1], np.arange(1), H, hd, 1, t + 1,
                             split=True)
            check(got[g * T + t:g * T + t + 1], ref, "bf16")


def test_chunk_attention_standalone_size_sampled(P):
    """The stand-alone measurement's launch: 65536 sub-chunks x 16 heads,
    hd 96, 4 keys (1.6 GB of K/V); sampled groups against the oracle."""
    G, H, hd, Q, L = 65536, 16, 96, 1, 4
    gen = torch.Generator(device="cuda").manual_seed(1234)
    K = torch.randn((G, H, L, hd), generator=gen, device="cuda").to(torch.bfloat16)
    V = torch.randn((G, H, L, hd), generator=gen, device="cuda").to(torch.bfloat16)
    q = torch.randn((G * Q, H * hd), generator=gen, device="cuda")
    out = torch.empty((G * Q, H * hd), dtype=torch.bfloat16, device="cuda")
    P.Attention("chunk", G, H, hd, Q, L)(q, K, V, out, L)
    torch.cuda.synchronize()
    groups = np.array([0, 1, 4097, 33333, G - 2, G - 1])
    idx = torch.from_numpy(groups).cuda()
    qs = q.view(G, Q, H * hd)[idx].cpu().numpy().reshape(len(groups) * Q, H * hd)
    Ks = K[idx].float().cpu().numpy()
    Vs = V[idx].float().cpu().numpy()
    ref = oracle_out(qs, Ks, Vs, np.arange(len(groups)), H, hd, Q, L)
    got = out.view(G, Q, H * hd)[idx].float().cpu().numpy().reshape(len(groups) * Q, H * hd)
    check(got.astype(np.float64), ref, "bf16")
