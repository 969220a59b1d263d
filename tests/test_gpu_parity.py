"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on
seeded synthetic inputs.  See tests/parity.py for the tolerance rules."""
import numpy as np
import pytest

import photon_inputs as pi
from parity import gpu_generate, check_against_oracle, small_cfg

pytestmark = pytest.mark.gpu


def _inputs(cfg, B, P, seed, zero=()):
    return pi.gen_weights(cfg, seed, zero=zero), pi.gen_prompts(cfg, B, P, seed)


def _report(name, r):
    print(f"[parity] {name}: max_err={r['max_err']:.3g} noise_max={r['noise_max']:.3g} "
          f"near_ties={r['near_ties']}/{r['tokens']}", flush=True)


@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
def test_tiny_f32_exact_ids(mode):
    wl = pi.get(1)
    W, pr = _inputs(wl.cfg, wl.batch, wl.prompt, wl.seed)
    model, toks, lg = gpu_generate(wl.cfg, W, pr, wl.new_tokens, mode)
    r = check_against_oracle(wl.cfg, W, pr, toks, lg, mode)
    _report(f"tiny-f32 {mode}", r)


def test_tiny_f32_long_prompt_split_attention():
    # 300 top states: the top step's attention runs over several key splits
    # with a ragged last split
    cfg = pi.CONFIGS["tiny"]
    W, pr = _inputs(cfg, 2, 16 * 300, 21)
    model, toks, lg = gpu_generate(cfg, W, pr, 48)
    r = check_against_oracle(cfg, W, pr, toks, lg)
    _report("tiny-f32 P=4800", r)


def test_tiny_f32_long_cache_split_attention_rope_inside():
    # 1100 top states, a cache of 1103 slots (past the 1024 from which the
    # long-cache kernel runs): two sequences of two heads give 4 (sequence,
    # head) pairs, so the top step splits its keys over 5 workgroups per
    # pair, all resident at once, and that launch forms q, appends the new
    # K/V row and folds it in itself (last split), then the splits combine
    cfg = pi.CONFIGS["tiny"]
    W, pr = _inputs(cfg, 2, 16 * 1100, 23)
    model, toks, lg = gpu_generate(cfg, W, pr, 48)
    r = check_against_oracle(cfg, W, pr, toks, lg)
    _report("tiny-f32 P=17600", r)


@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
def test_small_bf16_ragged_batch(mode):
    cfg = small_cfg()
    W, pr = _inputs(cfg, 3, 64, 5)
    model, toks, lg = gpu_generate(cfg, W, pr, 48, mode)
    r = check_against_oracle(cfg, W, pr, toks, lg, mode)
    _report(f"small-bf16 B=3 {mode}", r)


@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
def test_small_bf16_hd96_chunk2x2(mode):
    cfg = small_cfg(d_model=384, n_heads=4, chunk=(2, 2), vocab=2000, n_top=2)
    W, pr = _inputs(cfg, 5, 40, 6)
    model, toks, lg = gpu_generate(cfg, W, pr, 24, mode)
    r = check_against_oracle(cfg, W, pr, toks, lg, mode)
    _report(f"bf16 hd96 2x2 {mode}", r)


def test_thm_a6_zero_chunker_gpu_recgen_equals_hiergen():
    cfg = small_cfg()
    W, pr = _inputs(cfg, 2, 32, 7, zero=("W_ch2",))
    m1, t1, l1 = gpu_generate(cfg, W, pr, 32, "recgen")
    kv1 = m1.top_kv().float().cpu().numpy()
    m2, t2, l2 = gpu_generate(cfg, W, pr, 32, "hiergen")
    kv2 = m2.top_kv().float().cpu().numpy()
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(kv1, kv2)


def test_deterministic_and_top_kv_matches_oracle():
    cfg = small_cfg()
    W, pr = _inputs(cfg, 2, 32, 8)
    m1, t1, l1 = gpu_generate(cfg, W, pr, 32)
    kv1 = m1.top_kv().float().cpu().numpy()
    m2, t2, l2 = gpu_generate(cfg, W, pr, 32)
    kv2 = m2.top_kv().float().cpu().numpy()
    np.testing.assert_array_equal(t1, t2)
    np.testing.assert_array_equal(l1, l2)
    np.testing.assert_array_equal(kv1, kv2)
    r = check_against_oracle(cfg, W, pr, t1, l1)
    st = r["state"]
    assert m1.position() == (st.top_len, 32 + 32)
    for l, e in enumerate(st.top):
        np.testing.assert_allclose(kv1[l, 0].transpose(0, 2, 1, 3), e["k"], atol=3e-2)
        np.testing.assert_allclose(kv1[l, 1].transpose(0, 2, 1, 3), e["v"], atol=3e-2)


def test_recgen_after_releasing_prefill_weights():
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon, PhotonError
    cfg = small_cfg()
    W, pr = _inputs(cfg, 2, 32, 9)
    ref_model, ref_t, _ = gpu_generate(cfg, W, pr, 32, logits=False)
    model = Photon(cfg, W)
    model.prefill(torch.from_numpy(pr).cuda(), 64)
    blob = model.w_prefill
    model.release_prefill_weights()
    blob.fill_(0xFF)                        # NaN bit patterns: decoding must not read them
    out = torch.empty((2, 2, cfg.S), dtype=torch.int32, device="cuda")
    model.decode_chunk(out[0])
    model.decode_chunk(out[1])
    torch.cuda.synchronize()
    got = out.permute(1, 0, 2).reshape(2, 32).cpu().numpy()
    np.testing.assert_array_equal(got, ref_t)
    with pytest.raises(PhotonError):
        model.decode_chunk(out[0])          # capacity: 64 tokens reached
    with pytest.raises(PhotonError):
        model.prefill(torch.from_numpy(pr).cuda(), 64)


def test_recgen_three_levels_never_reads_the_lower_encoders():
    # the prefill-only blob (every chunker and encoder below the top) is
    # overwritten after the prefill: RecGen's tokens do not change
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon
    cfg = small_cfg(chunk=(2, 3, 2), n_enc_hi=(1,), n_dec_hi=(1,))
    W, pr = _inputs(cfg, 2, 24, 10)
    ref_model, ref_t, _ = gpu_generate(cfg, W, pr, 24, logits=False)
    model = Photon(cfg, W)
    model.prefill(torch.from_numpy(pr).cuda(), 48)
    blob = model.w_prefill
    model.release_prefill_weights()
    blob.fill_(0xFF)
    out = torch.empty((2, 2, cfg.S), dtype=torch.int32, device="cuda")
    model.decode_chunk(out[0])
    model.decode_chunk(out[1])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.permute(1, 0, 2).reshape(2, 24).cpu().numpy(), ref_t)


def test_full_size_150m_sampled_sequences():
    # the benchmarked workload, full batch on the GPU; the oracle recomputes
    # sequences 0 and B-1 teacher-forced with the GPU's tokens
    wl = pi.get(2)
    W, pr = _inputs(wl.cfg, wl.batch, wl.prompt, wl.seed)
    rows = [0, wl.batch - 1]
    model, toks, lg = gpu_generate(wl.cfg, W, pr, wl.new_tokens, rows=rows)
    r = check_against_oracle(wl.cfg, W, pr[rows], toks, lg)
    _report("photon-150m B32 rows {0,31}", r)


def test_rewind_replays_identical_chunks():
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon
    cfg = small_cfg()
    W, pr = _inputs(cfg, 2, 32, 10)
    model = Photon(cfg, W)
    model.prefill(torch.from_numpy(pr).cuda(), 32 + 48)
    snap = model.state_snapshot()
    a = torch.empty((3, 2, cfg.S), dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    for c in range(3):
        model.decode_chunk(a[c])
    model.state_restore(snap, 32)
    assert model.position() == (2, 32)
    for c in range(3):
        model.decode_chunk(b[c])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())


@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
def test_graph_replay_matches_direct_launches(mode):
    import torch
    from hierarchical_autoregressive_lm_amd.photon import Photon
    cfg = small_cfg()
    W, pr = _inputs(cfg, 3, 32, 11)
    outs = []
    for graphs in (False, True):
        model = Photon(cfg, W)
        model.use_graphs(graphs)
        toks, _ = model.generate(torch.from_numpy(pr).cuda(), 64, mode=mode, logits=False)
        torch.cuda.synchronize()
        outs.append((toks.cpu().numpy(), model.top_kv().float().cpu().numpy(),
                     model.h_state().float().cpu().numpy()))
        assert model.position() == (6, 96)
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("mode", ["recgen", "hiergen"])
def test_bf16_prompt_sized_gemms(mode):
    # 2 x 4096 prompt tokens at C1 = 2: 4096 level-1 rows, so the prefill
    # GEMMs take the prompt-sized plan (run-time k loop, 128 x 256 tiles);
    # d = 384 and 4d = 1536 are multiples of its 3 x 64 k stages
    cfg = small_cfg(d_model=384, n_heads=4, chunk=(2, 2), vocab=2000, n_top=2)
    W, pr = _inputs(cfg, 2, 4096, 13)
    model, toks, lg = gpu_generate(cfg, W, pr, 16, mode)
    r = check_against_oracle(cfg, W, pr, toks, lg, mode)
    _report(f"bf16 long prompt {mode}", r)
