#!/usr/bin/env python
"""Decode benchmark of PHOTON recursive generation (RecGen) on one MI355X.

A step is one decode chunk (one replay of the chunk's captured HIP graph):
the whole hot path (Converter^2, level-1
decoder, C1 token-decoder steps with the greedy head, Chunker^2 feedback and
the top-encoder step over the global K/V) for every sequence of the batch,
B * S tokens (S = C1 * C2, or C1 * ... * CL with --chunk).  The workload is prefilled once (untimed); the timed
steps decode chunk after chunk from the prompt end, rewinding to the prompt
end (restore h, reset the position) whenever the workload's new_tokens are
used up, so every step runs at the workload's real cache lengths.

The default workload is the largest one that fits one GPU: the 600M shape
with 2x2 chunks, 256 sequences, 8192-token prompts and 512 new tokens.

Prints one JSON line: decode tok/s (value), TPM = tok/s per GiB of resident
decode weights + top K/V + decoder K/V + state, the whole path's fraction of
the HBM roofline (algorithmic bytes per chunk at 8 TB/s), the achieved
bandwidth of the kernel class that moves the most bytes (events recorded by
every kernel dispatch, in a traced pass over the same steps right after the
timed ones) against 8 TB/s and against a measured plain copy, the two
attention kernels' own fractions, per-class figures, decode tok/s and TPM of
every other workload (one timed pass each), and the CPU oracle timed on a
bounded sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
METRIC = "decode tok/s and TPM (tok/s/GiB) at 1 MI355X; % HBM roofline"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(wl, W, prompt, seqs, threads, target_s=15.0, vanilla=False, sampling=None, compute="f64"):
    """The oracle as it stands, RecGen decode phase only (perf_counter),
    prefill and weight setup untimed.  seqs = 0: one sequence is decoded
    first to size the sample, then as many sequences (up to the batch) as
    fill about target_s seconds at that rate, or the whole batch when that
    rate puts it under 2 * target_s (a batch decodes faster per sequence
    than one sequence alone); when the whole batch takes less than
    target_s / 2, its decode is repeated from the same prefill state until
    target_s is filled."""
    from threadpoolctl import threadpool_limits
    import photon_inputs as pi
    from oracle import photon_oracle as O

    def decode(st):
        t0 = time.perf_counter()
        if vanilla:
            O.vanilla_decode(m, st, wl.new_tokens)
        else:
            for _ in range(wl.chunks):
                O.decode_chunk(m, st, sampling=sampling)
        return time.perf_counter() - t0

    prefill = O.vanilla_prefill if vanilla else O.prefill
    with threadpool_limits(limits=threads):
        m = O.Model(pi.vanilla_of(wl.cfg) if vanilla else wl.cfg, W, compute=compute)
        reps = 1
        if seqs <= 0:
            t1 = decode(prefill(m, prompt[:1]))
            fit = target_s / t1
            seqs = wl.batch if fit >= wl.batch / 2 else max(1, min(wl.batch, round(fit)))
            if seqs == 1:
                return wl.new_tokens / t1, t1, 1, 1
        st0 = prefill(m, prompt[:seqs])
        copy = (lambda st: O.VanillaState([{"k": e["k"].copy(), "v": e["v"].copy()} for e in st.cache],
                                          st.z.copy(), st.n)) if vanilla else (lambda st: st.copy())
        dt = decode(copy(st0))
        if seqs == wl.batch and dt < target_s / 2:
            reps = max(1, round(target_s / dt))
            dt += sum(decode(copy(st0)) for _ in range(reps - 1))
    return reps * seqs * wl.new_tokens / dt, dt, seqs, reps


def cpu_baseline_injected(wl, W, threads, mode="recgen", target_s=15.0, sampling=None, compute="f64"):
    """The oracle as it stands, decode phase only (perf_counter), on the
    fixed sample of sequences {0, B-1}, starting at the prompt end from the
    seeded decode state the parity tests inject
    (photon_inputs.gen_decode_state): the top K/V over the prompt's top
    states, the last top output, and for HierGen the level-1 K/V.  The
    oracle's prefill of even two sequences of the long prompts takes it many
    minutes, and the decode work does not depend on the state's values.
    Chunks are decoded in order until about target_s seconds are filled or
    the workload's chunks are used up, and then again from the same state.
    Returns (tok/s, seconds, sequences, chunks decoded)."""
    from threadpoolctl import threadpool_limits
    import photon_inputs as pi
    from oracle import photon_oracle as O

    rows = sorted({0, wl.batch - 1})
    n = wl.prompt // wl.cfg.S
    with threadpool_limits(limits=threads):
        m = O.Model(wl.cfg, W, compute=compute)
        seqs = [pi.gen_decode_state(wl.cfg, r, n, mode, wl.seed) for r in rows]
        dt, done = 0.0, 0
        while dt < target_s:
            st = O.state_from_arrays(m, seqs)
            for _ in range(wl.chunks):
                t0 = time.perf_counter()
                O.decode_chunk(m, st, mode, sampling=sampling)
                dt += time.perf_counter() - t0
                done += 1
                if dt >= target_s:
                    break
    return len(rows) * wl.cfg.S * done / dt, dt, rows, done


def per_config_lines(P, torch, skip, mode, only=None, trace=False):
    """Decode tok/s and TPM of every workload but `skip` (or of workload
    `only`): the workload's seeded weights and prompts, prefill, one untimed
    pass over its chunks, then one timed pass (graph replay, the headline's
    method); with `trace`, a third pass with every dispatch traced gives the
    line its path-roofline fraction and the top attention's in place."""
    import photon_inputs as pi
    out = {}
    for idx in sorted(pi.WORKLOADS):
        if idx == skip or (only is not None and idx != only):
            continue
        wl = pi.get(idx)
        log(f"per-config line: {wl.name}")
        W = pi.gen_weights(wl.cfg, wl.seed)
        model = P.Photon(wl.cfg, W)
        del W
        model.prefill(torch.from_numpy(pi.gen_prompts(wl.cfg, wl.batch, wl.prompt, wl.seed)).cuda(),
                      wl.max_tokens, mode)
        if mode == "recgen":
            model.release_prefill_weights()
        snap = model.state_snapshot()
        tok = torch.empty((wl.batch, wl.cfg.S), dtype=torch.int32, device="cuda")
        for timed in (False, True):
            model.state_restore(snap, wl.prompt)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(wl.chunks):
                model.decode_chunk(tok)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
        path = None
        if trace:
            # the same pass again, every dispatch traced: algorithmic bytes
            # per chunk, so the line carries its own HBM-roofline fraction
            model.state_restore(snap, wl.prompt)
            model.trace_enable(None)
            for _ in range(wl.chunks):
                model.decode_chunk(tok)
            torch.cuda.synchronize()
            cls = model.trace_read()
            model.trace_enable([])
            chunk_bytes = sum(v["bytes"] for v in cls.values()) / wl.chunks
            roof = wl.batch * wl.cfg.S / (chunk_bytes / (HBM_PEAK_GBS * 1e9))
            path = {"algorithmic_bytes_per_step": round(chunk_bytes), "roofline_tok_s": round(roof, 1),
                    "frac": round(wl.batch * wl.new_tokens / dt / roof, 4)}
            if "attn_top" in cls:
                # the top attention in place (the other branch beside it)
                v = cls["attn_top"]
                gbs = v["bytes"] / (v["ms"] * 1e-3) / 1e9
                path["attn_top"] = {"frac": round(gbs / HBM_PEAK_GBS, 4), "GB_s": round(gbs, 1),
                                    "avg_us": round(v["ms"] * 1e3 / v["launches"], 2),
                                    "bytes_per_launch": round(v["bytes"] / v["launches"])}
        rep = model.report(wl.batch, wl.max_tokens, mode)
        resident = rep["weights_decode"] + rep["top_kv"] + rep["dec_kv"] + rep["state"]
        if mode == "hiergen":
            resident += rep["weights_prefill_only"] + rep["lower_kv"]
        kv = rep["top_kv"] + rep["dec_kv"] + rep["lower_kv"]
        tok_s = wl.batch * wl.new_tokens / dt
        out[wl.name] = {"tok_s": round(tok_s, 1), "ms_per_step": round(dt / wl.chunks * 1e3, 4),
                        "steps": wl.chunks, "dtype": "bf16" if wl.cfg.dtype == "bf16" else "f32",
                        "tpm": round(tok_s / (resident / 2 ** 30), 1), "resident_gib": round(resident / 2 ** 30, 4),
                        "tpm_kv_only": round(tok_s / (kv / 2 ** 30), 1),
                        **({"path_roofline": path} if path else {})}
        model.close()
        del model, snap, tok
        torch.cuda.empty_cache()
    return out


def host_info():
    """CPU model (from /proc/cpuinfo) and the BLAS numpy calls."""
    from threadpoolctl import threadpool_info
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
    return model, ", ".join(blas) or None


def copy_peak(torch):
    """Achievable HBM bandwidth: a plain device-to-device copy of 1 GiB
    (read + write counted), alternating two sources so no pass is served
    from the Infinity Cache; GB/s."""
    n = 1 << 28
    srcs = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    dst = torch.empty(n, dtype=torch.float32, device="cuda")
    for i in range(3):
        dst.copy_(srcs[i % 2])
    iters = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        dst.copy_(srcs[i % 2])
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 4 * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del srcs, dst
    torch.cuda.empty_cache()
    return gbs


def measured_traffic(wl, cls):
    """HBM bytes per launch of kernel class `cls` on this workload from the
    committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary (calibrated against a
    plain copy) and their ratio to the algorithmic bytes of the profiled
    launches, or None when there is none or the kernel's source files
    changed since the counters were taken."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json"))):
        rec = json.load(open(path))
        if rec.get("workload") != wl.name or rec.get("kernel_class") != cls:
            continue
        h = hashlib.sha256()
        for f in rec["source_files"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != rec["source_sha256"]:
            log(f"{os.path.basename(path)}: kernel sources changed since the counters were taken")
            return None, None, None
        return rec["traffic_bytes_per_launch"], rec["traffic_over_algorithmic"], os.path.relpath(path, ROOT)
    return None, None, None


def measured_counters(wl):
    """MFMA use and DRAM traffic of the workload's kernels from the committed
    rocprofv3 counter summary (profiles/counters_photon600m.json), while the
    kernels' sources still hash to it: the time-weighted MFMA busy fraction
    and executed TFLOP/s of the prompt GEMMs (M >= 2048 rows), the prompt
    attention and the decode GEMMs, and the top attention's DRAM reads per
    launch.  None when the workload was not profiled or a source changed."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters_photon600m.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["source_files"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["source_sha256"] or wl.name not in rec["workloads"]:
        return None
    ks = rec["workloads"][wl.name]

    def group(pred):
        sel = {k: v for k, v in ks.items() if pred(k)}
        t = sum(v["avg_us"] * v["dispatches"] for v in sel.values())
        if not t:
            return None
        return {"mfma_busy": round(sum(v["mfma_busy"] * v["avg_us"] * v["dispatches"] for v in sel.values()) / t, 4),
                "mfma_tflop_s_executed": round(sum(v["mfma_tflop_s"] * v["avg_us"] * v["dispatches"]
                                                   for v in sel.values()) / t, 1),
                "kernels": len(sel)}
    # prompt-sized GEMMs: the LDS-streaming kernel with a run-time k loop
    # (template argument NKB, the sixth, is 0)
    prompt = lambda k: k.startswith("gemm_lds_kernel<") and k[len("gemm_lds_kernel<"):].split(",")[5].strip() == "0"
    top = [v for k, v in ks.items() if k.startswith("attn_decode_kernel")]
    return {"source": "profiles/counters_photon600m.json",
            "prompt_gemm": group(prompt),
            "prompt_attention": group(lambda k: k.startswith("attn_prefill_mfma")),
            "decode_gemm": group(lambda k: k.startswith("gemm_") and not prompt(k)),
            "attn_top_dram_read_bytes": top[0]["dram_read_bytes"] if top else None}


def attn_standalone(P, torch, wl, top_len, top_cap):
    """photon_attention alone, K/V rotated over copies larger than the
    Infinity Cache: the chunk kernel at the token decoder's shape (one query
    over C1 keys per (sub-chunk, head)) over enough sub-chunks for >= 1 GB of
    K/V, and the global kernel at the workload's top step (B sequences over
    the final top length).  Algorithmic bytes: K and V read once, q
    (float32) read and the output written once."""
    cfg = wl.cfg
    H, hd = cfg.n_heads, cfg.d_model // cfg.n_heads
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    eb = 2 if cfg.dtype == "bf16" else 4
    res = {}
    C1 = cfg.chunk[0]
    per_group = H * C1 * hd * 2 * eb
    G = 1 << max(0, math.ceil(math.log2(1.05e9 / per_group)))
    specs = [("chunk", G, 1, C1, C1), ("global", wl.batch, 1, top_len, top_cap)]
    for kind, G, Q, L, cap in specs:
        kv_bytes = G * H * cap * hd * eb
        copies = max(2, math.ceil(600e6 / (2 * kv_bytes)) + 1)
        gen = torch.Generator(device="cuda").manual_seed(5)
        Ks = [torch.randn((G, H, cap, hd), generator=gen, device="cuda").to(tdt) for _ in range(copies)]
        Vs = [torch.randn((G, H, cap, hd), generator=gen, device="cuda").to(tdt) for _ in range(copies)]
        q = torch.randn((G * Q, H * hd), generator=gen, device="cuda")
        out = torch.empty((G * Q, H * hd), dtype=tdt, device="cuda")
        att = P.Attention(kind, G, H, hd, Q, cap)
        for i in range(3):
            att(q, Ks[i % copies], Vs[i % copies], out, L)
        iters = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(iters):
            att(q, Ks[i % copies], Vs[i % copies], out, L)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        nbytes = G * H * L * hd * 2 * eb + G * Q * H * hd * (4 + eb)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[kind] = {"groups": G, "heads": H, "head_dim": hd, "queries": Q, "keys": L,
                     "bytes_per_launch": nbytes, "avg_us": round(us, 2), "GB_s": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}
        del Ks, Vs, q, out, att
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed decode chunks (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed decode chunks (default: the workload's)")
    ap.add_argument("--workload", type=int, default=5,
                    help="1..5 (default 5: photon-600m-2x2 B256 P8192 N512, the largest single-GPU workload)")
    ap.add_argument("--mode", default="recgen", choices=["recgen", "hiergen", "vanilla"],
                    help="PHOTON RecGen / HierGen, or the flat Transformer baseline matched to the workload's "
                         "shape (same width, heads, vocabulary; as many layers as the PHOTON stacks)")
    ap.add_argument("--cpu-seqs", type=int, default=0,
                    help="-1: skip the oracle baseline.  PHOTON modes time sequences {0, B-1} from an injected "
                         "state; the flat baseline: 0 sizes its sample for ~15 s, N > 0 takes N sequences")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the decode tok/s and TPM lines of the other workloads")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch (stress runs)")
    ap.add_argument("--prompt", type=int, default=None, help="override the workload's prompt length")
    ap.add_argument("--new-tokens", type=int, default=None, help="override the workload's generated tokens")
    ap.add_argument("--no-attn-standalone", action="store_true", help="skip the stand-alone attention figures")
    ap.add_argument("--chunk", default=None, metavar="C1,C2[,C3[,C4]]",
                    help="override the hierarchy's chunk sizes (2 to 4 levels); each level added above the "
                         "second gets as many encoder and decoder layers as level 1")
    ap.add_argument("--sample", default=None, metavar="T,K",
                    help="sampling decode at temperature T with a top-K cut (K = 0: whole vocabulary) instead of "
                         "greedy; also times the multi-query aggregation of the batch in groups of 9")
    ap.add_argument("--no-trace", action="store_true",
                    help="skip the traced passes (per-class figures, roofline): for runs under a profiler, "
                         "which gives its own per-kernel figures")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the decode path shards by batch "
              "with no collective, so N GPUs give N x the one-GPU figure; nothing here uses a second GPU.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import photon_inputs as pi
    from hierarchical_autoregressive_lm_amd import photon as P
    from hierarchical_autoregressive_lm_amd.photon import Photon, Vanilla

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = pi.get(args.workload)
    if args.batch or args.prompt or args.new_tokens:
        import dataclasses
        b = args.batch or wl.batch
        p = args.prompt or wl.prompt
        n = args.new_tokens or wl.new_tokens
        name = wl.name.split(" B")[0] + f" bf16 B{b} P{p} N{n}"
        wl = dataclasses.replace(wl, name=name + " (override)", batch=b, prompt=p, new_tokens=n)
    if args.chunk:
        import dataclasses
        chunk = tuple(int(x) for x in args.chunk.split(","))
        extra = len(chunk) - 2
        c0 = wl.cfg
        cfg_l = c0.with_(chunk=chunk, n_enc_hi=(c0.n_enc1,) * extra, n_dec_hi=(c0.n_dec1,) * extra)
        if (wl.prompt % cfg_l.S) or (wl.new_tokens % cfg_l.S):
            sys.exit(f"prompt and new tokens must be multiples of S = {cfg_l.S}")
        wl = dataclasses.replace(wl, cfg=cfg_l, name=wl.name + " chunk " + "x".join(map(str, chunk)))
    cfg = wl.cfg
    K = args.steps if args.steps is not None else wl.chunks
    Wm = args.warmup if args.warmup is not None else wl.chunks
    B, S = wl.batch, cfg.S
    log(f"workload {wl.name}: generating weights")
    vanilla = args.mode == "vanilla"
    mcfg = pi.vanilla_of(cfg) if vanilla else cfg
    W = pi.gen_weights(mcfg, wl.seed)
    prompt = pi.gen_prompts(cfg, B, wl.prompt, wl.seed)
    model = Vanilla(mcfg, W, S) if vanilla else Photon(cfg, W)
    # prefill (untimed for the decode metric): wall time and per-class kernel
    # time of the one prefill, against the bf16 dense MFMA peak
    d_prompt = torch.from_numpy(prompt).cuda()
    model.trace_enable([] if args.no_trace else None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    model.prefill(d_prompt, wl.max_tokens, args.mode)
    torch.cuda.synchronize()
    pre_s = time.perf_counter() - t0
    pre_cls = model.trace_read()
    model.trace_enable([])
    pre_flops = sum(v["flops"] for v in pre_cls.values())

    def tf(names):
        ms = sum(pre_cls[n]["ms"] for n in names if n in pre_cls)
        fl = sum(pre_cls[n]["flops"] for n in names if n in pre_cls)
        return {"ms": round(ms, 3), "tflop": round(fl / 1e12, 3),
                "tflop_s": round(fl / (ms * 1e-3) / 1e12, 1) if ms else None}
    counters = measured_counters(wl)
    prefill = {"seconds": round(pre_s, 4), "tok_s": round(B * wl.prompt / pre_s, 1),
               "tflop": round(pre_flops / 1e12, 3), "tflop_s": round(pre_flops / pre_s / 1e12, 1),
               "attention": tf(["attn_prefill"]),
               "gemm": tf(["gemm_qkv", "gemm_o", "gemm_up", "gemm_down", "gemm_chunk"]),
               "by_class": {n: tf([n]) for n in sorted(pre_cls)},
               "note": "bf16 prompts: gemm_qkv includes the RoPE rotation and the K/V cache append in its "
                       "epilogue (no rope_kv launch); attention flops are the causal half, counted once "
                       "although q and p each enter the products as two bf16 terms",
               "mfma_peak_tflop_s": MFMA_BF16_PEAK_TFLOPS}
    log(f"prefill {pre_s:.3f} s ({prefill['tflop_s']} TFLOP/s)")
    if args.mode == "recgen":
        model.release_prefill_weights()
    sampling = None
    if args.sample:
        if vanilla:
            raise SystemExit("--sample applies to the PHOTON modes")
        t_, k_ = args.sample.split(",")
        sampling = {"temperature": float(t_), "top_k": int(k_), "seed": wl.seed}
        model.set_sampling(sampling["temperature"], sampling["top_k"], sampling["seed"], B)
    snap = model.state_snapshot()
    tok = torch.empty((B, S), dtype=torch.int32, device="cuda")
    pos = [0]

    def step():
        if pos[0] == wl.chunks:
            model.state_restore(snap, wl.prompt)
            pos[0] = 0
        model.decode_chunk(tok)
        pos[0] += 1

    # warmup, then the timed steps: each chunk replays the captured HIP graph
    model.trace_enable([])
    model.state_restore(snap, wl.prompt)
    pos[0] = 0
    for _ in range(Wm):
        step()
    model.state_restore(snap, wl.prompt)
    pos[0] = 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    # the same K steps again, traced: every kernel dispatch records its own
    # start and stop events (tracing launches the chunk's kernels directly
    # instead of through the graph; the kernels are the same), giving the
    # per-class times and bytes; the class that moves the most algorithmic
    # bytes per step is the one whose HBM roofline bounds the path
    per_class, dominant, dom = {}, None, None
    if not args.no_trace:
        model.state_restore(snap, wl.prompt)
        pos[0] = 0
        model.trace_enable(None)
        for _ in range(K):
            step()
        torch.cuda.synchronize()
        per_class = model.trace_read()
        model.trace_enable([])
        dominant = max(per_class, key=lambda k: per_class[k]["bytes"])
        dom = per_class[dominant]
        log(f"dominant kernel class (bytes): {dominant}")

    tok_s = B * S * K / dt
    rep = model.report(B, wl.max_tokens, args.mode)
    resident = rep["weights_decode"] + rep["top_kv"] + rep["dec_kv"] + rep["state"]
    if args.mode == "hiergen":
        resident += rep["weights_prefill_only"] + rep["lower_kv"]
    # vanilla: weights_decode is its one blob, top_kv its token K/V
    gib = resident / 2 ** 30
    kv_gib = (rep["top_kv"] + rep["dec_kv"] + rep["lower_kv"]) / 2 ** 30
    path_roof = roofline = None
    if dom:
        chunk_bytes = sum(v["bytes"] for v in per_class.values()) / K
        ideal_s = chunk_bytes / (HBM_PEAK_GBS * 1e9)
        roof_tok_s = B * S / ideal_s
        achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        traffic, traffic_ratio, traffic_src = measured_traffic(wl, dominant)
        path_roof = {"algorithmic_bytes_per_step": round(chunk_bytes), "ideal_us_per_step": round(ideal_s * 1e6, 2),
                     "roofline_tok_s": round(roof_tok_s, 1), "frac": round(tok_s / roof_tok_s, 4)}
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "traffic_over_algorithmic": traffic_ratio, "traffic_source": traffic_src,
                    "copy_peak": None, "frac_of_copy": None,
                    "kernel": dominant, "launches": dom["launches"],
                    "avg_us": round(dom["ms"] * 1e3 / dom["launches"], 2),
                    "bytes_per_launch": round(dom["bytes"] / dom["launches"])}

    if roofline:
        cp = copy_peak(torch)
        roofline["copy_peak"] = round(cp, 1)
        roofline["frac_of_copy"] = round(roofline["achieved"] / cp, 4)
        log(f"copy peak {cp:.0f} GB/s")

    agg = None
    if sampling:
        # best-of-N and majority vote over groups of 9 queries of the batch,
        # on the workload's shape (B sequences x new_tokens)
        gen = torch.Generator(device="cuda").manual_seed(7)
        at = torch.randint(0, cfg.vocab, (B, wl.new_tokens), generator=gen, device="cuda", dtype=torch.int32)
        al = -torch.rand((B, wl.new_tokens), generator=gen, device="cuda") * 8
        for _ in range(3):
            P.aggregate(at, al, 9)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            P.aggregate(at, al, 9)
        e1.record()
        torch.cuda.synchronize()
        agg = {"group": 9, "groups": (B + 8) // 9, "tokens_per_query": wl.new_tokens,
               "us": round(e0.elapsed_time(e1) * 1e3 / 20, 2)}

    attn = None
    model.close()
    del model, snap
    torch.cuda.empty_cache()
    if not args.no_attn_standalone and not vanilla:
        log("stand-alone attention")
        attn = attn_standalone(P, torch, wl, wl.max_tokens // S, rep["top_len"])

    per_config = None
    if not args.no_per_config and not vanilla and not (args.chunk or args.batch or args.prompt or args.new_tokens):
        per_config = per_config_lines(P, torch, args.workload, args.mode, trace=not args.no_trace)
    versus = None
    if vanilla and not (args.chunk or args.batch or args.prompt or args.new_tokens):
        # PHOTON RecGen on the same workload (same batch, prompt and new
        # tokens; one timed pass of its chunks) for the TPM ratio
        ph = per_config_lines(P, torch, None, "recgen", only=args.workload, trace=True)[wl.name]
        versus = {"photon_recgen": ph,
                  "tpm_ratio": round(ph["tpm"] / (tok_s / gib), 1),
                  "tpm_kv_only_ratio": round(ph["tpm_kv_only"] / (tok_s / kv_gib), 1),
                  "tok_s_ratio": round(ph["tok_s"] / tok_s, 2)}

    cpu = None
    if args.cpu_seqs >= 0:
        # the oracle's BLAS threads: the host's CPU share for this GPU where
        # the environment states it (OMP_NUM_THREADS), else every core this
        # process may run on
        visible = len(os.sched_getaffinity(0))
        threads = min(visible, int(os.environ.get("OMP_NUM_THREADS") or visible))
        log(f"oracle baseline, {threads} threads ({visible} visible)")
        # bf16 models: the oracle's float32 arithmetic (its second
        # implementation of the rounding contract); fp32 models: float64
        compute = "f64" if cfg.dtype == "f32" else "f32"
        prec = "float64" if cfg.dtype == "f32" else "float32 arithmetic with the bf16 rounding contract"
        cpu_model, blas = host_info()
        if vanilla:
            cv, cdt, ns, reps = cpu_baseline(wl, W, prompt, args.cpu_seqs, threads, vanilla=True, compute=compute)
            rep_txt = f", decoded {reps} times from the same prefill" if reps > 1 else ""
            sample = (f"flat-baseline decode phase of {ns} of {B} sequences, all {wl.chunks} chunks{rep_txt} "
                      f"({reps * ns * wl.new_tokens} tokens, {cdt:.1f} s), numpy {prec}")
        else:
            cv, cdt, rows, done = cpu_baseline_injected(wl, W, threads, args.mode, sampling=sampling, compute=compute)
            what = ("sampled " if sampling else "") + ("HierGen" if args.mode == "hiergen" else "RecGen")
            sample = (f"{what} decode phase of sequences {rows} of {B}, {done} chunks from the prompt end "
                      f"({len(rows) * S * done} tokens, {cdt:.1f} s) from the seeded decode state the parity "
                      f"tests inject (decode work does not depend on its values), numpy {prec}")
        cpu = {"value": round(cv, 2), "unit": "tok/s", "cores": threads, "visible_cores": visible,
               "kind": "oracle", "cpu_model": cpu_model, "blas": blas, "sample": sample}

    attn_roof = None
    if per_class:
        attn_roof = {}
        for k in ("attn_top", "attn_chunk"):
            if k in per_class:
                v = per_class[k]
                gbs = v["bytes"] / (v["ms"] * 1e-3) / 1e9
                attn_roof[k] = {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(gbs / HBM_PEAK_GBS, 4), "launches_per_step": v["launches"] // K,
                                "avg_us": round(v["ms"] * 1e3 / v["launches"], 2),
                                "bytes_per_launch": round(v["bytes"] / v["launches"])}

    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(dt / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "mode": args.mode, "batch": B, "prompt": wl.prompt,
                   "new_tokens": wl.new_tokens, "d_model": cfg.d_model, "heads": cfg.n_heads,
                   "chunk": list(cfg.chunk),
                   **({"layers": mcfg.n_layers} if vanilla else
                      {"layers_top_enc1_dec1_dec0": [cfg.n_top, cfg.n_enc1, cfg.n_dec1, cfg.n_dec0],
                       **({"layers_enc_dec_above_level1": [list(cfg.n_enc_hi), list(cfg.n_dec_hi)]}
                          if cfg.L > 2 else {})}),
                   "vocab": cfg.vocab, "tokens_per_step": B * S,
                   **({"sampling": {"temperature": sampling["temperature"], "top_k": sampling["top_k"]}}
                      if sampling else {})},
        "tpm": round(tok_s / gib, 1),
        "tpm_unit": ("tok/s/GiB (weights + token K/V + state)" if vanilla else
                     "tok/s/GiB (decode weights + top K/V + decoder K/V + state)"),
        "resident_gib": round(gib, 4),
        "tpm_kv_only": round(tok_s / kv_gib, 1),
        "path_roofline": path_roof,
        "roofline": roofline,
        "attention_roofline": attn_roof,
        "kernels": {k: {"launches_per_step": v["launches"] // K,
                        "us_per_step": round(v["ms"] * 1e3 / K, 2),
                        "GB_s": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1),
                        "hbm_frac": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "TFLOP_s": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 2),
                        "mfma_frac": (round(v["flops"] / (v["ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
                                      if k.startswith("gemm") else None)}
                    for k, v in sorted(per_class.items(), key=lambda kv: -kv[1]["ms"])},
        "prefill": prefill,
        "aggregate": agg,
        "attn_standalone": attn,
        "counters": counters,
        "versus_photon": versus,
        "per_config": per_config,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
