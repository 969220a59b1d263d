"""ctypes binding of the PHOTON C ABI (include/photon.h).

Argument marshalling only: every step of prefill and decoding runs in the
HIP kernels of libphoton.so.  PyTorch supplies device memory and the stream.
The library must have been built (``__graft_entry__.build()``); importing
this module without it raises, there is no fallback path.
"""
import ctypes
import os

import numpy as np
# torch first: it loads its own HIP runtime (SONAME libamdhip64.so.7), and
# libphoton.so must bind to that same runtime instance, not a second copy
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
# PHOTON_LIB selects another build of the same library (the host-sanitized
# one that the CPU tests load)
LIB_PATH = os.environ.get("PHOTON_LIB") or os.path.join(_PKG, "libphoton.so")

OK, EINVAL, ESHAPE, ECAPACITY, ESTATE, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
RECGEN, HIERGEN = 0, 1
_MODES = {"recgen": RECGEN, "hiergen": HIERGEN}
ATTN_GLOBAL, ATTN_CHUNK, ATTN_PREFILL = 0, 1, 2
_ATTN = {"global": ATTN_GLOBAL, "chunk": ATTN_CHUNK, "prefill": ATTN_PREFILL}


class PhotonError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"photon status {status}: {msg}")
        self.status = status


MAX_LEVELS = 4   # PHOTON_MAX_LEVELS


class Config(ctypes.Structure):
    _fields_ = [("n_levels", ctypes.c_int32), ("chunk", ctypes.c_int32 * MAX_LEVELS),
                ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("mlp_mult", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_top", ctypes.c_int32), ("n_enc1", ctypes.c_int32),
                ("n_dec1", ctypes.c_int32), ("n_dec0", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float),
                ("n_enc_hi", ctypes.c_int32 * (MAX_LEVELS - 2)),
                ("n_dec_hi", ctypes.c_int32 * (MAX_LEVELS - 2))]


class VanillaConfig_(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("mlp_mult", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("norm_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("steps", ctypes.c_int32)]


class KvReport(ctypes.Structure):
    _fields_ = [("top_len", ctypes.c_int64), ("lower_len", ctypes.c_int64),
                ("top_kv", ctypes.c_uint64), ("lower_kv", ctypes.c_uint64),
                ("dec_kv", ctypes.c_uint64), ("state", ctypes.c_uint64),
                ("decode_scratch", ctypes.c_uint64),
                ("workspace_total", ctypes.c_uint64),
                ("weights_decode", ctypes.c_uint64),
                ("weights_prefill_only", ctypes.c_uint64),
                ("off_top_kv", ctypes.c_uint64), ("off_lower_kv", ctypes.c_uint64),
                ("off_dec_kv", ctypes.c_uint64), ("off_state", ctypes.c_uint64),
                ("off_scratch", ctypes.c_uint64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class TensorInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("blob", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("offset", ctypes.c_uint64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class Sampling_(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32), ("seed", ctypes.c_uint64)]


def make_sampling(temperature, top_k=0, seed=0):
    return Sampling_(float(temperature), int(top_k), int(seed) & 0xFFFFFFFFFFFFFFFF)


class TraceStat(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int64), ("ms", ctypes.c_double),
                ("bytes", ctypes.c_double), ("flops", ctypes.c_double)]


# kernel classes of photon_trace_enable, in photon_kernel_class order
KERNEL_CLASSES = ["gemm_qkv", "gemm_o", "gemm_up", "gemm_down", "gemm_head",
                  "gemm_conv", "gemm_chunk", "attn_top", "attn_chunk",
                  "attn_prefill", "norm", "rope_kv", "embed", "argmax", "sample"]

EXPORTS = ["photon_kv_bytes", "photon_prefill_scratch_bytes",
           "photon_weight_layout", "photon_weight_tensor", "photon_open",
           "photon_release_prefill_weights", "photon_close",
           "photon_last_error", "photon_prefill", "photon_decode_chunk",
           "photon_position", "photon_set_position", "photon_use_graphs",
           "photon_trace_enable", "photon_trace_read",
           "photon_attention_scratch_bytes", "photon_attention", "photon_attention_noalloc",
           "photon_vanilla_kv_bytes", "photon_vanilla_prefill_scratch_bytes",
           "photon_vanilla_weight_layout", "photon_vanilla_weight_tensor",
           "photon_vanilla_open", "photon_vanilla_prefill", "photon_vanilla_decode",
           "photon_sampling_bytes", "photon_set_sampling", "photon_decode_chunk_lp", "photon_sample",
           "photon_aggregate", "photon_consistency"]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P, V = ctypes.POINTER, ctypes.c_void_p
    i32, i64, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    sig = {
        "photon_kv_bytes": [P(Config), i32, i64, i32, P(KvReport)],
        "photon_prefill_scratch_bytes": [P(Config), i32, i32, i32, P(u64)],
        "photon_weight_layout": [P(Config), P(u64), P(u64), P(i32)],
        "photon_weight_tensor": [P(Config), i32, P(TensorInfo)],
        "photon_open": [P(Config), V, V, P(V)],
        "photon_release_prefill_weights": [V],
        "photon_close": [V],
        "photon_last_error": [],
        "photon_prefill": [V, i32, V, u64, V, u64, V, i32, i32, i64, V],
        "photon_decode_chunk": [V, V, V, V],
        "photon_position": [V, P(i64), P(i64)],
        "photon_set_position": [V, i64, V],
        "photon_use_graphs": [V, i32],
        "photon_trace_enable": [V, ctypes.c_uint32],
        "photon_trace_read": [V, P(TraceStat)],
        "photon_attention_scratch_bytes": [i32, i32, i32, i32, i32, i32, P(u64)],
        "photon_attention": [i32, i32, V, V, V, V, i32, i32, i32, i32, i32, i32, V, u64, V],
        "photon_attention_noalloc": [i32, i32, V, V, V, V, i32, i32, i32, i32, i32, i32, V],
        "photon_vanilla_kv_bytes": [P(VanillaConfig_), i32, i64, P(KvReport)],
        "photon_vanilla_prefill_scratch_bytes": [P(VanillaConfig_), i32, i32, P(u64)],
        "photon_vanilla_weight_layout": [P(VanillaConfig_), P(u64), P(i32)],
        "photon_vanilla_weight_tensor": [P(VanillaConfig_), i32, P(TensorInfo)],
        "photon_vanilla_open": [P(VanillaConfig_), V, P(V)],
        "photon_vanilla_prefill": [V, V, u64, V, u64, V, i32, i32, i64, V],
        "photon_vanilla_decode": [V, V, V, V],
        "photon_sampling_bytes": [P(Config), i32, P(u64)],
        "photon_set_sampling": [V, P(Sampling_), V, u64],
        "photon_decode_chunk_lp": [V, V, V, V, V],
        "photon_sample": [i32, i32, V, i64, P(Sampling_), V, V, V, V, V],
        "photon_aggregate": [i32, i32, i32, V, i64, V, i64, i32, i32, V, V, V, V, V],
        "photon_consistency": [V, V, V, V, V],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "photon_last_error" else ctypes.c_int
    return lib


_lib = _load()


def _check(status):
    if status != OK:
        raise PhotonError(status, _lib.photon_last_error().decode())


def make_config(cfg):
    """photon_config from a photon_inputs.PhotonConfig."""
    c = Config()
    if len(cfg.chunk) > MAX_LEVELS:
        raise ValueError(f"at most {MAX_LEVELS} levels")
    c.n_levels = len(cfg.chunk)
    for i, C in enumerate(cfg.chunk):
        c.chunk[i] = C
    c.d_model, c.n_heads, c.mlp_mult, c.vocab = cfg.d_model, cfg.n_heads, cfg.mlp_mult, cfg.vocab
    c.n_top, c.n_enc1, c.n_dec1, c.n_dec0 = cfg.n_top, cfg.n_enc1, cfg.n_dec1, cfg.n_dec0
    for i, (ne, nd) in enumerate(zip(cfg.n_enc_hi, cfg.n_dec_hi)):
        c.n_enc_hi[i], c.n_dec_hi[i] = ne, nd
    c.dtype = BF16 if cfg.dtype == "bf16" else F32
    c.norm_eps, c.rope_theta = cfg.norm_eps, cfg.rope_theta
    return c


def kv_bytes(cfg, batch, tokens, mode="recgen"):
    rep = KvReport()
    _check(_lib.photon_kv_bytes(ctypes.byref(make_config(cfg)), batch, tokens,
                                _MODES[mode], ctypes.byref(rep)))
    return rep.as_dict()


def prefill_scratch_bytes(cfg, batch, prompt_len, mode="recgen"):
    out = ctypes.c_uint64()
    _check(_lib.photon_prefill_scratch_bytes(ctypes.byref(make_config(cfg)), batch,
                                             prompt_len, _MODES[mode], ctypes.byref(out)))
    return out.value


def weight_layout(cfg):
    c = make_config(cfg)
    dec, pre, n = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_int32()
    _check(_lib.photon_weight_layout(ctypes.byref(c), ctypes.byref(dec), ctypes.byref(pre), ctypes.byref(n)))
    tensors = []
    for i in range(n.value):
        t = TensorInfo()
        _check(_lib.photon_weight_tensor(ctypes.byref(c), i, ctypes.byref(t)))
        tensors.append({"name": t.name.decode(), "blob": t.blob, "dtype": t.dtype,
                        "offset": t.offset, "rows": t.rows, "cols": t.cols})
    return dec.value, pre.value, tensors


def make_vanilla_config(cfg, steps):
    """photon_vanilla_config from a photon_inputs.VanillaConfig; `steps`
    tokens per sequence per decode call."""
    c = VanillaConfig_()
    c.d_model, c.n_heads, c.mlp_mult, c.vocab = cfg.d_model, cfg.n_heads, cfg.mlp_mult, cfg.vocab
    c.n_layers = cfg.n_layers
    c.dtype = BF16 if cfg.dtype == "bf16" else F32
    c.norm_eps, c.rope_theta = cfg.norm_eps, cfg.rope_theta
    c.steps = steps
    return c


def vanilla_kv_bytes(cfg, steps, batch, tokens):
    rep = KvReport()
    _check(_lib.photon_vanilla_kv_bytes(ctypes.byref(make_vanilla_config(cfg, steps)), batch, tokens,
                                        ctypes.byref(rep)))
    return rep.as_dict()


def _stream_handle(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def sampling_bytes(cfg, batch):
    out = ctypes.c_uint64()
    c = make_config(cfg)
    _check(_lib.photon_sampling_bytes(ctypes.byref(c), batch, ctypes.byref(out)))
    return out.value


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def sample(logits, temperature, top_k, seed, seq, pos, logprobs=True):
    """photon_sample on torch tensors: logits [rows, V] float32 (row stride
    logits.stride(0)), seq and pos int32 [rows]; returns (ids int32 [rows],
    log-likelihoods float32 [rows] or None)."""
    rows, V = logits.shape
    assert logits.dtype == torch.float32 and logits.stride(1) == 1
    seq = seq.to(device=logits.device, dtype=torch.int32).contiguous()
    pos = pos.to(device=logits.device, dtype=torch.int32).contiguous()
    ids = torch.empty(rows, dtype=torch.int32, device=logits.device)
    lp = torch.empty(rows, dtype=torch.float32, device=logits.device) if logprobs else None
    sp = make_sampling(temperature, top_k, seed)
    _check(_lib.photon_sample(rows, V, _ptr(logits), logits.stride(0), ctypes.byref(sp), _ptr(seq), _ptr(pos),
                              _ptr(ids), _ptr(lp), _stream_handle(torch)))
    return ids, lp


def aggregate(tokens, logprobs, group, span=None, n_tok=None):
    """photon_aggregate on torch tensors tokens int32 [B, N], logprobs
    float32 [B, N]; returns (best, major, votes, scores)."""
    B, N = tokens.shape
    n_tok = N if n_tok is None else n_tok
    b0, b1 = (0, N) if span is None else span
    assert tokens.dtype == torch.int32 and tokens.stride(1) == 1 and logprobs.stride(1) == 1
    G = (B + group - 1) // group
    dev = tokens.device
    best = torch.empty(G, dtype=torch.int32, device=dev)
    major = torch.empty(G, dtype=torch.int32, device=dev)
    votes = torch.empty(G, dtype=torch.int32, device=dev)
    scores = torch.empty(B, dtype=torch.float32, device=dev)
    _check(_lib.photon_aggregate(B, group, n_tok, _ptr(tokens), tokens.stride(0), _ptr(logprobs), logprobs.stride(0),
                                 b0, b1, _ptr(best), _ptr(major), _ptr(votes), _ptr(scores), _stream_handle(torch)))
    return best, major, votes, scores


def attention_scratch_bytes(kind, groups, heads, head_dim, queries, cap):
    out = ctypes.c_uint64()
    _check(_lib.photon_attention_scratch_bytes(_ATTN[kind], groups, heads, head_dim, queries, cap,
                                               ctypes.byref(out)))
    return out.value


class Attention:
    """photon_attention on torch tensors: q [G*Q, H*hd] float32 and K, V
    [G, H, cap, hd] (float32 or bfloat16) on the current GPU; the scratch
    for split partials is allocated once per shape."""

    def __init__(self, kind, groups, heads, head_dim, queries, cap):
        self.kind, self.shape = kind, (groups, heads, head_dim, queries, cap)
        n = attention_scratch_bytes(kind, groups, heads, head_dim, queries, cap)
        self.scratch = torch.empty(max(n, 1) + 256, dtype=torch.uint8, device="cuda")
        off = (-self.scratch.data_ptr()) % 256
        self.scratch_ptr, self.scratch_bytes = self.scratch.data_ptr() + off, n

    def __call__(self, q, K, V, out, keys):
        G, H, hd, Q, cap = self.shape
        dt = BF16 if K.dtype == torch.bfloat16 else F32
        assert q.dtype == torch.float32 and tuple(q.shape) == (G * Q, H * hd) and q.is_contiguous()
        assert tuple(K.shape) == (G, H, cap, hd) and K.shape == V.shape and K.dtype == V.dtype
        assert K.is_contiguous() and V.is_contiguous() and out.is_contiguous()
        assert out.dtype == K.dtype and tuple(out.shape) == (G * Q, H * hd)
        _check(_lib.photon_attention(_ATTN[self.kind], dt, ctypes.c_void_p(q.data_ptr()),
                                     ctypes.c_void_p(K.data_ptr()), ctypes.c_void_p(V.data_ptr()),
                                     ctypes.c_void_p(out.data_ptr()), G, H, hd, Q, keys, cap,
                                     ctypes.c_void_p(self.scratch_ptr), self.scratch_bytes,
                                     _stream_handle(torch)))
        return out


NOALLOC_SCRATCH_BYTES = 8 << 20   # PHOTON_NOALLOC_SCRATCH_BYTES


def attention_noalloc(kind, q, K, V, out, keys, queries=1):
    """photon_attention_noalloc on torch tensors laid out as for Attention
    (q [G*Q, H*hd] float32, K and V [G, H, cap, hd], out like q in K's
    dtype); the split partials live in the library's built-in device array."""
    G, H, cap, hd = K.shape
    dt = BF16 if K.dtype == torch.bfloat16 else F32
    assert q.dtype == torch.float32 and tuple(q.shape) == (G * queries, H * hd) and q.is_contiguous()
    assert K.shape == V.shape and K.dtype == V.dtype and K.is_contiguous() and V.is_contiguous()
    assert out.dtype == K.dtype and tuple(out.shape) == (G * queries, H * hd) and out.is_contiguous()
    _check(_lib.photon_attention_noalloc(_ATTN[kind], dt, ctypes.c_void_p(q.data_ptr()),
                                         ctypes.c_void_p(K.data_ptr()), ctypes.c_void_p(V.data_ptr()),
                                         ctypes.c_void_p(out.data_ptr()), G, H, hd, queries, keys, cap,
                                         _stream_handle(torch)))
    return out


class Photon:
    """One model on the current GPU: packed weight blobs plus a context.

    weights: mapping name -> float32 numpy array (bf16-exact for bf16
    models), as produced by photon_inputs.gen_weights.
    """

    def __init__(self, cfg, weights, device="cuda"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.c = make_config(cfg)
        dec, pre, tensors = weight_layout(cfg)
        blobs = [torch.zeros(dec, dtype=torch.uint8, device=self.device),
                 torch.zeros(max(pre, 256), dtype=torch.uint8, device=self.device)]
        for t in tensors:
            w = np.ascontiguousarray(weights[t["name"]], dtype=np.float32)
            assert w.size == t["rows"] * t["cols"], t["name"]
            src = torch.from_numpy(w.reshape(-1)).to(self.device)
            if t["dtype"] == BF16:
                src = src.to(torch.bfloat16)
            raw = src.view(torch.uint8)
            blobs[t["blob"]][t["offset"]:t["offset"] + raw.numel()].copy_(raw)
        self.w_decode, self.w_prefill = blobs
        self.weight_bytes = {"decode": dec, "prefill_only": pre}
        ctx = ctypes.c_void_p()
        _check(_lib.photon_open(ctypes.byref(self.c), ctypes.c_void_p(self.w_decode.data_ptr()),
                                ctypes.c_void_p(self.w_prefill.data_ptr()), ctypes.byref(ctx)))
        self.ctx = ctx
        self.workspace = None
        self.mode = None
        self.batch = None

    def close(self):
        if self.ctx:
            _lib.photon_close(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def release_prefill_weights(self):
        """Drop the Chunker^1 / level-1 encoder blob (RecGen never uses it
        after prefill)."""
        _check(_lib.photon_release_prefill_weights(self.ctx))
        self.w_prefill = None

    def report(self, batch, tokens, mode="recgen"):
        return kv_bytes(self.cfg, batch, tokens, mode)

    def prefill(self, prompt, max_tokens, mode="recgen"):
        """prompt: int32 CUDA tensor [B, P]."""
        torch = self.torch
        B, P = prompt.shape
        rep = kv_bytes(self.cfg, B, max_tokens, mode)
        if self.workspace is None or self.workspace.numel() < rep["workspace_total"]:
            self.workspace = torch.empty(rep["workspace_total"], dtype=torch.uint8, device=self.device)
        scratch_n = prefill_scratch_bytes(self.cfg, B, P, mode)
        scratch = torch.empty(scratch_n, dtype=torch.uint8, device=self.device)
        prompt = prompt.to(device=self.device, dtype=torch.int32).contiguous()
        _check(_lib.photon_prefill(self.ctx, _MODES[mode], ctypes.c_void_p(self.workspace.data_ptr()),
                                   self.workspace.numel(), ctypes.c_void_p(scratch.data_ptr()), scratch_n,
                                   ctypes.c_void_p(prompt.data_ptr()), B, P, max_tokens,
                                   _stream_handle(torch)))
        self._scratch_hold = (scratch, prompt)   # freed at the next prefill
        self.report_ = rep
        self.mode = mode
        self.batch = B

    def set_sampling(self, temperature=None, top_k=0, seed=0, batch=None):
        """Sampling decode from the next chunk on (temperature None: greedy).
        The sampling workspace is sized for `batch` (default: the prefilled
        batch)."""
        torch = self.torch
        if temperature is None:
            _check(_lib.photon_set_sampling(self.ctx, None, None, 0))
            self.sampling_ws = None
            return
        batch = batch or self.batch
        if batch is None:
            raise ValueError("set_sampling needs a batch size before the first prefill")
        n = sampling_bytes(self.cfg, batch)
        ws = torch.empty(n + 256, dtype=torch.uint8, device=self.device)
        off = (-ws.data_ptr()) % 256
        sp = make_sampling(temperature, top_k, seed)
        _check(_lib.photon_set_sampling(self.ctx, ctypes.byref(sp), ctypes.c_void_p(ws.data_ptr() + off), n))
        self.sampling_ws = ws

    def decode_chunk(self, tokens_out, logits_out=None, logprobs_out=None):
        """tokens_out: int32 CUDA [B, S]; logits_out: float32 [B, S, V] or
        None; logprobs_out: float32 [B, S] or None (sampling only)."""
        _check(_lib.photon_decode_chunk_lp(self.ctx, _ptr(tokens_out), _ptr(logits_out), _ptr(logprobs_out),
                                           _stream_handle(self.torch)))

    def consistency(self, copies=False):
        """The Eq. 1 diagnostic of the last HierGen chunk: [B, C_L] float32
        (and, with copies, A-hat_i and A_i as [B, C_L, d] storage-dtype
        tensors), at the level under the top."""
        torch = self.torch
        B, C2, d = self.batch, self.cfg.chunk[-1], self.cfg.d_model
        dist = torch.empty((B, C2), dtype=torch.float32, device=self.device)
        dt = torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32
        ah = torch.empty((B, C2, d), dtype=dt, device=self.device) if copies else None
        a = torch.empty((B, C2, d), dtype=dt, device=self.device) if copies else None
        _check(_lib.photon_consistency(self.ctx, _ptr(dist), _ptr(ah), _ptr(a), _stream_handle(torch)))
        return (dist, ah, a) if copies else dist

    def position(self):
        a, b = ctypes.c_int64(), ctypes.c_int64()
        _check(_lib.photon_position(self.ctx, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def use_graphs(self, enable=True):
        _check(_lib.photon_use_graphs(self.ctx, 1 if enable else 0))

    def set_position(self, tokens):
        _check(_lib.photon_set_position(self.ctx, tokens, _stream_handle(self.torch)))

    def state_snapshot(self):
        """Copy of the h region (enough, with set_position, to rewind)."""
        return self.h_state().clone()

    def state_restore(self, snap, tokens):
        self.h_state().copy_(snap)
        self.set_position(tokens)

    def trace_enable(self, classes=None):
        """classes: iterable of KERNEL_CLASSES names (None = all, [] = off)."""
        names = KERNEL_CLASSES if classes is None else list(classes)
        mask = 0
        for n in names:
            mask |= 1 << KERNEL_CLASSES.index(n)
        _check(_lib.photon_trace_enable(self.ctx, mask))

    def trace_read(self):
        out = (TraceStat * len(KERNEL_CLASSES))()
        _check(_lib.photon_trace_read(self.ctx, out))
        return {n: {"launches": out[i].launches, "ms": out[i].ms, "bytes": out[i].bytes,
                    "flops": out[i].flops} for i, n in enumerate(KERNEL_CLASSES) if out[i].launches}

    def generate(self, prompt, new_tokens, mode="recgen", logits=False, max_tokens=None, sampling=None,
                 logprobs=False):
        """Prefill, then the chunks up to P + new_tokens (a multiple of S;
        with a ragged prompt the first chunk's leading P mod S tokens are the
        prompt's tail and are left out of the result).  sampling: None
        (greedy) or dict(temperature, top_k, seed).  Returns (tokens [B, N],
        logits [B, N, V] or None), plus the log-likelihoods [B, N] when
        logprobs (sampling only)."""
        torch = self.torch
        B, P = prompt.shape
        S = self.cfg.S
        if (P + new_tokens) % S:
            raise ValueError("prompt + new tokens must end on a multiple of S")
        r = P % S
        chunks = (P + new_tokens) // S - P // S
        self.prefill(prompt, max_tokens or P + new_tokens, mode)
        if sampling is not None:
            self.set_sampling(sampling["temperature"], sampling.get("top_k", 0), sampling.get("seed", 0), B)
        else:
            self.set_sampling(None)
        toks = torch.empty((chunks, B, S), dtype=torch.int32, device=self.device)
        lg = torch.empty((chunks, B, S, self.cfg.vocab), dtype=torch.float32,
                         device=self.device) if logits else None
        lp = torch.empty((chunks, B, S), dtype=torch.float32, device=self.device) if logprobs else None
        for c in range(chunks):
            self.decode_chunk(toks[c], lg[c] if logits else None, lp[c] if logprobs else None)
        toks = toks.permute(1, 0, 2).reshape(B, chunks * S)[:, r:]
        if logits:
            lg = lg.permute(1, 0, 2, 3).reshape(B, chunks * S, self.cfg.vocab)[:, r:]
        if logprobs:
            return toks, lg, lp.permute(1, 0, 2).reshape(B, chunks * S)[:, r:]
        return toks, lg

    # ---- views into the workspace (tests read the caches directly) ----
    def top_kv(self):
        """Top-level K/V as a tensor [n_top, 2, B, H, top_cap, hd] (storage dtype)."""
        torch = self.torch
        rep = self.report_
        cfg = self.cfg
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        eb = 2 if cfg.dtype == "bf16" else 4
        n = rep["top_kv"] // eb
        raw = self.workspace[rep["off_top_kv"]:rep["off_top_kv"] + rep["top_kv"]]
        return raw.view(dt)[:n].view(cfg.n_top, 2, self.batch, cfg.n_heads, rep["top_len"], cfg.head_dim)

    def lower_kv(self):
        """HierGen's level-1 encoder K/V as a tensor [n_enc1, 2, B, H, lower_cap, hd]
        (storage dtype); the first region of the lower-level K/V."""
        torch = self.torch
        rep = self.report_
        cfg = self.cfg
        if not rep["lower_kv"]:
            raise ValueError("no lower-level K/V is kept (RecGen)")
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        eb = 2 if cfg.dtype == "bf16" else 4
        cap = rep["lower_len"]
        n = cfg.n_enc1 * 2 * self.batch * cfg.n_heads * cap * cfg.head_dim
        raw = self.workspace[rep["off_lower_kv"]:rep["off_lower_kv"] + n * eb]
        return raw.view(dt).view(cfg.n_enc1, 2, self.batch, cfg.n_heads, cap, cfg.head_dim)

    def h_state(self):
        torch = self.torch
        cfg = self.cfg
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        eb = 2 if cfg.dtype == "bf16" else 4
        off = self.report_["off_state"]
        return self.workspace[off:off + self.batch * cfg.d_model * eb].view(dt).view(self.batch, cfg.d_model)


class Vanilla(Photon):
    """The flat Transformer baseline on the current GPU (one weight blob and
    a context from photon_vanilla_open); decode calls emit `steps` tokens per
    sequence.  Shares Photon's position, graph, tracing and snapshot
    helpers (the state region holds the last position's stack output)."""

    def __init__(self, cfg, weights, steps, device="cuda"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.steps = steps
        self.device = torch.device(device)
        self.c = make_vanilla_config(cfg, steps)
        nbytes, n = ctypes.c_uint64(), ctypes.c_int32()
        _check(_lib.photon_vanilla_weight_layout(ctypes.byref(self.c), ctypes.byref(nbytes), ctypes.byref(n)))
        blob = torch.zeros(nbytes.value, dtype=torch.uint8, device=self.device)
        for i in range(n.value):
            t = TensorInfo()
            _check(_lib.photon_vanilla_weight_tensor(ctypes.byref(self.c), i, ctypes.byref(t)))
            w = np.ascontiguousarray(weights[t.name.decode()], dtype=np.float32)
            assert w.size == t.rows * t.cols, t.name
            src = torch.from_numpy(w.reshape(-1)).to(self.device)
            if t.dtype == BF16:
                src = src.to(torch.bfloat16)
            raw = src.view(torch.uint8)
            blob[t.offset:t.offset + raw.numel()].copy_(raw)
        self.w_decode, self.w_prefill = blob, None
        self.weight_bytes = {"decode": nbytes.value, "prefill_only": 0}
        ctx = ctypes.c_void_p()
        _check(_lib.photon_vanilla_open(ctypes.byref(self.c), ctypes.c_void_p(blob.data_ptr()), ctypes.byref(ctx)))
        self.ctx = ctx
        self.workspace = None
        self.mode = "vanilla"
        self.batch = None

    def release_prefill_weights(self):
        pass

    def report(self, batch, tokens, mode=None):
        return vanilla_kv_bytes(self.cfg, self.steps, batch, tokens)

    def prefill(self, prompt, max_tokens, mode=None):
        torch = self.torch
        B, P = prompt.shape
        rep = self.report(B, max_tokens)
        if self.workspace is None or self.workspace.numel() < rep["workspace_total"]:
            self.workspace = torch.empty(rep["workspace_total"], dtype=torch.uint8, device=self.device)
        n = ctypes.c_uint64()
        _check(_lib.photon_vanilla_prefill_scratch_bytes(ctypes.byref(self.c), B, P, ctypes.byref(n)))
        scratch = torch.empty(n.value, dtype=torch.uint8, device=self.device)
        prompt = prompt.to(device=self.device, dtype=torch.int32).contiguous()
        _check(_lib.photon_vanilla_prefill(self.ctx, ctypes.c_void_p(self.workspace.data_ptr()),
                                           self.workspace.numel(), ctypes.c_void_p(scratch.data_ptr()), n.value,
                                           ctypes.c_void_p(prompt.data_ptr()), B, P, max_tokens,
                                           _stream_handle(torch)))
        self._scratch_hold = (scratch, prompt)
        self.report_ = rep
        self.batch = B

    def decode_chunk(self, tokens_out, logits_out=None):
        """tokens_out: int32 CUDA [B, steps]; logits_out: float32 [B, steps, V] or None."""
        lp = ctypes.c_void_p(logits_out.data_ptr()) if logits_out is not None else None
        _check(_lib.photon_vanilla_decode(self.ctx, ctypes.c_void_p(tokens_out.data_ptr()), lp,
                                          _stream_handle(self.torch)))

    def generate(self, prompt, new_tokens, mode=None, logits=False, max_tokens=None):
        torch = self.torch
        B, P = prompt.shape
        S = self.steps
        if new_tokens % S:
            raise ValueError("new_tokens must be a multiple of steps")
        self.prefill(prompt, max_tokens or P + new_tokens)
        toks = torch.empty((new_tokens // S, B, S), dtype=torch.int32, device=self.device)
        lg = torch.empty((new_tokens // S, B, S, self.cfg.vocab), dtype=torch.float32,
                         device=self.device) if logits else None
        for c in range(new_tokens // S):
            self.decode_chunk(toks[c], lg[c] if logits else None)
        toks = toks.permute(1, 0, 2).reshape(B, new_tokens)
        if logits:
            lg = lg.permute(1, 0, 2, 3).reshape(B, new_tokens, self.cfg.vocab)
        return toks, lg

    def kv(self):
        """Token K/V as a tensor [n_layers, 2, B, H, cap, hd] (storage dtype)."""
        torch = self.torch
        rep, cfg = self.report_, self.cfg
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        eb = 2 if cfg.dtype == "bf16" else 4
        raw = self.workspace[rep["off_top_kv"]:rep["off_top_kv"] + rep["top_kv"]]
        return raw.view(dt).view(cfg.n_layers, 2, self.batch, cfg.n_heads, rep["top_len"], cfg.head_dim)

