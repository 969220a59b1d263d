"""CPU oracle for PHOTON recursive generation (RecGen) and hierarchical
generation (HierGen).  TEST INFRASTRUCTURE ONLY: the product never imports,
calls or links this module; only the tests, the smoke check and the CPU
baseline leg of the benchmark do.

Plain, slow and meant to be read against the pages:
  [abstract]  PHOTON paper record (ACL 2026 long paper "PHOTON: Hierarchical
              Autoregressive Modeling for Lightspeed and Memory-Efficient
              Language Generation"), abstract.
  [modules]   PHOTON explainer (mokumoku.ipfde.com, Fujitsu PHOTON vertical
              scan), module table: Context Chunker / Encoder / Converter /
              Decoder rows, and the hierarchy-shape paragraph under it.
  [recgen]    same explainer, recursive-generation section: HierGen's three
              steps, RecGen's feedback of the bottleneck reconstruction,
              Theorem A.6 (paper appendix A), the cache-drop paragraph.
  [tpm]       same explainer, 1.2B decode-heavy table and the paragraph on
              why both factors come from the hierarchy (decoder span).

Every float is float64 (``compute="f64"``, the reference).  The same code
can run its arithmetic in float32 (``compute="f32"``): that is not a
reference but a second, equally valid implementation of the rounding
contract, used to measure how far two implementations that differ only in
accumulation precision drift apart (the contract's intrinsic noise).  For
bf16 models a rounding contract (round to the nearest bf16, ties to even) is
applied at fixed points; for fp32 models the rounding is the identity and
the oracle is plain fp64.  Contract:
  * weights are bf16 (they arrive bf16-exact from the input generator);
  * every activation operand of a matrix product is rounded: RMSNorm outputs,
    attention outputs, GELU outputs, stack outputs (A, A-hat, h, z) and the
    concatenated chunker inputs;
  * K and V are rounded when they enter a cache (K after RoPE); q is not;
  * accumulation, residual stream, norms, softmax, GELU and logits are not
    rounded.
Block internals are not given by the pages (they only say encoder and decoder
are Transformers inside); the reading taken is a pre-norm block with RMSNorm
(eps 1e-5), bias-free linears, multi-head attention with rotary position
embedding (theta 1e4, rotate-half) and a d -> 4d -> d GELU MLP.

Parity status: attention, RMSNorm, GELU, RoPE, chunker, converter, rounding
and the cache/equivalence invariants are pinned by the CPU tests.  The
overall model outputs are parity unpinned against the pages, which print no
model output: the block internals above are a reading, not a checked fact.
"""
import math
import numpy as np
from scipy.special import erf

from . import photon_sampling as S_

F64 = np.float64


# --------------------------------------------------------------------------
# rounding
# --------------------------------------------------------------------------
def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bf16 has an 8-bit significand and fp32's exponent range.  For |x| in
    [2^e, 2^(e+1)) the spacing is 2^(e-7); below 2^-126 (subnormal) it is the
    fixed 2^-133.  numpy's rint rounds half to even.  Values beyond the
    largest finite bf16 overflow to +-inf.
    """
    x = np.asarray(x, dtype=F64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    ax = np.abs(x[nz])
    e = np.floor(np.log2(ax))
    # guard floor(log2) at exact powers of two and rounding of log2
    e = np.where(2.0 ** e > ax, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= ax, e + 1, e)
    q = 2.0 ** np.maximum(e - 7, -133)
    r = np.rint(x[nz] / q) * q
    big = np.abs(r) > 3.3895313892515355e38
    r[big] = np.copysign(np.inf, r[big])
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


class Precision:
    """Applies the rounding contract: ``r`` is round_bf16 for bf16 models and
    the identity for fp32 models; values are held in the compute dtype."""

    def __init__(self, dtype, compute="f64"):
        assert dtype in ("f32", "bf16") and compute in ("f64", "f32")
        self.bf16 = dtype == "bf16"
        self.dt = np.float64 if compute == "f64" else np.float32

    def r(self, x):
        if self.bf16:
            return round_bf16(x).astype(self.dt)
        return np.asarray(x, dtype=self.dt)


# --------------------------------------------------------------------------
# primitives
# --------------------------------------------------------------------------
def rmsnorm(x, g, eps):
    """g * x / sqrt(mean(x^2) + eps) over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return g * (x / np.sqrt(ms + eps))


def gelu(z):
    """Exact GELU: z * Phi(z) = z/2 * (1 + erf(z / sqrt 2))."""
    return 0.5 * z * (1.0 + erf(z / z.dtype.type(math.sqrt(2.0))))


def rope_angles(pos, hd, theta):
    """phi[p, i] = pos[p] * theta^(-2i/hd), i < hd/2."""
    i = np.arange(hd // 2, dtype=F64)
    inv = theta ** (-2.0 * i / hd)
    return np.asarray(pos, dtype=F64)[:, None] * inv[None, :]


def rope(x, pos, theta):
    """Rotate-half rotary embedding over the full head dim.

    x: [..., T, H, hd]; pos: [T].  Pair (x_i, x_{i+hd/2}) is rotated by
    phi = pos * theta^(-2i/hd) (angles in float64, then the compute dtype).
    """
    hd = x.shape[-1]
    h = hd // 2
    phi = rope_angles(pos, hd, theta)[:, None, :]       # [T, 1, h]
    c, s = np.cos(phi).astype(x.dtype), np.sin(phi).astype(x.dtype)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention(q, k, v, n_prev):
    """Causal multi-head attention with a cache prefix.

    q: [B, Tq, H, hd] queries at absolute key indices n_prev .. n_prev+Tq-1;
    k, v: [B, n_prev+Tq, H, hd] (cache followed by the new keys).
    Query t sees keys 0 .. n_prev + t.  softmax(q k^T / sqrt(hd)) v.
    """
    B, Tq, H, hd = q.shape
    Tk = k.shape[1]
    s = np.einsum("bthe,bshe->bhts", q, k) / q.dtype.type(math.sqrt(hd))
    allowed = np.arange(Tk)[None, :] <= (n_prev + np.arange(Tq))[:, None]
    s = np.where(allowed[None, None], s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("bhts,bshe->bthe", p, v)


def linear(x, W):
    """y = x W^T, W[out, in], row by row over every leading axis of x (one
    library matrix product over the flattened rows)."""
    x = np.asarray(x)
    y = x.reshape(-1, x.shape[-1]) @ W.T
    return y.reshape(x.shape[:-1] + (W.shape[0],))


# --------------------------------------------------------------------------
# model pieces
# --------------------------------------------------------------------------
class Model:
    """Weights (float64) plus the precision contract for one configuration."""

    def __init__(self, cfg, weights, compute="f64"):
        self.cfg = cfg
        self.pr = Precision(cfg.dtype, compute)
        self.dt = self.pr.dt
        self.w = {k: np.asarray(v, dtype=self.dt) for k, v in weights.items()}

    def layers(self, prefix, n):
        return [{p: self.w[f"{prefix}.{l}.{p}"] for p in
                 ("g1", "Wq", "Wk", "Wv", "Wo", "g2", "W1", "W2")}
                for l in range(n)]

    # ---- a Transformer stack with optional per-layer KV cache ----
    def stack(self, prefix, n_layers, x, pos, cache=None, log=None):
        """Run a stack of pre-norm blocks then its final RMSNorm.

        x: [B, T, d] residual input (float); pos: [T] rotary positions of the
        new rows.  cache: None (no history, nothing kept) or a list with one
        entry per layer, each a dict {"k": [B, n, H, hd], "v": ...} holding
        the rounded K/V of earlier positions; the new K/V are appended in
        place.  Returns the rounded stack output r(RMSNorm(x; gf)).  ``log``,
        if given, is called with a short progress string after each layer.
        """
        cfg, r = self.cfg, self.pr.r
        B, T, d = x.shape
        H, hd = cfg.n_heads, cfg.head_dim
        x = np.array(x, dtype=self.dt)
        eps = self.dt(cfg.norm_eps)
        for l, L in enumerate(self.layers(prefix, n_layers)):
            a = r(rmsnorm(x, L["g1"], eps))
            q = linear(a, L["Wq"]).reshape(B, T, H, hd)
            k = linear(a, L["Wk"]).reshape(B, T, H, hd)
            v = linear(a, L["Wv"]).reshape(B, T, H, hd)
            q = rope(q, pos, cfg.rope_theta)
            k = r(rope(k, pos, cfg.rope_theta))
            v = r(v)
            if cache is not None:
                ent = cache[l]
                n_prev = ent["k"].shape[1]
                ent["k"] = np.concatenate([ent["k"], k], axis=1)
                ent["v"] = np.concatenate([ent["v"], v], axis=1)
                kk, vv = ent["k"], ent["v"]
            else:
                n_prev, kk, vv = 0, k, v
            o = r(attention(q, kk, vv, n_prev).reshape(B, T, d))
            x = x + linear(o, L["Wo"])
            a = r(rmsnorm(x, L["g2"], eps))
            hmid = r(gelu(linear(a, L["W1"])))
            x = x + linear(hmid, L["W2"])
            if log:
                log(f"{prefix} layer {l + 1}/{n_layers} done ({T} rows)")
        return r(rmsnorm(x, self.w[prefix + ".gf"], eps))

    def empty_cache(self, n_layers, B):
        H, hd = self.cfg.n_heads, self.cfg.head_dim
        return [{"k": np.zeros((B, 0, H, hd), self.dt),
                 "v": np.zeros((B, 0, H, hd), self.dt)}
                for _ in range(n_layers)]

    # ---- chunker and converter [modules] ----
    def chunker(self, name, z):
        """Context Chunker: concatenate C consecutive vectors in time order,
        then one bias-free linear C*d -> d.  z: [B, T, d], T % C == 0."""
        B, T, d = z.shape
        W = self.w[name]
        C = W.shape[1] // d
        cat = self.pr.r(z).reshape(B, T // C, C * d)
        return linear(cat, W)

    def converter(self, name, h):
        """Context Converter: transposed 1-D convolution with kernel = stride
        = C on a length-1 input, i.e. output j = W[j*d:(j+1)*d, :] h.
        h: [..., d] -> [..., C, d]."""
        W = self.w[name]
        d = h.shape[-1]
        C = W.shape[0] // d
        y = linear(self.pr.r(h), W)
        return y.reshape(h.shape[:-1] + (C, d))

    def embed(self, ids):
        return self.w["E"][np.asarray(ids)]

    def logits(self, z):
        return linear(self.pr.r(z), self.w["W_out"])


# --------------------------------------------------------------------------
# generation
# --------------------------------------------------------------------------
class State:
    """Decode state kept after prefill: the top-level K/V of every top layer,
    the latest top output h, the number of top states, and (HierGen only)
    the K/V of the encoder of every level below the top (``lower[l]``,
    l = 1 .. L-1)."""

    def __init__(self, top_cache, h_last, n_top_states, lower=None, tail=None):
        self.top = top_cache
        self.h = h_last
        self.top_len = n_top_states
        self.lower = lower
        self.tail = tail      # prompt tokens past the last whole chunk, or None

    @property
    def lvl1(self):
        return None if self.lower is None else self.lower[1]

    def copy(self):
        cp = lambda c: [{"k": e["k"].copy(), "v": e["v"].copy()} for e in c]
        low = None if self.lower is None else {l: cp(c) for l, c in self.lower.items()}
        return State(cp(self.top), self.h.copy(), self.top_len, low,
                     None if self.tail is None else self.tail.copy())


def state_from_arrays(model, seqs):
    """A State built from given cache contents instead of a prefill: seqs is
    a list (one entry per sequence, in batch order) of dicts with top_k,
    top_v [n_top, n, H, hd], h [d] and, to keep the lower encoders' caches
    (HierGen), low_k, low_v {l: [layers_l, n_l, H, hd]} -- the layout of
    photon_inputs.gen_decode_state.  The values are taken as they are (no
    rounding); the state sits at top position n (a prompt of n*S tokens)."""
    dt = model.dt
    n = seqs[0]["top_k"].shape[1]

    def cache(pick):
        layers = pick(seqs[0], "k").shape[0]
        return [{"k": np.stack([pick(s, "k")[i] for s in seqs]).astype(dt),
                 "v": np.stack([pick(s, "v")[i] for s in seqs]).astype(dt)} for i in range(layers)]

    top = cache(lambda s, kv: s["top_" + kv])
    h = np.stack([s["h"] for s in seqs]).astype(dt)
    lower = None
    if "low_k" in seqs[0]:
        lower = {l: cache(lambda s, kv, l=l: s["low_" + kv][l]) for l in range(1, model.cfg.L)}
    return State(top, h, n, lower)


def prefill(model, prompt, mode="recgen", log=None):
    """Bottom-up pass over the prompt [modules], [recgen].

    tokens -> embedding, then for every level l = 1 .. L-1: Chunker^l (C_l
    states of level l-1 -> 1) -> level-l encoder (causal, pos = level-l
    index); then Chunker^L -> top encoder (causal, pos = top index).  RecGen
    keeps only the top K/V and the last top output; HierGen also keeps the
    K/V of every lower encoder (the caches RecGen drops after prefill).
    """
    cfg = model.cfg
    prompt = np.asarray(prompt)
    B, P = prompt.shape
    S = cfg.S
    if P < S:
        raise ValueError("the prompt must hold at least one chunk of S tokens")
    # a ragged prompt: only whole chunks form top states; the r = P mod S
    # tail tokens open the next chunk, whose decoders take them as given
    # tokens (teacher forcing) before drawing the rest
    n = P // S
    tail = prompt[:, n * S:].copy() if P % S else None
    prompt = prompt[:, :n * S]
    P = n * S
    z = model.embed(prompt)
    lower = {}
    for l in range(1, cfg.L):
        u = model.chunker(f"W_ch{l}", z)
        lower[l] = model.empty_cache(cfg.enc_layers(l), B)
        z = model.stack(f"enc{l}", cfg.enc_layers(l), u, np.arange(P // cfg.span(l)), lower[l], log=log)
    u = model.chunker(f"W_ch{cfg.L}", z)
    ct = model.empty_cache(cfg.n_top, B)
    h = model.stack("top", cfg.n_top, u, np.arange(n), ct, log=log)
    return State(ct, h[:, -1], n, lower if mode == "hiergen" else None, tail)


def _decode_tokens(model, A_hat, forced_tokens=None, sampling=None, t0=0, tail=None):
    """Top-down token generation for one chunk [modules], [recgen].

    A_hat: [B, K, d] level-1 decoder outputs, K = S / C1 level-1 positions
    per chunk (C2 for two levels; written C2 below).  Each of the B*C2
    level-1 positions is expanded independently: Converter^1 gives C1 conditioning
    vectors c_0..c_{C1-1}; the token decoder runs C1 steps with attention
    confined to the sub-chunk (in-chunk KV, positions 0..j); step j's input
    is c_j plus the embedding of the previous token of the same sub-chunk
    (c_0 alone at j = 0); greedy argmax with the lowest index on ties.
    Returns (tokens [B, C2*C1], logits [B, C2*C1, V]) in k-major order,
    token index k*C1 + j.  forced_tokens [B, C2*C1] replaces the fed-back
    token (teacher forcing); the argmax is still reported.
    sampling = dict(temperature, top_k, seed) draws every token instead
    (photon_sampling.sample; sequence b, absolute position t0 + k*C1 + j)
    in place of the argmax.  tail [B, r] (the end of a ragged prompt) fixes
    the chunk's first r tokens: they are reported and fed as given.
    """
    cfg = model.cfg
    B, C2, d = A_hat.shape
    C1 = cfg.C1
    c0 = model.converter("W_cv1", A_hat)              # [B, C2, C1, d]
    rows = c0.reshape(B * C2, C1, d)
    cache = model.empty_cache(cfg.n_dec0, B * C2)
    toks = np.zeros((B * C2, C1), dtype=np.int64)
    logits = np.zeros((B * C2, C1, cfg.vocab), dtype=model.dt)
    forced = None if forced_tokens is None else \
        np.asarray(forced_tokens).reshape(B * C2, C1)
    given = np.full((B, C2 * C1), -1, dtype=np.int64)
    if tail is not None:
        given[:, :tail.shape[1]] = tail
    given = given.reshape(B * C2, C1)
    prev = None
    for j in range(C1):
        x = rows[:, j, :].copy()
        if j > 0:
            x = x + model.embed(prev)
        z = model.stack("dec0", cfg.n_dec0, x[:, None, :], np.array([j]), cache)
        lg = model.logits(z[:, 0, :])
        logits[:, j] = lg
        if sampling is None:
            toks[:, j] = np.argmax(lg, axis=-1)       # first maximum
        else:
            for r in range(B * C2):
                toks[r, j] = S_.sample(lg[r], sampling["temperature"], sampling["top_k"], sampling["seed"],
                                       r // C2, t0 + (r % C2) * C1 + j)
        fixed = given[:, j] >= 0
        toks[fixed, j] = given[fixed, j]
        prev = toks[:, j] if forced is None else np.where(fixed, given[:, j], forced[:, j])
    return toks.reshape(B, C2 * C1), logits.reshape(B, C2 * C1, cfg.vocab)


def _top_step(model, state, u):
    """One top-encoder step at position state.top_len: append the new K/V to
    the global cache, attend over all top states, return h."""
    h = model.stack("top", model.cfg.n_top, u[:, None, :],
                    np.array([state.top_len]), state.top)
    state.top_len += 1
    state.h = h[:, 0]
    return state.h


def decode_down(model, h):
    """The decoders of one chunk below the top [modules], [recgen].

    Converter^L expands h [B, d] into C_L conditioning vectors and the
    level-(L-1) decoder (causal inside the chunk, pos 0..C_L-1, no cache
    kept) gives the bottleneck reconstruction A-hat [B, C_L, d]; then for
    l = L-1 down to 2 every level-l vector is expanded the same way by
    Converter^l and the level-(l-1) decoder, each group of C_l positions on
    its own.  Returns (A-hat at level L-1, the level-1 outputs
    [B, S/C1, d], in time order); for two levels both are the level-1
    decoder's output."""
    cfg = model.cfg
    L, B, d = cfg.L, h.shape[0], cfg.d_model
    c = model.converter(f"W_cv{L}", h)                # [B, C_L, d]
    top_hat = model.stack(f"dec{L - 1}", cfg.dec_layers(L - 1), c, np.arange(cfg.chunk[L - 1]), None)
    z = top_hat
    for l in range(L - 1, 1, -1):
        m, C = z.shape[1], cfg.chunk[l - 1]
        c = model.converter(f"W_cv{l}", z).reshape(B * m, C, d)
        z = model.stack(f"dec{l - 1}", cfg.dec_layers(l - 1), c, np.arange(C), None).reshape(B, m * C, d)
    return top_hat, z


def decode_chunk(model, state, mode="recgen", forced_tokens=None,
                 forced_u=None, sampling=None):
    """Generate the next chunk of S = C1*...*CL tokens; updates ``state``.

    The decoders below the top (decode_down) turn h_{i-1} into the
    bottleneck reconstruction A-hat_i (level L-1) and the level-1 outputs,
    from which the tokens are written (_decode_tokens).
      RecGen  [recgen]: u_i = Chunker^L(A-hat_i), fed straight to the top.
      HierGen [recgen]: the chunk's tokens are re-encoded bottom-up:
              embedding, then for l = 1 .. L-1 Chunker^l and one level-l
              encoder step over the chunk's S/span(l) new level-l positions
              with the kept level-l cache, ending in A_i (level L-1) ->
              u_i = Chunker^L(A_i).
    forced_u replaces u_i (used to force the premise of Theorem A.6).
    sampling (dict(temperature, top_k, seed)) draws the tokens instead of
    the argmax; the chunk's first token is at absolute position
    top_len * S.
    Returns a dict with tokens, logits, A_hat, u (and A for HierGen).
    """
    cfg = model.cfg
    A_hat, A_hat1 = decode_down(model, state.h)
    tail, state.tail = state.tail, None
    toks, logits = _decode_tokens(model, A_hat1, forced_tokens, sampling, state.top_len * cfg.S, tail)
    out = {"tokens": toks, "logits": logits, "A_hat": A_hat}
    if mode == "recgen":
        u = model.chunker(f"W_ch{cfg.L}", A_hat)[:, 0]
    else:
        fed = toks if forced_tokens is None else np.asarray(forced_tokens)
        z = model.embed(fed)                           # [B, S, d]
        for l in range(1, cfg.L):
            u_l = model.chunker(f"W_ch{l}", z)        # [B, S/span(l), d]
            m = cfg.S // cfg.span(l)
            z = model.stack(f"enc{l}", cfg.enc_layers(l), u_l, state.top_len * m + np.arange(m),
                            state.lower[l])
        out["A"] = z
        u = model.chunker(f"W_ch{cfg.L}", z)[:, 0]
    if forced_u is not None:
        u = np.asarray(forced_u, dtype=model.dt)
    out["u"] = u
    out["h"] = _top_step(model, state, u)
    return out


def consistency(A_hat, A):
    """The recursive loss of the pages (Eq. 1) as a diagnostic [recgen]: the
    cosine distance 1 - cos(A-hat_i[k], A_i[k]) between the decoder's
    reconstruction and the encoder's summary at each of the C_L positions
    of a chunk at level L-1 (the level the top reads: level 1 for two
    levels), on the values as stored (post-norm, rounded).  A_hat, A:
    [B, C_L, d]; returns [B, C_L] float64."""
    a = np.asarray(A_hat, dtype=F64)
    e = np.asarray(A, dtype=F64)
    dot = (a * e).sum(axis=-1)
    return 1.0 - dot / (np.sqrt((a * a).sum(axis=-1)) * np.sqrt((e * e).sum(axis=-1)))


def generate(model, prompt, new_tokens, mode="recgen", forced_tokens=None, log=None, sampling=None):
    """Prefill then the decode chunks up to P + new_tokens (which must end
    on a chunk boundary).  Returns (tokens [B, N], logits [B, N, V], final
    state, per-chunk records) for the N new tokens: with a ragged prompt the
    first chunk's leading r tokens are the prompt's tail and are left out.
    ``log`` receives progress strings (per prefill layer and per decoded
    chunk)."""
    S = model.cfg.S
    P = np.asarray(prompt).shape[1]
    if (P + new_tokens) % S:
        raise ValueError("prompt + new tokens must end on a multiple of S")
    st = prefill(model, prompt, mode, log=log)
    r = P % S
    chunks = (P + new_tokens) // S - P // S
    if forced_tokens is not None and r:
        forced_tokens = np.concatenate([np.asarray(prompt)[:, P - r:], np.asarray(forced_tokens)], 1)
    toks, lg, recs = [], [], []
    for c in range(chunks):
        ft = None if forced_tokens is None else \
            np.asarray(forced_tokens)[:, c * S:(c + 1) * S]
        o = decode_chunk(model, st, mode, ft, sampling=sampling)
        toks.append(o["tokens"])
        lg.append(o["logits"])
        recs.append(o)
        if log and (c + 1) % 8 == 0:
            log(f"decoded chunk {c + 1}/{chunks}")
    return np.concatenate(toks, 1)[:, r:], np.concatenate(lg, 1)[:, r:], st, recs


# --------------------------------------------------------------------------
# flat (vanilla) Transformer baseline [tpm]: the comparison model of the
# decode-heavy table, whose cache holds the K/V of every token.  Same blocks
# and rounding contract as the PHOTON stacks; Model works with a
# photon_inputs.VanillaConfig (weights E, layers.*, layers.gf, W_out).
# --------------------------------------------------------------------------
class VanillaState:
    """K/V of every layer over every token so far, the rounded final-norm
    output z of the last position (which the next head reads), and the
    number of tokens."""

    def __init__(self, cache, z, n):
        self.cache, self.z, self.n = cache, z, n


def vanilla_prefill(model, prompt, log=None):
    """The prompt through the causal stack at positions 0..P-1, keeping the
    K/V of every position; z = the stack output at the last position."""
    B, P = prompt.shape
    cache = model.empty_cache(model.cfg.n_layers, B)
    z = model.stack("layers", model.cfg.n_layers, model.embed(prompt), np.arange(P), cache=cache, log=log)
    return VanillaState(cache, z[:, -1], P)


def vanilla_decode(model, st, steps, forced_tokens=None):
    """``steps`` greedy tokens per sequence: logits = W_out z, y = first
    argmax, then z = stack(E[y]) at the next position over the cache.
    Returns tokens [B, steps] and logits [B, steps, V].  forced_tokens
    [B, steps] replaces the fed-back token (teacher forcing); the argmax is
    still reported."""
    toks, lgs = [], []
    for j in range(steps):
        lg = model.logits(st.z)
        am = np.argmax(lg, axis=-1).astype(np.int64)
        y = am if forced_tokens is None else np.asarray(forced_tokens)[:, j]
        toks.append(am)
        lgs.append(lg)
        z = model.stack("layers", model.cfg.n_layers, model.embed(y[:, None]), np.array([st.n]), cache=st.cache)
        st.z = z[:, 0]
        st.n += 1
    return np.stack(toks, 1), np.stack(lgs, 1)


def vanilla_generate(model, prompt, new_tokens, forced_tokens=None, log=None):
    st = vanilla_prefill(model, prompt, log=log)
    toks, lgs = vanilla_decode(model, st, new_tokens, forced_tokens)
    return toks, lgs, st


def vanilla_full_logits(model, tokens):
    """Causal forward over tokens [B, T] with no cache: the logits at every
    position (the prediction of the token after it)."""
    T = tokens.shape[1]
    z = model.stack("layers", model.cfg.n_layers, model.embed(tokens), np.arange(T))
    return model.logits(z)


def vanilla_kv_bytes(cfg, batch, tokens):
    """K and V of every layer for every token: the baseline's cache."""
    eb = 4 if cfg.dtype == "f32" else 2
    return cfg.n_layers * 2 * batch * tokens * cfg.d_model * eb


# --------------------------------------------------------------------------
# full recompute (no caches), for the incremental == full checks
# --------------------------------------------------------------------------
def top_full(model, u_all):
    """Causal top-encoder forward over all inputs u_all [B, n, d] at once."""
    n = u_all.shape[1]
    return model.stack("top", model.cfg.n_top, u_all, np.arange(n), None)


def hier_full_logits(model, tokens, n_prompt_states):
    """Teacher-forced HierGen forward over a whole token sequence [B, T]:
    bottom-up over all tokens (every encoder level over its whole stream at
    once, no cache), then for every chunk i >= n_prompt_states the top-down
    pass conditioned on h_{i-1}, with the true previous tokens fed to the
    token decoder.  Returns logits [B, T - P, V]."""
    cfg = model.cfg
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    S, C1 = cfg.S, cfg.C1
    K = S // C1
    z = model.embed(tokens)
    for l in range(1, cfg.L):
        z = model.stack(f"enc{l}", cfg.enc_layers(l), model.chunker(f"W_ch{l}", z),
                        np.arange(T // cfg.span(l)), None)
    h = top_full(model, model.chunker(f"W_ch{cfg.L}", z))     # [B, T/S, d]
    out = []
    for i in range(n_prompt_states, T // S):
        _, A_hat1 = decode_down(model, h[:, i - 1])
        c0 = model.converter("W_cv1", A_hat1).reshape(B * K, C1, -1)
        y = tokens[:, i * S:(i + 1) * S].reshape(B * K, C1)
        x = c0.copy()
        x[:, 1:] += model.embed(y[:, :-1])
        z = model.stack("dec0", cfg.n_dec0, x, np.arange(C1), None)
        out.append(model.logits(z).reshape(B, S, cfg.vocab))
    return np.concatenate(out, 1)


# --------------------------------------------------------------------------
# memory accounting (the TPM denominator) [tpm], [recgen]
# --------------------------------------------------------------------------
def top_states(cfg, tokens):
    """Top-level KV length after ``tokens`` tokens: ceil(T / S)."""
    return -(-tokens // cfg.S)


def kv_bytes(cfg, batch, tokens, mode="recgen"):
    """Resident cache bytes after ``tokens`` tokens.

    top: n_top layers x K,V x B x ceil(T/S) states x d, the only O(T) state.
    dec: the token decoder's in-chunk K/V, n_dec0 x K,V x B*S/C1 sub-chunks
         x C1 positions x d -- independent of T (the decoder's span is the
         chunk).
    lower: HierGen's encoder K/V of every level l below the top, layers x
         K,V x B x ceil(T/span(l)) x d; RecGen drops them after prefill (0).
    """
    b = 2 if cfg.dtype == "bf16" else 4
    d = cfg.d_model
    top = cfg.n_top * 2 * batch * top_states(cfg, tokens) * d * b
    dec = cfg.n_dec0 * 2 * batch * cfg.S * d * b
    lower = 0 if mode == "recgen" else \
        sum(cfg.enc_layers(l) * 2 * batch * (-(-tokens // cfg.span(l))) * d * b for l in range(1, cfg.L))
    return {"top": top, "dec": dec, "lower": lower}


def tpm(ktok_per_s, gib):
    """Throughput per unit memory: K tok/s divided by GiB."""
    return ktok_per_s / gib
