"""Seeded weight and prompt generators.

Weights: every matrix is drawn in a fixed canonical order from one stream,
``numpy.random.default_rng([seed, 0])``, as ``standard_normal(float32) * 0.02``
(N(0, 0.02^2)). Norm gains are 1 and there are no biases. For bf16 models the
drawn matrices are stored as bf16 (round to nearest, ties to even), so both
the oracle and the GPU receive bit-identical values.

Prompts: ``default_rng([seed, 1]).integers(0, V, (B, P), dtype=int32)``.

Matrices are W[out, in]; a linear layer computes y = x W^T.
"""
from collections import OrderedDict
import numpy as np

from .configs import VanillaConfig

MATRIX_STD = np.float32(0.02)
LAYER_PARTS = ("g1", "Wq", "Wk", "Wv", "Wo", "g2", "W1", "W2")


def _layer_shapes(prefix, n, d, dff):
    out = []
    for l in range(n):
        p = f"{prefix}.{l}."
        out += [(p + "g1", (d,)), (p + "Wq", (d, d)), (p + "Wk", (d, d)),
                (p + "Wv", (d, d)), (p + "Wo", (d, d)), (p + "g2", (d,)),
                (p + "W1", (dff, d)), (p + "W2", (d, dff))]
    out.append((prefix + ".gf", (d,)))
    return out


def weight_shapes(cfg):
    """Canonical (name, shape) list, in generation order: the embedding,
    then bottom-up the chunker and encoder of every level below the top,
    the top chunker and encoder, then top-down the converter and decoder of
    every level, then the output head.  Level l's tensors are W_ch<l>,
    enc<l>.*, W_cv<l> and dec<l-1>.* (the converter of level l feeds the
    decoder one level down)."""
    if isinstance(cfg, VanillaConfig):
        d, dff, V = cfg.d_model, cfg.d_ff, cfg.vocab
        return [("E", (V, d))] + _layer_shapes("layers", cfg.n_layers, d, dff) + [("W_out", (V, d))]
    d, dff, V, L = cfg.d_model, cfg.d_ff, cfg.vocab, cfg.L
    s = [("E", (V, d))]
    for l in range(1, L):
        s += [(f"W_ch{l}", (d, cfg.chunk[l - 1] * d))]
        s += _layer_shapes(f"enc{l}", cfg.enc_layers(l), d, dff)
    s += [(f"W_ch{L}", (d, cfg.chunk[L - 1] * d))]
    s += _layer_shapes("top", cfg.n_top, d, dff)
    for l in range(L, 0, -1):
        s += [(f"W_cv{l}", (cfg.chunk[l - 1] * d, d))]
        s += _layer_shapes(f"dec{l - 1}", cfg.dec_layers(l - 1), d, dff)
    s += [("W_out", (V, d))]
    return s


def weight_names(cfg):
    return [n for n, _ in weight_shapes(cfg)]


def bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even.

    Input values here are finite (weights), so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs: u + 0x8000 cannot wrap a uint32
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def _bf16_values(x):
    return (bf16_bits(x).astype(np.uint32) << 16).view(np.float32)


def gen_weights(cfg, seed, zero=()):
    """Seeded weights as float32 arrays (bf16-exact when cfg.dtype == 'bf16').

    ``zero`` names tensors to replace by zeros after drawing (the stream is
    unchanged, so every other tensor keeps its value).
    """
    rng = np.random.default_rng([seed, 0])
    out = OrderedDict()
    for name, shape in weight_shapes(cfg):
        if len(shape) == 1:
            w = np.ones(shape, dtype=np.float32)
        else:
            w = rng.standard_normal(shape, dtype=np.float32) * MATRIX_STD
            if cfg.dtype == "bf16":
                w = _bf16_values(w)
        if name in zero:
            w = np.zeros_like(w)
        out[name] = w
    return out


def gen_prompts(cfg, batch, prompt, seed):
    rng = np.random.default_rng([seed, 1])
    return rng.integers(0, cfg.vocab, size=(batch, prompt), dtype=np.int32)


def gen_decode_state(cfg, seq, n_top_states, mode="recgen", seed=0):
    """Seeded stand-in for the decode state one sequence holds after a
    prefill of n_top_states top states (a prompt of n_top_states * S
    tokens), for tests that inject the same state into both sides.

    Stream ``default_rng([seed, 2, seq])``, so a sequence's values do not
    depend on which other sequences are drawn.  Returns a dict:
      top_k, top_v: [n_top, n_top_states, H, hd], one entry per top layer;
      h:            [d], the last top output;
      low_k, low_v: (HierGen only) {l: [layers_l, n_l, H, hd]} for every
                    encoder level l = 1 .. L-1, n_l = n_top_states * S / span(l).
    Cached keys and values are N(0, (0.02 sqrt(d))^2): the spread of a
    projection of a unit-RMS row by N(0, 0.02^2) weights.  h is N(0, 1), the
    spread of a normalized row with unit gains.  bf16 models get bf16-exact
    values (round to nearest even), like every stored cache entry."""
    rng = np.random.default_rng([seed, 2, seq])
    H, hd, d = cfg.n_heads, cfg.head_dim, cfg.d_model
    sd = np.float32(0.02 * np.sqrt(d))
    cast = _bf16_values if cfg.dtype == "bf16" else (lambda a: a)

    def kv(layers, n):
        return [cast(rng.standard_normal((layers, n, H, hd), dtype=np.float32) * sd) for _ in range(2)]

    out = {}
    out["top_k"], out["top_v"] = kv(cfg.n_top, n_top_states)
    out["h"] = cast(rng.standard_normal(d, dtype=np.float32))
    if mode == "hiergen":
        out["low_k"], out["low_v"] = {}, {}
        for l in range(1, cfg.L):
            n_l = n_top_states * cfg.S // cfg.span(l)
            out["low_k"][l], out["low_v"][l] = kv(cfg.enc_layers(l), n_l)
    return out
