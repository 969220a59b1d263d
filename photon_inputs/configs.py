"""Model shapes and decode workloads (synthetic, seeded).

Every workload is uniform-random token ids with independent sequences; decode
cost does not depend on the ids (dense math, fixed token count, no end token).
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class PhotonConfig:
    """Shape of an L-level PHOTON hourglass (L = len(chunk) >= 2).

    chunk = (C1, ..., CL): C_l level-(l-1) states form one level-l state
    (level 0 = tokens, level L = the top).  One level-l state covers
    span(l) = C1*...*C_l tokens; one top state covers S = span(L).
    Layer counts: n_top (top encoder), n_enc1 / n_dec1 (level-1 encoder /
    decoder), n_dec0 (token decoder); for L > 2, n_enc_hi[l-2] and
    n_dec_hi[l-2] are the level-l encoder and decoder, l = 2 .. L-1.
    """
    d_model: int
    n_heads: int
    chunk: tuple
    vocab: int
    n_top: int
    n_enc1: int
    n_dec1: int
    n_dec0: int
    dtype: str = "bf16"          # "f32" or "bf16" (storage of weights/KV)
    mlp_mult: int = 4
    norm_eps: float = 1e-5
    rope_theta: float = 10000.0
    n_enc_hi: tuple = ()
    n_dec_hi: tuple = ()

    def __post_init__(self):
        if len(self.chunk) < 2:
            raise ValueError("a hierarchy needs at least two levels")
        if len(self.n_enc_hi) != len(self.chunk) - 2 or len(self.n_dec_hi) != len(self.chunk) - 2:
            raise ValueError("n_enc_hi and n_dec_hi need one entry per level 2 .. L-1")

    @property
    def head_dim(self):
        return self.d_model // self.n_heads

    @property
    def L(self):
        return len(self.chunk)

    @property
    def C1(self):
        return self.chunk[0]

    @property
    def C2(self):
        return self.chunk[1]

    def span(self, l):
        """Tokens per level-l state (1 for level 0)."""
        out = 1
        for c in self.chunk[:l]:
            out *= c
        return out

    @property
    def S(self):
        return self.span(self.L)

    def enc_layers(self, l):
        """Layers of the level-l encoder, 1 <= l <= L-1."""
        return self.n_enc1 if l == 1 else self.n_enc_hi[l - 2]

    def dec_layers(self, l):
        """Layers of the level-l decoder, 0 <= l <= L-1."""
        return (self.n_dec0, self.n_dec1)[l] if l < 2 else self.n_dec_hi[l - 2]

    @property
    def d_ff(self):
        return self.mlp_mult * self.d_model

    def with_(self, **kw):
        return replace(self, **kw)


@dataclass(frozen=True)
class VanillaConfig:
    """A flat decoder-only Transformer for the decode baseline: one causal
    stack over the tokens (its K/V cache holds every token) with the same
    blocks as the PHOTON stacks, an embedding and an untied output head."""
    d_model: int
    n_heads: int
    vocab: int
    n_layers: int
    dtype: str = "bf16"
    mlp_mult: int = 4
    norm_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def head_dim(self):
        return self.d_model // self.n_heads

    @property
    def d_ff(self):
        return self.mlp_mult * self.d_model


def vanilla_of(cfg):
    """The baseline matched to a PHOTON shape: same width, heads, MLP,
    vocabulary and precision, and as many layers as all PHOTON stacks
    together (top + every encoder + every decoder)."""
    n = cfg.n_top + sum(cfg.enc_layers(l) for l in range(1, cfg.L)) + sum(cfg.dec_layers(l) for l in range(cfg.L))
    return VanillaConfig(d_model=cfg.d_model, n_heads=cfg.n_heads, vocab=cfg.vocab,
                         n_layers=n,
                         dtype=cfg.dtype, mlp_mult=cfg.mlp_mult, norm_eps=cfg.norm_eps,
                         rope_theta=cfg.rope_theta)


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: PhotonConfig
    batch: int
    prompt: int
    new_tokens: int
    seed: int

    @property
    def chunks(self):
        return self.new_tokens // self.cfg.S

    @property
    def prompt_states(self):
        return self.prompt // self.cfg.S

    @property
    def max_tokens(self):
        return self.prompt + self.new_tokens


TINY = PhotonConfig(d_model=64, n_heads=2, chunk=(4, 4), vocab=256,
                    n_top=1, n_enc1=1, n_dec1=1, n_dec0=1, dtype="f32")
M150 = PhotonConfig(d_model=768, n_heads=12, chunk=(4, 4), vocab=32000,
                    n_top=8, n_enc1=2, n_dec1=2, n_dec0=2, dtype="bf16")
M600 = PhotonConfig(d_model=1536, n_heads=16, chunk=(4, 4), vocab=32000,
                    n_top=16, n_enc1=4, n_dec1=4, n_dec0=4, dtype="bf16")
M600_2x2 = M600.with_(chunk=(2, 2))

CONFIGS = {"tiny": TINY, "m150": M150, "m600": M600, "m600_2x2": M600_2x2}

# Index 1..5 follows the order in which the workloads are listed for this
# project: tiny fp32, 150M-shaped, 600M-shaped, long context, 2x2 multi-query.
WORKLOADS = {
    1: Workload("tiny-f32 B2 P64 N32", TINY, 2, 64, 32, 0),
    2: Workload("photon-150m bf16 B32 P1024 N256", M150, 32, 1024, 256, 1),
    3: Workload("photon-600m bf16 B64 P4096 N512", M600, 64, 4096, 512, 2),
    4: Workload("photon-600m-long bf16 B16 P32768 N256", M600, 16, 32768, 256, 3),
    5: Workload("photon-600m-2x2 bf16 B256 P8192 N512", M600_2x2, 256, 8192, 512, 4),
}


def get(idx):
    return WORKLOADS[idx]
