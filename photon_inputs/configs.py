"""Model shapes and decode workloads (synthetic, seeded).

Every workload is uniform-random token ids with independent sequences; decode
cost does not depend on the ids (dense math, fixed token count, no end token).
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class PhotonConfig:
    """Shape of a two-level PHOTON hourglass.

    chunk = (C1, C2): level-0 tokens per level-1 state, level-1 states per
    top state. One top state covers S = C1*C2 tokens.
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

    @property
    def head_dim(self):
        return self.d_model // self.n_heads

    @property
    def C1(self):
        return self.chunk[0]

    @property
    def C2(self):
        return self.chunk[1]

    @property
    def S(self):
        return self.chunk[0] * self.chunk[1]

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
    together (top + level-1 encoder + both decoders)."""
    return VanillaConfig(d_model=cfg.d_model, n_heads=cfg.n_heads, vocab=cfg.vocab,
                         n_layers=cfg.n_top + cfg.n_enc1 + cfg.n_dec1 + cfg.n_dec0,
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
