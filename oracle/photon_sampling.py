"""CPU oracle for sampling decode and multi-query aggregation.  TEST
INFRASTRUCTURE ONLY: the product never imports, calls or links this module;
only the tests, the smoke check and the CPU baseline leg of the benchmark do.

  [multiquery]  PHOTON explainer (mokumoku.ipfde.com, Fujitsu PHOTON vertical
                scan), the paragraph on quality recovery: several slightly
                varied queries are run and bound together by majority vote or
                best-of-N (about nine queries reach the quality of a
                conventional Transformer).
  [philox]      J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
                Random Numbers: As Easy as 1, 2, 3", SC 2011, section on the
                Philox family: Philox-4x32 with 10 rounds.
  [gumbel]      the Gumbel-max identity: argmax_v (x_v + G_v) with G_v i.i.d.
                standard Gumbel is distributed as softmax(x) (E. J. Gumbel,
                1954; the "Gumbel trick" of the sampling literature).

Readings (the pages name the mechanism, not its details):
  * the variation between queries is stochastic decoding: temperature
    sampling with an optional top-k cut, one independent random stream per
    sequence of the batch;
  * top-k keeps every id whose logit is at least the k-th largest logit
    (ties at the cut are kept);
  * a token is drawn as argmax over the kept ids of logit / temperature +
    Gumbel noise, lowest id on ties;
  * the random numbers: Philox-4x32-10 keyed by the 64-bit seed (low word
    first), counter (id // 4, absolute token position, sequence, 0), word
    id % 4 of the output; u = ((word >> 9) + 1/2) / 2^23 = (2m + 1) / 2^24,
    in (0, 1) and exact in float32 (24 significant bits); Gumbel noise
    -log(-log u);
  * the score of a query for best-of-N is the model's log-likelihood of its
    generated tokens: the sum over them of logit[y] - logsumexp(logits)
    (temperature 1, whole vocabulary);
  * the vote of a query is its answer: a span of its generated tokens; the
    majority answer is the one shared by the most queries of the group,
    ties broken by the higher score, then the lower query index;
  * groups are runs of `group` consecutive sequences of the batch (the last
    one may be shorter).
"""
import numpy as np

F64 = np.float64
MASK32 = np.uint64(0xFFFFFFFF)

# [philox]: the two round multipliers and the two key increments of
# Philox-4x32 (the latter the golden ratio and sqrt(3) - 1 in 0.32 fixed point)
PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint64(0x9E3779B9)
PHILOX_W1 = np.uint64(0xBB67AE85)


def philox4x32_10(counter, key):
    """Philox-4x32 with 10 rounds [philox].

    counter: [..., 4] unsigned 32-bit words; key: two unsigned 32-bit words.
    Each round multiplies words 0 and 2 by the two constants (64-bit
    products split into high and low halves), mixes the high halves with the
    odd words and the round key, and permutes; the round key grows by the two
    increments between rounds.  Returns [..., 4] uint32."""
    c = np.asarray(counter, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    for r in range(10):
        if r:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        p0 = PHILOX_M0 * c0                  # < 2^64: no wrap in uint64
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def seed_key(seed):
    """The 64-bit seed as the two key words, low word first."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def uniforms(seed, seq, pos, ids):
    """The uniform variate of every id in `ids` for sequence `seq` at
    absolute token position `pos`: u = ((x >> 9) + 1/2) / 2^23 with x word
    id % 4 of Philox(counter (id // 4, pos, seq, 0), key = seed)."""
    ids = np.asarray(ids, dtype=np.int64)
    ctr = np.zeros(ids.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = ids // 4
    ctr[..., 1] = pos
    ctr[..., 2] = seq
    words = philox4x32_10(ctr, seed_key(seed))
    x = np.take_along_axis(words, (ids % 4)[..., None], axis=-1)[..., 0]
    return ((x >> 9).astype(F64) + 0.5) / float(1 << 23)


def gumbel(u):
    """Standard Gumbel noise from uniforms in (0, 1) [gumbel]."""
    return -np.log(-np.log(np.asarray(u, dtype=F64)))


def top_k_threshold(logits, top_k):
    """The k-th largest logit (ties counted), or -inf for the whole
    vocabulary (top_k = 0 or top_k >= vocab)."""
    lg = np.asarray(logits, dtype=F64)
    if top_k <= 0 or top_k >= lg.shape[-1]:
        return -np.inf
    return np.sort(lg)[::-1][top_k - 1]


def kept_ids(logits, top_k):
    """Ids the top-k cut keeps: every id whose logit reaches the k-th largest."""
    lg = np.asarray(logits, dtype=F64)
    return np.nonzero(lg >= top_k_threshold(lg, top_k))[0]


def sample_scores(logits, temperature, top_k, seed, seq, pos):
    """Perturbed scores logit / temperature + Gumbel noise of every kept id
    (-inf for the ids the cut removes), float64."""
    lg = np.asarray(logits, dtype=F64)
    keep = kept_ids(lg, top_k)
    sc = np.full(lg.shape, -np.inf)
    sc[keep] = lg[keep] / float(temperature) + gumbel(uniforms(seed, seq, pos, keep))
    return sc


def sample(logits, temperature, top_k, seed, seq, pos):
    """One sampled id for one row of logits [V] [multiquery], [gumbel]:
    the first maximum of the perturbed scores."""
    return int(np.argmax(sample_scores(logits, temperature, top_k, seed, seq, pos)))


def loglik(logits, ids):
    """Log-likelihood of each chosen id under the model's distribution
    (temperature 1, whole vocabulary): logit[y] - logsumexp(logits).
    logits [..., V], ids [...]."""
    lg = np.asarray(logits, dtype=F64)
    m = lg.max(axis=-1, keepdims=True)
    lse = (m + np.log(np.exp(lg - m).sum(axis=-1, keepdims=True)))[..., 0]
    y = np.asarray(ids, dtype=np.int64)
    return np.take_along_axis(lg, y[..., None], axis=-1)[..., 0] - lse


def aggregate(tokens, logprobs, group, span=None):
    """Multi-query aggregation [multiquery] over groups of `group`
    consecutive sequences.

    tokens [B, N] generated ids, logprobs [B, N] their log-likelihoods;
    span = (begin, end) of the generated tokens that form a query's answer
    (default: all N).  Returns per group: best (the member, 0-based within
    the group, with the highest summed log-likelihood; lowest index on
    ties), major (the member whose answer the most members share; ties: the
    higher score, then the lower index), votes (how many members share the
    majority answer), and the per-sequence scores [B]."""
    tokens = np.asarray(tokens)
    B, N = tokens.shape
    b0, b1 = (0, N) if span is None else span
    scores = np.asarray(logprobs, dtype=F64).sum(axis=1)
    best, major, votes = [], [], []
    for g0 in range(0, B, group):
        members = list(range(g0, min(B, g0 + group)))
        sc = [scores[m] for m in members]
        best.append(int(np.argmax(sc)))
        ans = [tuple(tokens[m, b0:b1].tolist()) for m in members]
        count = [sum(a == o for o in ans) for a in ans]
        # lexicographic: most votes, then the higher score, then the lower index
        pick = 0
        for i in range(1, len(members)):
            if (count[i], sc[i]) > (count[pick], sc[pick]):
                pick = i
        major.append(pick)
        votes.append(count[pick])
    return np.array(best), np.array(major), np.array(votes), scores
