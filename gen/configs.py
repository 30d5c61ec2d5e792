"""Seeded synthetic inputs for ragged batched token log-probabilities.

This module only draws random numbers: request lengths, echo flags, top_n,
token ids and logits.  It holds none of the method's arithmetic, and it is
the one module that both the CPU oracle's tests and the HIP path's tests and
benchmark use.

The five named workloads mirror the shapes the pages talk about: a vocabulary
of 32000 as in the FlashInfer ``logits_processor`` page's tests, 128256 (the
Llama-3-8B vocabulary named on the SGLang page "logprob、finish reason 与 output
processing"), and larger vocabularies of 151936 and 256000.  The pages
measure nothing on a public dataset, so these seeded draws stand in for real
logits.

Seeding: structure arrays come from ``SeedSequence([cfg])``; the logits of
request n come from ``SeedSequence([cfg, 1, n])``, so any request's rows can be
regenerated on their own.  ``device_logits`` draws the same distributions
with torch's device generator (seeded from the same sequences) for sizes
where host generation would take minutes; the values then differ from the
host draw, so a check always reads its oracle inputs from the tensor it gave
the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Case:
    name: str
    vocab: int
    offsets: np.ndarray        # uint32, batch+1
    echo: np.ndarray           # bool, batch
    top_n: np.ndarray          # int32, batch
    tokens: np.ndarray         # uint32, offsets[-1]
    sampled: np.ndarray        # uint32, batch
    has_logits: bool           # False: only next_token_logits exist
    dist: dict = field(default_factory=dict)
    seed: int = 0

    @property
    def batch(self) -> int:
        return int(self.offsets.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.offsets[-1])

    @property
    def logits_rows(self) -> int:
        return self.total_tokens if self.has_logits else self.batch

    def request_rows(self, n: int) -> tuple[int, int]:
        """[first, last) rows of request n inside the logits the op reads."""
        if self.has_logits:
            return int(self.offsets[n]), int(self.offsets[n + 1])
        return n, n + 1


def _structure_rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed]))


def _request_seq(seed: int, n: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([seed, 1, n])


def make_case(name: str, seed: int, vocab: int, lengths, echo, top_n,
              has_logits: bool, dist: dict, rng: np.random.Generator) -> Case:
    lengths = np.asarray(lengths, dtype=np.int64)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    total = int(offsets[-1])
    tokens = rng.integers(0, vocab, size=total, dtype=np.int64).astype(np.uint32)
    sampled = rng.integers(0, vocab, size=len(lengths), dtype=np.int64).astype(np.uint32)
    dist = dict(dist)
    if dist.get("kind") == "normal" and dist.get("boost"):
        # one boosted id per request row; a greedy decoder would emit it
        boost_ids = rng.integers(0, vocab, size=len(lengths), dtype=np.int64)
        dist["boost_ids"] = boost_ids
        sampled = boost_ids.astype(np.uint32)
    if dist.get("kind") == "quant":
        rows = total if has_logits else len(lengths)
        dist["equal_rows"] = rng.random(rows) < dist.get("p_equal", 0.0)
        dist["equal_level"] = rng.integers(-16, 17, size=rows, dtype=np.int64) / 2.0
    return Case(name, int(vocab), offsets, np.asarray(echo, dtype=bool),
                np.asarray(top_n, dtype=np.int32), tokens, sampled, has_logits,
                dist, seed)


# ---------------------------------------------------------------- named workloads

def no_echo_next_token(seed: int = 1) -> Case:
    """Batch 4, one row each, V=32000, N(0,1), no echo, top_n=5."""
    rng = _structure_rng(seed)
    b = 4
    return make_case("no_echo_next_token", seed, 32000, np.ones(b), np.zeros(b, bool),
                     np.full(b, 5), False, {"kind": "normal", "sigma": 1.0}, rng)


def ragged_echo_mix(seed: int = 2, batch: int = 8, vocab: int = 32000,
                    lmin: int = 16, lmax: int = 512) -> Case:
    """Batch 8, lengths U{16..512}, V=32000, N(0,1.5^2), echo Bernoulli(0.5),
    top_n U{0..7}."""
    rng = _structure_rng(seed)
    lengths = rng.integers(lmin, lmax + 1, size=batch)
    echo = rng.random(batch) < 0.5
    top_n = rng.integers(0, 8, size=batch)
    return make_case("ragged_echo_mix", seed, vocab, lengths, echo, top_n, True,
                     {"kind": "normal", "sigma": 1.5}, rng)


def decode_peaked(seed: int = 3, batch: int = 256, vocab: int = 128256) -> Case:
    """Batch 256 x 1 row, V=128256, N(0,2^2) with one id per row boosted by
    +10, no echo, top_n=7; the sampled token is the boosted id."""
    rng = _structure_rng(seed)
    return make_case("decode_peaked", seed, vocab, np.ones(batch), np.zeros(batch, bool),
                     np.full(batch, 7), False,
                     {"kind": "normal", "sigma": 2.0, "boost": 10.0}, rng)


def prefill_echo_large(seed: int = 4, batch: int = 16, vocab: int = 151936,
                       mean_len: int = 2048, max_len: int = 4096) -> Case:
    """Batch 16, lengths Geometric(mean 2048) clipped to [1, 4096], V=151936,
    N(0,1), all echo, top_n=5."""
    rng = _structure_rng(seed)
    lengths = np.clip(rng.geometric(1.0 / mean_len, size=batch), 1, max_len)
    return make_case("prefill_echo_large", seed, vocab, lengths, np.ones(batch, bool),
                     np.full(batch, 5), True, {"kind": "normal", "sigma": 1.0}, rng)


def tie_edge_stress(seed: int = 5, batch: int = 64, vocab: int = 256000,
                    lmax: int = 128) -> Case:
    """Batch 64, lengths U{1..128}, V=256000, logits k/2 for k~U{-16..16},
    -inf with probability 0.1, 2% rows all-equal, all echo, top_n=7."""
    rng = _structure_rng(seed)
    lengths = rng.integers(1, lmax + 1, size=batch)
    return make_case("tie_edge_stress", seed, vocab, lengths, np.ones(batch, bool),
                     np.full(batch, 7), True,
                     {"kind": "quant", "p_ninf": 0.1, "p_equal": 0.02}, rng)


WORKLOADS = {
    "no_echo_next_token": no_echo_next_token,
    "ragged_echo_mix": ragged_echo_mix,
    "decode_peaked": decode_peaked,
    "prefill_echo_large": prefill_echo_large,
    "tie_edge_stress": tie_edge_stress,
}


# ---------------------------------------------------------------- logits (host)

def request_logits_host(case: Case, n: int) -> np.ndarray:
    """Rows of request n (its full range, or its one next-token row)."""
    r0, r1 = case.request_rows(n)
    return _draw_rows(case, n, r0, r1 - r0)


def request_rows_sample(case: Case, n: int, k: int) -> np.ndarray:
    """The first min(k, rows of request n) rows of request n's draw, without
    drawing the rest: for the normal distributions these are exactly the
    first rows of ``request_logits_host``; for the tie workload they are rows
    of the same distribution from the same seed (its draw interleaves two
    arrays, so a prefix is a different draw)."""
    r0, r1 = case.request_rows(n)
    return _draw_rows(case, n, r0, min(int(k), r1 - r0))


def _draw_rows(case: Case, n: int, r0: int, rows: int) -> np.ndarray:
    rng = np.random.default_rng(_request_seq(case.seed, n))
    d = case.dist
    if d["kind"] == "normal":
        x = rng.standard_normal((rows, case.vocab), dtype=np.float32)
        x *= np.float32(d["sigma"])
        if "boost_ids" in d:
            x[:, int(d["boost_ids"][n])] += np.float32(d["boost"])
        return x
    if d["kind"] == "quant":
        k = rng.integers(-16, 17, size=(rows, case.vocab), dtype=np.int8)
        x = k.astype(np.float32) * np.float32(0.5)
        ninf = rng.random((rows, case.vocab), dtype=np.float32) < d["p_ninf"]
        for i in range(rows):
            if d["equal_rows"][r0 + i]:
                x[i, :] = np.float32(d["equal_level"][r0 + i])
            else:
                x[i, ninf[i]] = -np.inf
        return x
    if d["kind"] == "gumbel":
        return rng.gumbel(size=(rows, case.vocab)).astype(np.float32)
    raise ValueError(f"unknown distribution {d['kind']}")


def host_logits(case: Case) -> np.ndarray:
    """All logits rows the op reads: (tokens, V) or (batch, V) float32."""
    out = np.empty((case.logits_rows, case.vocab), dtype=np.float32)
    for n in range(case.batch):
        r0, r1 = case.request_rows(n)
        out[r0:r1] = request_logits_host(case, n)
    return out


def next_token_rows(case: Case, logits: np.ndarray) -> np.ndarray:
    """With full logits, a request's next-token row is its last row."""
    if not case.has_logits:
        return logits
    last = case.offsets[1:].astype(np.int64) - 1
    return logits[last]


# ---------------------------------------------------------------- logits (device)

def device_logits(case: Case, device, torch):
    """Same distributions, drawn on the device with torch's generator.

    ``torch`` is passed in so this module does not import it on CPU-only
    paths.  Returns a contiguous (rows, V) float32 tensor.
    """
    out = torch.empty((case.logits_rows, case.vocab), dtype=torch.float32, device=device)
    d = case.dist
    g = torch.Generator(device=device)
    for n in range(case.batch):
        r0, r1 = case.request_rows(n)
        g.manual_seed(int(_request_seq(case.seed, n).generate_state(1, np.uint64)[0] >> 1))
        blk = out[r0:r1]
        if d["kind"] == "normal":
            blk.normal_(0.0, float(d["sigma"]), generator=g)
            if "boost_ids" in d:
                blk[:, int(d["boost_ids"][n])] += float(d["boost"])
        elif d["kind"] == "quant":
            k = torch.randint(-16, 17, blk.shape, device=device, generator=g,
                              dtype=torch.int32)
            blk.copy_(k.to(torch.float32) * 0.5)
            u = torch.rand(blk.shape, device=device, generator=g)
            blk.masked_fill_(u < d["p_ninf"], float("-inf"))
            for i in range(r1 - r0):
                if d["equal_rows"][r0 + i]:
                    blk[i].fill_(float(d["equal_level"][r0 + i]))
            del k, u
        elif d["kind"] == "gumbel":
            u = torch.rand(blk.shape, device=device, generator=g).clamp_(1e-20, 1.0)
            blk.copy_(-torch.log(-torch.log(u)))
            del u
        else:
            raise ValueError(d["kind"])
    return out
