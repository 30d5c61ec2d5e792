"""Glue for the GPU parity tests: run the library through its binding, run the
oracle on the same inputs, compare.  Holds no arithmetic of the method."""
from __future__ import annotations

import sys

import numpy as np

import oracle.logprob_oracle as LO

ATOL = 1e-5   # logprob tolerance (fp32 GPU vs float64 oracle rounded to fp32)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class DeviceRows:
    """Row source for the oracle that copies single rows back from a GPU tensor."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, r):
        return self.t[int(r)].cpu().numpy()


def shard_bounds(vocab, n_shards, rng):
    """Uneven vocabulary ranges covering [0, vocab) once each."""
    cuts = sorted(rng.choice(np.arange(1, vocab), size=n_shards - 1, replace=False).tolist())
    b = [0] + cuts + [vocab]
    return list(zip(b[:-1], b[1:]))


def run_sharded(R, torch, off, logits, ntl, tokens, sampled, top_n, echo, levels, bounds,
                top_k=None):
    """The batch through the vocabulary-shard path: each shard's columns (as
    their own contiguous device arrays) to lp_shard_records, the records
    stacked, then lp_merge_shards; returns host (lp, ids, out_off)."""
    dev = torch.device("cuda")
    has_logits = logits is not None
    plan = R.Plan(off, echo, top_n, ntl.shape[1], has_logits, levels=levels)
    if top_k is not None:
        plan.set_top_k(top_k)
    words = plan.info()["record_words"]
    lp, ids, ws = R.alloc_outputs(plan, dev, torch)
    stream = torch.cuda.current_stream()
    plan.stage(tokens, sampled, ws, stream)
    records = torch.zeros((len(bounds), plan.out_rows, words), dtype=torch.int64, device=dev)

    def cols(x, b, e):
        return torch.from_numpy(np.ascontiguousarray(x[:, b:e])).cuda()

    for k, (b, e) in enumerate(bounds):
        sl = cols(logits, b, e) if has_logits else None
        plan.shard_records(b, sl, cols(ntl, b, e), records[k], ws, stream)
    plan.merge_shards(len(bounds), records, lp, ids, ws, stream)
    torch.cuda.synchronize()
    out = lp.cpu().numpy(), ids.cpu().numpy(), plan.out_off.copy()
    plan.close()
    return out


def run_library(R, torch, offsets, logits, ntl, tokens, sampled, top_n, echo, split=None,
                waves=None, depth=None, levels=3, deterministic=False):
    lp, ids, out_off = R.compute_log_probabilities_ragged(
        offsets, logits, ntl, tokens, sampled, top_n, echo, split=split, waves=waves, depth=depth,
        levels=levels, deterministic=deterministic)
    torch.cuda.synchronize()
    return lp.cpu().numpy(), ids.cpu().numpy(), out_off


def assert_lp_close(got, want, where, atol=ATOL):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert got.shape == want.shape, (where, got.shape, want.shape)
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    bad = nan_g != nan_w
    inf_w = np.isinf(want) | np.isinf(got)
    bad |= inf_w & ~nan_g & ~nan_w & (got != want)
    fin = ~nan_g & ~nan_w & ~inf_w
    diff = np.zeros_like(got)
    diff[fin] = np.abs(got[fin] - want[fin])
    bad |= diff > atol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{where}: {int(bad.sum())} logprobs differ; first at {idx.tolist()}: "
                             f"got {[float(got[tuple(i)]) for i in idx]} "
                             f"want {[float(want[tuple(i)]) for i in idx]}; max |d| {diff.max()}")


def assert_parity(lp, ids, out_off, ref, where, rows=None):
    ref_lp, ref_ids, ref_off = ref
    assert np.array_equal(out_off, ref_off), (where, "output offsets")
    sel = slice(None) if rows is None else np.asarray(rows)
    g_ids, w_ids = ids[sel], ref_ids[sel]
    if not np.array_equal(g_ids, w_ids):
        bad = np.argwhere(g_ids != w_ids)[:5]
        raise AssertionError(f"{where}: ids differ at {bad.tolist()}: "
                             f"got {[int(g_ids[tuple(b)]) for b in bad]} "
                             f"want {[int(w_ids[tuple(b)]) for b in bad]}")
    assert_lp_close(lp[sel], ref_lp[sel], where)


def assert_close_rel(got, want, where):
    """Logprobs at a temperature T != 1: |lp| reaches |x - max| / T.  The
    kernels divide by T in fp64, so the value carries the same few-1e-7 error
    as at T = 1 before its one rounding to fp32; where |lp| >= 128 an fp32 ulp
    exceeds 1e-5, and the two roundings (oracle, kernel) may then land one ulp
    apart.  The bound is 1e-5, plus one ulp of the expected value where
    |lp| >= 128 (NaN and infinities exactly)."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    nan = np.isnan(want)
    assert np.array_equal(nan, np.isnan(got)), where
    inf = np.isinf(want)
    assert np.array_equal(got[inf], want[inf]), where
    fin = ~nan & ~inf
    mag = np.abs(want[fin])
    tol = 1e-5 + np.where(mag >= 128.0, np.spacing(mag), 0.0)
    d = np.abs(got[fin].astype(np.float64) - want[fin])
    assert np.all(d <= tol), (where, float(d.max()), float(np.abs(want[fin]).max()))


def oracle(offsets, logits, ntl, tokens, sampled, top_n, echo, rows=None, levels=3):
    return LO.compute_log_probabilities_ragged(offsets, logits, ntl, tokens, sampled,
                                               list(top_n), list(echo), rows=rows, levels=levels)


def check_all_rows_properties(torch, src, desc, lp_dev, ids_dev, vocab, chunk=256):
    """Checks every output row on the device, at any size, from properties:

    * the ranked ids are an exact top-k of the raw fp32 row under (value
      descending, id ascending): the listed values are non-increasing, ids
      increase within equal values, and exactly j elements rank above the
      j-th listed one;
    * lp = x - logsumexp(x) within ATOL, logsumexp taken in float64 by torch;
    * the last column is (x[chosen] - lse, chosen); padding is (-inf, PAD).
    ``desc`` is the oracle's row list (src_row, chosen, top_n) per output row.
    """
    dev = lp_dev.device
    R = lp_dev.shape[0]
    src_rows = torch.tensor([d.src_row for d in desc], dtype=torch.int64, device=dev)
    chosen = torch.tensor([d.chosen for d in desc], dtype=torch.int64, device=dev)
    topn = torch.tensor([d.top_n for d in desc], dtype=torch.int64, device=dev)
    ids64 = ids_dev.to(torch.int64)
    pad = ids64 == 0xFFFFFFFF
    col = torch.arange(8, device=dev)
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        tn = topn[r0:r1]
        live = tn > 0
        if not bool(live.any()):
            assert bool(pad[r0:r1].all())
            continue
        x = src.index_select(0, src_rows[r0:r1])                       # (n, V) fp32
        lse = torch.logsumexp(x.double(), dim=1)                        # (n,)
        kk = torch.minimum(tn, torch.full_like(tn, vocab))
        ranked = col[:7].unsqueeze(0) < kk.unsqueeze(1)                 # (n, 7)
        idr = ids64[r0:r1, :7]
        assert bool((pad[r0:r1, :7] == ~ranked).all()), "padding layout"
        safe = torch.where(ranked, idr, torch.zeros_like(idr))
        v = torch.gather(x, 1, safe)                                    # listed values
        v = torch.where(ranked, v, torch.full_like(v, float("nan")))
        # exact rank of each listed element
        for j in range(7):
            m = ranked[:, j]
            if not bool(m.any()):
                continue
            vj = v[:, j:j + 1]
            ij = safe[:, j:j + 1]
            ar = torch.arange(vocab, device=dev).unsqueeze(0)
            above = (x > vj) | ((x == vj) & (ar < ij))
            cnt = above.sum(dim=1)
            assert bool((cnt[m] == j).all()), f"rank of slot {j} in rows {r0}..{r1}"
            del above
        want = (v.double() - lse.unsqueeze(1)).float()
        got = lp_dev[r0:r1, :7]
        diff = torch.where(ranked, (got - want).abs(), torch.zeros_like(got))
        nanok = torch.isnan(got) == torch.isnan(want)
        assert bool(nanok[ranked].all()), "NaN pattern"
        d = torch.nan_to_num(diff, nan=0.0, posinf=0.0)
        assert float(d.max()) <= ATOL, f"logprob diff {float(d.max())} in rows {r0}..{r1}"
        assert bool(torch.isneginf(got[~ranked]).all())
        # chosen column
        ch = chosen[r0:r1]
        xc = torch.gather(x, 1, ch.unsqueeze(1)).squeeze(1)
        wc = (xc.double() - lse).float()
        gc = lp_dev[r0:r1, 7]
        ok = ((gc - wc).abs() <= ATOL) | (torch.isnan(gc) & torch.isnan(wc)) | (gc == wc)
        assert bool(ok[live].all()), f"chosen column in rows {r0}..{r1}"
        assert bool((ids64[r0:r1, 7][live] == ch[live]).all())
        assert bool(pad[r0:r1][~live].all())
        del x


def special_rows(rng, n, vocab):
    """Rows covering the degenerate cases: all-equal, +-0.0, -inf heavy, all
    -inf, one finite entry, a boosted token, heavy ties."""
    rows = []
    kinds = ["normal", "equal", "zeros", "ninf_heavy", "all_ninf", "one_finite", "boost",
             "ties", "ninf_prefix"]
    for i in range(n):
        k = kinds[i % len(kinds)]
        if k == "normal":
            x = rng.standard_normal(vocab).astype(np.float32) * 2
        elif k == "equal":
            x = np.full(vocab, -0.5, np.float32)
        elif k == "zeros":
            x = np.where(rng.random(vocab) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
            x[rng.random(vocab) < 0.2] = -1.0
        elif k == "ninf_heavy":
            x = rng.standard_normal(vocab).astype(np.float32)
            x[rng.random(vocab) < 0.9] = -np.inf
        elif k == "all_ninf":
            x = np.full(vocab, -np.inf, np.float32)
        elif k == "one_finite":
            x = np.full(vocab, -np.inf, np.float32)
            x[rng.integers(vocab)] = 3.0
        elif k == "boost":
            x = rng.standard_normal(vocab).astype(np.float32)
            x[rng.integers(vocab)] += 30.0
        elif k == "ties":
            x = (rng.integers(-3, 4, vocab) * 0.5).astype(np.float32)
        else:  # a long -inf run at the start, then values
            x = rng.standard_normal(vocab).astype(np.float32)
            x[: vocab * 3 // 4] = -np.inf
        rows.append(x)
    return np.stack(rows)
