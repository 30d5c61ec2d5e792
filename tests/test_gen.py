"""Seeded generators: shapes, ranges and determinism (CPU only)."""
import numpy as np

import gen


def test_workload_structures():
    c = gen.no_echo_next_token()
    assert (c.batch, c.vocab, c.has_logits) == (4, 32000, False)
    assert c.offsets.tolist() == [0, 1, 2, 3, 4] and (c.top_n == 5).all() and not c.echo.any()
    c = gen.ragged_echo_mix()
    L = np.diff(c.offsets.astype(np.int64))
    assert c.batch == 8 and L.min() >= 16 and L.max() <= 512 and c.has_logits
    assert c.top_n.min() >= 0 and c.top_n.max() <= 7
    c = gen.decode_peaked()
    assert (c.batch, c.vocab) == (256, 128256) and (c.top_n == 7).all()
    assert np.array_equal(c.sampled, c.dist["boost_ids"].astype(np.uint32))
    c = gen.prefill_echo_large()
    L = np.diff(c.offsets.astype(np.int64))
    assert c.batch == 16 and L.min() >= 1 and L.max() <= 4096 and c.echo.all()
    c = gen.tie_edge_stress()
    L = np.diff(c.offsets.astype(np.int64))
    assert c.vocab == 256000 and L.min() >= 1 and L.max() <= 128 and (c.top_n == 7).all()
    for c in (gen.WORKLOADS[k]() for k in gen.WORKLOADS):
        assert c.tokens.dtype == np.uint32 and c.tokens.shape[0] == c.total_tokens
        assert int(c.tokens.max()) < c.vocab and int(c.sampled.max()) < c.vocab


def test_host_logits_deterministic_and_distributed():
    c = gen.ragged_echo_mix(batch=2, lmin=3, lmax=5)
    a, b = gen.host_logits(c), gen.host_logits(c)
    assert a.dtype == np.float32 and a.shape == (c.total_tokens, c.vocab)
    assert np.array_equal(a, b)
    assert abs(float(a.std()) - 1.5) < 0.05
    r = gen.request_logits_host(c, 1)
    assert np.array_equal(r, a[c.offsets[1]:c.offsets[2]])


def test_quantised_rows():
    c = gen.tie_edge_stress(batch=3, vocab=4000, lmax=20)
    x = gen.host_logits(c)
    fin = x[np.isfinite(x)]
    assert np.all(fin * 2 == np.round(fin * 2)) and fin.min() >= -8 and fin.max() <= 8
    eq = c.dist["equal_rows"]
    for r in range(x.shape[0]):
        if eq[r]:
            assert np.all(x[r] == x[r, 0])
        else:
            assert 0.05 < np.isneginf(x[r]).mean() < 0.15


def test_boosted_rows():
    c = gen.decode_peaked(batch=4, vocab=5000)
    x = gen.host_logits(c)
    assert np.array_equal(np.argmax(x, axis=1), c.dist["boost_ids"])
