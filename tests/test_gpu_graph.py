"""lp_launch_ragged captured in a HIP graph (needs an MI355X).

The launch enqueues kernels only (no copy, no memset, no event), so a caller
can capture it once and replay it per step, staging that step's descriptors
into the workspace outside the graph.  Each case captures the launch, then
replays it several times; between replays the program changes the logits in
place, stages other sampled tokens, and runs the same launch eagerly into
separate outputs.  Every replay must equal the eager launch bit for bit (the
plans use the deterministic chunk order), and the last one the oracle.
"""
import numpy as np
import pytest

import gen
from tests.gpu_helpers import assert_parity, log, oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def R():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_token_log_amd as lib
    lib.load()
    return lib


def _cases():
    mix = gen.ragged_echo_mix(seed=71, batch=6, lmin=5, lmax=40, vocab=20011)
    mix.top_n[2] = 0                                # a padding-only request among them
    dec = gen.decode_peaked(seed=72, batch=48, vocab=50021)
    return [("ragged echo mix, whole rows", mix, 1), ("decode, 4 segments and a merge", dec, 4)]


@pytest.mark.parametrize("which", [0, 1])
def test_launch_replayed_from_a_graph(R, which):
    where, case, split = _cases()[which]
    dev = torch.device("cuda")
    rng = np.random.default_rng(700 + which)
    base = gen.host_logits(case)
    variants = [base] + [(base + rng.standard_normal(base.shape).astype(np.float32)).astype(np.float32)
                         for _ in range(3)]
    sampled = [case.sampled] + [rng.integers(0, case.vocab, case.batch).astype(np.uint32)
                                for _ in range(3)]
    plan = R.Plan(case.offsets, case.echo, case.top_n, case.vocab, case.has_logits)
    plan.set_split(split)
    plan.set_deterministic(True)
    log(f"{where}: {plan.info()['out_rows']} rows, split {plan.info()['split']}")
    logits = torch.from_numpy(variants[0]).to(dev)
    ntl = torch.from_numpy(np.ascontiguousarray(gen.next_token_rows(case, variants[0]))).to(dev)
    lp, ids, ws = R.alloc_outputs(plan, dev, torch)
    lp_e, ids_e, _ = R.alloc_outputs(plan, dev, torch)
    src = (logits, ntl) if case.has_logits else (None, ntl)

    stream = torch.cuda.Stream()
    plan.stage(case.tokens, sampled[0], ws, stream)
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        plan.launch(*src, lp, ids, ws, torch.cuda.current_stream())
    torch.cuda.synchronize()

    for k in range(len(variants)):
        # the step's inputs, outside the graph: logits in place, descriptors staged
        logits.copy_(torch.from_numpy(variants[k]))
        ntl.copy_(torch.from_numpy(np.ascontiguousarray(gen.next_token_rows(case, variants[k]))))
        torch.cuda.synchronize()                    # the copies ran on the default stream
        with torch.cuda.stream(stream):
            plan.stage(case.tokens, sampled[k], ws, stream)
            graph.replay()
            plan.launch(*src, lp_e, ids_e, ws, stream)
        torch.cuda.synchronize()
        got_lp, got_ids = lp.cpu().numpy(), ids.cpu().numpy()
        assert np.array_equal(got_ids, ids_e.cpu().numpy()), f"{where}: replay {k} ids"
        assert np.array_equal(got_lp.view(np.uint32), lp_e.cpu().numpy().view(np.uint32)), \
            f"{where}: replay {k} logprobs"
        if k == len(variants) - 1:
            ref = oracle(case.offsets, variants[k] if case.has_logits else None,
                         gen.next_token_rows(case, variants[k]), case.tokens, sampled[k],
                         case.top_n, case.echo)
            assert_parity(got_lp, got_ids, plan.out_off, ref, f"{where}: replay {k} vs oracle")
    plan.close()
