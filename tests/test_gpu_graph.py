"""A scoring step captured as a HIP graph (ScoringGraph) against eager steps on the same
inputs: every replay's per-row outputs and statistics bitwise equal to those of an
uncaptured ScoringStep, over several replays with new input data written in place and
eager work and synchronizations between them; once with the single-block selection and
once above 65536 rows (the multi-block digit launches)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _same_stats(got, want):
    assert set(got) == set(want)
    for k, w in want.items():
        g = got[k]
        if isinstance(w, float):
            assert np.float64(g).tobytes() == np.float64(w).tobytes(), (k, g, w)
        else:
            assert g == w, (k, g, w)


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.parametrize("spec", [dict(name="qwen8b", B=3, L=96),
                                  dict(name="large", B=4, L=20000, V=8, prompt=4)],
                         ids=["qwen8b_small", "large_V8_80000_rows"])
def test_graph_replays_match_eager_steps(spec):
    from helpers import device_inputs, make_small
    from train_rollout_logprob_amd import binding as B
    print(f"[case] graph {spec}", flush=True)
    case = make_small(spec)
    ids, att, act, cu = device_inputs(case)
    train, rollout = case.train.clone(), case.rollout.clone()
    mk = lambda: B.ScoringStep(train, rollout, ids, att, act, case.layout, case.B, case.L, cu,
                               case.eps_low, case.eps_high)
    step, ref = mk(), mk()
    graph = B.ScoringGraph(step)
    gen = torch.Generator(device="cuda").manual_seed(7)
    for k in range(3):
        if k:  # new logits in place, then other eager work before the replay
            noise = torch.randn(train.shape, generator=gen, device="cuda") * (0.01 * k)
            train.copy_((train.float() + noise).to(train.dtype))
            torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert ref.run() == B.DRIFT_OK      # eager step on the same inputs, its own buffers
        for g, w in zip(step.out, ref.out):
            assert torch.equal(_bits(g), _bits(w))
        want = ref.stats.as_dict()
        assert want["n_active"] > 0
        _same_stats(graph.stats().as_dict(), want)
    if case.N > 65536:
        assert step.N > 65536
