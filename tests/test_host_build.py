"""sce_build_candidates_host (the candidate build on the host, in the library) against the
oracle's build, bit for bit: random workloads up to the full sizes, a window that wraps,
the page's fallback, P = V, the vocabulary limit, no labels, and the asserted conditions
(which are flagged, as the device build flags them). CPU only: the call does no device
work."""
import numpy as np
import pytest

from oracle import OracleError, build_candidates
from sampled_softmax_cross_amd import binding, synth


def _check(y, p, V, P, stride, offset):
    got = binding.build_candidates_host(y, p, V, P, stride, offset)
    ref = build_candidates(V, P, stride, offset, y, p)
    T = len(y)
    assert np.array_equal(got["C"].numpy(), ref["C"])
    assert np.array_equal(got["target_pos"].numpy()[:T], ref["target_pos"])
    if p is not None:
        assert np.array_equal(got["prefix_pos"].numpy()[:T], ref["prefix_pos"])
    assert got["aux"].tolist() == [ref["num_targets"], ref["N"], ref["next_offset"], 0]
    return ref


@pytest.mark.parametrize("name", ["tiny", "stage01", "s2early", "s2late"])
def test_workloads(name):
    w = synth.workload(name)
    for call in range(w.calls):
        y, p = synth.make_labels(w, call)
        _check(y, p, w.V, w.P, w.stride, w.call_offset(call))


def test_random_cases_and_edges():
    rng = np.random.default_rng(5)
    for it in range(60):
        V = int(rng.choice([7, 64, 65, 1000, 4096, 12345, 131072]))
        T = int(rng.integers(0, 3000))
        y = rng.integers(-1, V, T)
        distinct = len(np.unique(y[y >= 0]))
        P = int(rng.integers(max(distinct, 1), V + 1))
        p = rng.integers(-1, V, T) if it % 2 else None
        stride = int(rng.integers(1, 10 * V))
        while np.gcd(stride, V) != 1:
            stride += 1
        _check(y, p, V, P, stride, int(rng.integers(-10 * V, 10 * V)))


def test_fallback_and_wrap():
    V, P, stride = 4096, 2048, 1021
    y = (np.arange(1300) * stride) % V            # the first 1300 window classes: fallback
    ref = _check(y, None, V, P, stride, 0)
    assert ref["fallback"]
    ref = _check(np.array([3, 5, -1]), None, 1000, 300, 7, 995)  # window runs past the sweep's end
    assert not ref["fallback"]
    _check(np.zeros(0, dtype=np.int64), None, 1000, 1000, 7, 3)  # P = V, no labels


def test_asserted_conditions_are_flagged():
    V = 500
    y = np.arange(64, dtype=np.int64)
    out = binding.build_candidates_host(y, None, V, 50, 7, 0)      # 64 distinct > P = 50
    assert out["aux"][3].item() & binding.DEV_TOO_MANY_TARGETS
    assert np.array_equal(out["C"].numpy(), np.arange(50))
    with pytest.raises(OracleError):
        build_candidates(V, 50, 7, 0, y)
    y2 = np.array([3, V + 5, -7], dtype=np.int64)
    out = binding.build_candidates_host(y2, None, V, 50, 7, 0)
    assert out["aux"][3].item() & binding.DEV_LABEL_RANGE
    with pytest.raises(binding.SceError):
        binding.build_candidates_host(y2, None, V, 50, 2 * 5, 0)    # gcd(10, 500) != 1
