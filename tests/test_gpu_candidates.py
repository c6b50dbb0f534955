"""GPU candidate build (sce_build_candidates) vs the oracle: bit-exact integers."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import build_candidates
from sampled_softmax_cross_amd import binding, synth
from tests.gpu_util import labels_dev

pytestmark = pytest.mark.gpu


def _run(V, P, stride, offset, y, p):
    r = binding.build_candidates(labels_dev(y), labels_dev(p), V, P, stride, offset,
                                 want_vocab_pos=True)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if torch.is_tensor(v) else v) for k, v in r.items()}


def _check(V, P, stride, offset, y, p):
    g = _run(V, P, stride, offset, y, p)
    o = build_candidates(V, P, stride, offset, y, p)
    assert g["aux"][3] == 0
    assert np.array_equal(g["C"], o["C"])
    assert np.array_equal(g["vocab_pos"], o["vocab_pos"])
    assert np.array_equal(g["target_pos"], o["target_pos"])
    assert np.array_equal(g["prefix_pos"], o["prefix_pos"])
    assert g["aux"].tolist() == [o["num_targets"], o["N"], o["next_offset"], 0]
    return g, o


def test_handworked_cases(golden_dir):
    with open(os.path.join(golden_dir, "candidates_handworked.json")) as f:
        for c in json.load(f)["cases"]:
            print("case", c["name"], flush=True)
            y = np.array(c["targets"], dtype=np.int64)
            p = None if c["prefix"] is None else np.array(c["prefix"], dtype=np.int64)
            g, _ = _check(c["V"], c["P"], c["stride"], c["offset"], y, p)
            assert g["C"].tolist() == c["C"]


@pytest.mark.parametrize("seed,V,P,stride,T,s,prefix", [
    (0, 4096, 2048, 1021, 512, 1.1, False),
    (1, 4096, 700, 1021, 300, 1.1, True),
    (2, 50304, 10240, 20011, 16384, 1.1, False),
    (3, 50304, 14336, 20011, 49152, 1.05, True),
    (4, 50304, 24576, 20011, 49152, 1.05, True),
    (5, 1000, 333, 7, 200, 0.8, True),
    (6, 999, 998, 2, 50, 1.0, True),
    (7, 131072, 40000, 99991, 8000, 1.0, True),
    (8, 33, 33, 5, 40, 1.0, True),
    (9, 1, 1, 1, 3, 1.0, True),
])
def test_random_cases(seed, V, P, stride, T, s, prefix):
    perm = synth.class_permutation(seed, V)
    y = synth.zipf_classes(seed, 4, T, V, s, perm)
    p = synth.zipf_classes(seed, 5, T, V, s, perm) if prefix else None
    if seed % 2:
        y[::7] = -1
        if p is not None:
            p[::5] = -1
    for offset in (0, (seed * T) % V, V - 1, -3):
        print("seed", seed, "V", V, "P", P, "offset", offset, flush=True)
        _check(V, P, stride, offset, y, p)


def test_fallback_branch():
    V, P, stride = 4096, 2048, 1021
    y = (np.arange(1300, dtype=np.int64) * stride) % V
    g, o = _check(V, P, stride, 0, y, None)
    assert o["fallback"]


def test_p_equals_v_and_need_zero():
    V = 4096
    y = synth.zipf_classes(3, 4, 512, V, 1.1, synth.class_permutation(3, V))
    g, _ = _check(V, V, 1021, 5, y, None)
    assert np.array_equal(g["C"], np.arange(V))
    distinct = np.unique(y)
    g, o = _check(V, distinct.size, 1021, 5, y, None)
    assert np.array_equal(g["C"], distinct) and g["aux"][2] == 5


def test_device_detected_errors():
    V = 100
    y = np.arange(10, dtype=np.int64)
    g = _run(V, 9, 3, 0, y, None)       # 10 distinct targets > P = 9
    assert g["aux"][3] & binding.DEV_TOO_MANY_TARGETS
    # the map left behind keeps every later access in bounds: C = [0, P), positions
    # of the first P classes, -1 elsewhere
    assert np.array_equal(g["C"], np.arange(9))
    assert np.array_equal(g["vocab_pos"], np.where(np.arange(V) < 9, np.arange(V), -1))
    assert np.array_equal(g["target_pos"], np.where(y < 9, y, -1))
    g = _run(V, 20, 3, 0, np.array([1, 100], dtype=np.int64), None)
    assert g["aux"][3] & binding.DEV_LABEL_RANGE
    g = _run(V, 20, 3, 0, np.array([1, 2], dtype=np.int64), np.array([-2, 5], dtype=np.int64))
    assert g["aux"][3] & binding.DEV_LABEL_RANGE
    # a clean call after the failing ones is unaffected (state lives in the workspace)
    _check(V, 20, 3, 0, y, None)
