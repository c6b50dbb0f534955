"""sce_build_candidates_noalloc (the candidate build with the library's static scratch)
against sce_build_candidates with a caller workspace, bit for bit, on consecutive calls
whose second input is smaller (the scratch keeps the first call's contents), and against
the oracle."""
import numpy as np
import pytest
import torch

from oracle import build_candidates
from sampled_softmax_cross_amd import binding, synth
from tests.gpu_util import labels_dev

pytestmark = pytest.mark.gpu

KEYS = ("C", "target_pos", "prefix_pos", "vocab_pos", "aux")


def _case(seed, T, V, prefix):
    _, _, y, p = synth.small_case(seed, T, 8, V, "f32", prefix=prefix, ignore_frac=0.05)
    return y, p


def _check(y, p, V, P, stride, offset, want_prefix_pos):
    yd, pd = labels_dev(y), labels_dev(p)
    ref = binding.build_candidates(yd, pd, V, P, stride, offset, want_vocab_pos=True)
    got = binding.build_candidates_noalloc(yd, pd, V, P, stride, offset, want_vocab_pos=True,
                                           want_prefix_pos=want_prefix_pos)
    torch.cuda.synchronize()
    for k in KEYS:
        if k == "prefix_pos" and not want_prefix_pos:
            continue
        assert torch.equal(got[k], ref[k]), k
    orc = build_candidates(V, P, stride, offset, y, p)
    assert np.array_equal(got["C"].cpu().numpy(), orc["C"])
    assert np.array_equal(got["target_pos"].cpu().numpy(), orc["target_pos"])
    assert np.array_equal(got["vocab_pos"].cpu().numpy(), orc["vocab_pos"])
    aux = got["aux"].cpu().tolist()
    assert aux == [orc["num_targets"], orc["N"], orc["next_offset"], 0]
    if want_prefix_pos:
        assert np.array_equal(got["prefix_pos"].cpu().numpy(), orc["prefix_pos"])


@pytest.mark.parametrize("want_prefix_pos", [True, False])
def test_noalloc_matches_workspace_build_twice(want_prefix_pos):
    # first call: the stage-0/1 vocabulary and sizes; second: smaller in T, V and P
    print(f"noalloc build, prefix positions returned: {want_prefix_pos}", flush=True)
    y, p = _case(1, 16384, 50304, True)
    _check(y, p, 50304, 10240, 20011, 16384, want_prefix_pos)
    y, p = _case(2, 300, 1000, True)
    _check(y, p, 1000, 333, 7, 5, want_prefix_pos)


def test_noalloc_vocabulary_limit_and_no_prefix():
    print("noalloc build at V = SCE_MAX_V_SAMPLED, then without prefix targets", flush=True)
    y, p = _case(3, 4096, binding.MAX_V_SAMPLED, True)
    _check(y, p, binding.MAX_V_SAMPLED, 40000, 99991, 77, False)
    y, _ = _case(4, 512, 4096, False)
    _check(y, None, 4096, 2048, 1021, 0, False)
