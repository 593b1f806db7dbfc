"""GPU tests of comba_check_inputs, the on-demand check of the device-side
preconditions (alpha in (0, 1]; cu_seqlens from 0 to T, non-decreasing), and
of the binding's COMBA_DEBUG_CHECKS mode that runs it before every call."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import bilinear_rnn_amd as comba
from bilinear_rnn_amd import api
from bilinear_rnn_amd.inputs import WORKLOADS, make_inputs
from _util import dev_inputs

pytestmark = pytest.mark.gpu

A, O, B_ = api.COMBA_CHECK_ALPHA_RANGE, api.COMBA_CHECK_CU_ORDER, api.COMBA_CHECK_CU_BOUNDS


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def alpha_of(shape=(2, 300, 3), seed=5):
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.uniform(0.05, 1.0, shape).astype(np.float32)).cuda()


def test_valid_inputs_pass():
    a = alpha_of()
    assert comba.check_inputs(a) == 0
    a[0, 0, 0] = 1.0            # the closed end of (0, 1]
    a[1, 5, 2] = 1e-38          # positive, below the smallest normal float
    assert comba.check_inputs(a) == 0
    cu = torch.tensor([0, 0, 70, 300], dtype=torch.int32, device="cuda")  # an empty sequence is allowed
    assert comba.check_inputs(a[:1].contiguous(), cu, T=300) == 0


@pytest.mark.parametrize("value", [0.0, -0.5, 1.0000001, 2.0, math.nan, math.inf, -math.inf])
@pytest.mark.parametrize("where", [(0, 0, 0), (1, 299, 2), (1, 150, 1)])
def test_alpha_out_of_range_is_flagged(value, where):
    a = alpha_of()
    a[where] = value
    assert comba.check_inputs(a) == A
    assert comba.check_inputs(a, check_alpha=False) == 0


def test_one_bad_alpha_at_the_end_of_a_full_size_layer():
    w = WORKLOADS["layer_1p3b"]
    a = alpha_of((w.B, w.T, w.H))
    assert comba.check_inputs(a) == 0
    a.view(-1)[-1] = 0.0
    assert comba.check_inputs(a) == A


@pytest.mark.parametrize("cu,T,expect", [
    ([0, 70, 40, 300], 300, O),            # decreasing
    ([1, 70, 300], 300, B_),               # does not start at 0
    ([0, 70, 299], 300, B_),               # does not end at T
    ([0, 200, 100, 301], 300, O | B_),     # both
    ([0, 300], 300, 0),
])
def test_cu_seqlens_flags(cu, T, expect):
    a = alpha_of((1, 300, 2))
    assert comba.check_inputs(a, torch.tensor(cu, dtype=torch.int32, device="cuda"), T=T) == expect


def test_flags_word_is_cleared_by_each_call():
    a = alpha_of()
    a[0, 1, 1] = 0.0
    assert comba.check_inputs(a) == A
    a[0, 1, 1] = 0.5
    assert comba.check_inputs(a) == 0


def test_debug_mode_raises_before_launching(monkeypatch):
    inp = make_inputs(dataclasses.replace(WORKLOADS["layer_340m"], B=1, H=2), T=130, s0_std=0.02, seed=9)
    t = dev_inputs(inp)
    args = (t["q"], t["k"], t["v"], t["alpha"], t["beta"], t["d"], t["initial_state"])
    o_ref, s_ref = comba.chunk_fwd(*args)
    monkeypatch.setattr(api, "DEBUG_CHECKS", True)
    o, s = comba.chunk_fwd(*args)      # valid inputs: same results with the check in front
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    bad = t["alpha"].clone()
    bad[0, 64, 1] = 0.0
    with pytest.raises(comba.CombaError, match="alpha outside"):
        comba.chunk_fwd(t["q"], t["k"], t["v"], bad, t["beta"], t["d"], t["initial_state"])
    with pytest.raises(comba.CombaError, match="alpha outside"):
        comba.recurrent_step(t["q"][:, :1].contiguous(), t["k"][:, :1].contiguous(), t["v"][:, :1].contiguous(),
                             bad[:, 64:65].contiguous(), t["beta"][:, :1].contiguous(), t["d"], t["initial_state"])
