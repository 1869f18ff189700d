"""GPU threshold calibration against the oracle's quantile: bit-exact fp32.

The oracle (numpy's linear-interpolation quantile of |v| in fp64, rounded to
fp32) is the reference; the library finds the two order statistics by a
radix select on the GPU and interpolates them the same way."""
import numpy as np
import pytest
import torch

import activation_sparse_expert_amd as moe
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(v, q):
    t = moe.calibrate_threshold(torch.from_numpy(v).to(DEV), q)
    torch.cuda.synchronize()
    return np.float32(t.cpu().numpy()[0])


@pytest.mark.parametrize("n", [1, 2, 3, 1000, 65537, 917504])
@pytest.mark.parametrize("q", [0.0, 0.5, 0.7, 0.9, 1.0, 0.123456789])
def test_quantile_matches_oracle(n, q):
    rng = np.random.default_rng(n * 1000 + int(q * 1e6))
    v = (rng.standard_normal(n) * 0.02).astype(np.float32)
    got = run(v, q)
    want = oracle.calibrate_threshold(np.abs(v), q)
    assert got == want, f"n={n} q={q}: {got!r} vs {want!r}"


def test_quantile_ties_wide_range_and_signs():
    rng = np.random.default_rng(7)
    # repeated values, zeros, negative zero, subnormals and a wide exponent range
    base = np.array([0.0, -0.0, 1e-40, -1e-40, 3.0, -3.0, 1e30, 5e-8], dtype=np.float32)
    v = np.concatenate([np.repeat(base, 257), rng.standard_normal(4000).astype(np.float32) * 1e3])
    rng.shuffle(v)
    for q in (0.0, 0.01, 0.25, 0.5, 0.75, 0.9, 0.999, 1.0):
        got = run(v, q)
        want = oracle.calibrate_threshold(np.abs(v), q)
        assert got == want, f"q={q}: {got!r} vs {want!r}"


def test_calibration_from_the_expert_v_export():
    """The calibration flow the library supports: v of the calibration tokens
    exported by the expert call, then the quantile on the GPU."""
    import synth
    from gpu_helpers import HostExpert
    hx = HostExpert(synth.CFG_TINY, 3, 0, 256, 704)
    ex = hx.to_device(float("inf"))
    xc = torch.from_numpy(synth.calibration_f32(synth.CFG_TINY, 256, 1 / 16, 3, 0)).half().to(DEV)
    v = torch.empty((64, 704), dtype=torch.float32, device=DEV)
    moe.expert_forward_sparse(ex, xc, v_out=v)
    torch.cuda.synchronize()
    for q in (0.5, 0.9):
        got = np.float32(moe.calibrate_threshold(v, q).cpu().numpy()[0])
        want = oracle.calibrate_threshold(np.abs(v.cpu().numpy()), q)
        assert got == want
