"""GPU parity of dspark_schedule against the oracle, through the C ABI.

Confidences and throughput curves are seeded and synthetic: uniform
confidences, confidences with repeats and exact 0/1 values, and the verify
step's own alphas; curves with steps (a batch spilling into the next
hardware tile), random curves and linear ones. The lengths are integers
decided by floating point: they must equal the oracle's unless the oracle's
two best batch sizes are within 1e-12 (relative) of each other, in which
case the GPU's choice must be one of them (counted)."""

import numpy as np
import pytest
import torch

import lossless_verify_tv_amd as lv
from lossless_verify_tv_amd import synth
from oracle import schedule as osch

from .gpu_util import announce, device, verify_inputs

pytestmark = pytest.mark.gpu

THETA_RTOL = 1e-12


def _curve(rng, R, L, kind):
    B = np.arange(R * (L + 1) + 1, dtype=np.float64)
    if kind == "steps":
        tile = max(1, R // 2)
        return (4000.0 / (1.0 + np.floor(B / tile)) + rng.uniform(0, 5, B.size)).astype(np.float32)
    if kind == "random":
        return rng.uniform(1.0, 100.0, B.size).astype(np.float32)
    return (B.size * 3.0 - 2.0 * B).astype(np.float32)


def _run(conf, sps):
    dev = device()
    lens, best = lv.dspark_schedule(torch.from_numpy(conf).to(dev), torch.from_numpy(sps).to(dev))
    torch.cuda.synchronize(dev)
    return lens.cpu().numpy(), best.cpu().numpy()


def _check(conf, sps, tag):
    lens_g, best_g = _run(conf, sps)
    lens_o, best_o, B_o, theta = osch.schedule(conf, sps)
    R = conf.shape[0]
    B_g = int(best_g[1])
    assert B_g == R + int(lens_g.sum()), tag
    if B_g == B_o:
        assert np.array_equal(lens_g, lens_o), tag
        excused = 0
    else:
        # a near-tie between two batch sizes: the GPU's must be as good
        assert abs(theta[B_g - R] - best_o) <= THETA_RTOL * abs(best_o), (tag, B_g, B_o)
        excused = 1
    assert best_g[0] == pytest.approx(best_o, rel=THETA_RTOL), tag
    # the GPU's lengths achieve its Theta by the definition
    assert osch.objective(conf, sps, lens_g) == pytest.approx(best_g[0], rel=1e-9), tag
    return excused


@pytest.mark.parametrize("kind", ["steps", "random", "linear"])
@pytest.mark.parametrize("R,L", [(1, 1), (1, 16), (7, 5), (64, 8), (256, 16), (512, 16),
                                 (8192, 1), (1000, 8), (33, 31), (3, 2730), (1, 8192)])
def test_schedule_against_oracle(kind, R, L):
    rng = np.random.default_rng(R * 100 + L + {"steps": 0, "random": 1, "linear": 2}[kind])
    excused = 0
    for rep in range(3):
        conf = rng.uniform(0.05, 1.0, (R, L)).astype(np.float32)
        if rep == 1:   # repeats, exact 0 and 1, out-of-range and NaN entries
            conf = np.round(conf * 4) / 4
            conf.ravel()[:: 11] = 1.0
            conf.ravel()[5:: 13] = 0.0
            if conf.size > 20:
                conf.ravel()[3] = 1.7
                conf.ravel()[7] = -0.2
                conf.ravel()[9] = np.nan
        excused += _check(conf, _curve(rng, R, L, kind), f"{kind} R={R} L={L} rep={rep}")
    announce(f"schedule {kind} R={R} L={L}: near-tie batch choices {excused}")


def test_schedule_from_verify_alphas():
    """The pages' soft label for the confidences is 1 - d_TV, which is the
    verify step's alpha: schedule straight from spec_verify's output."""
    dev = device()
    case = synth.verify_case(3, temperature=1.0)
    acc, toks, alpha, status = lv.spec_verify(**verify_inputs(case, dev))
    conf = alpha.contiguous()
    R, L = conf.shape
    rng = np.random.default_rng(9)
    sps = _curve(rng, R, L, "steps")
    lens, best = lv.dspark_schedule(conf, torch.from_numpy(sps).to(dev))
    torch.cuda.synchronize(dev)
    _check(conf.cpu().numpy(), sps, "from alphas")
    assert np.all((lens.cpu().numpy() >= 0) & (lens.cpu().numpy() <= L))
