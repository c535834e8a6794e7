"""Randomised parity sweep of replay attention against the fp64 oracle.

Each case draws, from its own fixed seed, a head shape (D = 64 or 128 with a GQA ratio, or latent
KV 576/512), a prompt length (including 0 and lengths just past a tile boundary), one to four
responses of 1 to 300 tokens, and a call mode (one call over all responses, or one call per
response accumulating the prompt gradients). Shapes are small so that the oracle finishes in well
under a second; together the cases cover many tile remainders and response boundaries."""
import numpy as np
import pytest

from prefix_shared_branch_amd import inputs
from tests.test_gpu_attn import Case, _check_all, _serial

pytestmark = pytest.mark.gpu

SHAPES = [(64, 8, 2), (64, 4, 4), (64, 6, 1), (128, 8, 2), (128, 10, 2), (128, 3, 3), ("mla", 16, 1)]


def _draw(seed):
    g = np.random.default_rng(seed)
    shape = SHAPES[g.integers(len(SHAPES))]
    P = int(g.choice([0, 1, 63, 64, 65, 127, 129, 1000, 2049, 3001]))
    n = int(g.integers(1, 5))
    lengths = [int(x) for x in g.integers(1, 301, size=n)]
    serial = bool(g.integers(2)) and n > 1
    return shape, P, lengths, serial


@pytest.mark.parametrize("seed", list(range(900, 924)))
def test_random_case(seed):
    shape, P, lengths, serial = _draw(seed)
    if shape[0] == "mla":
        cfg = inputs.replace(inputs.CONFIGS["mla"], P=P, seed=seed)
    else:
        D, Hq, Hkv = shape
        cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=Hq, Hkv=Hkv, Dqk=D, Dv=D, P=P, seed=seed)
    case = Case(cfg, lengths)
    exact = P > 0
    if serial and exact:
        got = _serial(case)
    else:
        t = case.torch
        dkp, dvp = case.accums() if exact else (None, None)
        o, lse = case.fwd()
        dq, dks, dvs = case.bwd(o, lse, dkp, dvp)
        t.cuda.synchronize()
        got = dict(O=o, LSE=lse, dQ=dq, dKs=dks, dVs=dvs, dKp=dkp, dVp=dvp)
    # with a short or empty prompt, gradients are of order one: the relative bars apply
    _check_all(got, case.oracle(accumulate=exact), literal_abs=P >= 1000)


def _draw_blocks(seed):
    g = np.random.default_rng(seed)
    shape = SHAPES[g.integers(len(SHAPES))]
    P = int(g.choice([0, 1, 63, 65, 1000, 2049]))
    R = int(g.integers(1, 401))
    nb = int(g.integers(1, 5))
    cuts = sorted({int(c) for c in g.integers(1, R, size=nb - 1)}) if R > 1 else []
    return shape, P, R, [0, *cuts, R]


@pytest.mark.parametrize("seed", list(range(950, 962)))
def test_random_blocks(seed):
    """One response replayed in randomly cut blocks against the unblocked oracle."""
    from tests.test_gpu_block import _blockwise, _check
    shape, P, R, bounds = _draw_blocks(seed)
    if shape[0] == "mla":
        cfg = inputs.replace(inputs.CONFIGS["mla"], P=P, seed=seed)
    else:
        D, Hq, Hkv = shape
        cfg = inputs.replace(inputs.CONFIGS["tiny"], Hq=Hq, Hkv=Hkv, Dqk=D, Dv=D, P=P, seed=seed)
    case = Case(cfg, [R])
    exact = P > 0
    _check(_blockwise(case, bounds, exact), case.oracle(accumulate=exact), exact, literal_abs=P >= 1000)
