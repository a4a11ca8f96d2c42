"""Pins of the polar-express oracle (oracle/muon.py) against facts it does not
compute itself: the constants the guide prints (golden file), the SVD
(torch.linalg.svd) with a scalar polynomial on the singular values, and the
transpose symmetry of the two update forms. Planted mistakes must fail."""

import os

import pytest
import torch

import oracle
from oracle import muon as OM

F64 = torch.float64
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "polar_express_coeffs.txt")


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=F64)


def _golden_coeffs():
    rows = []
    for ln in open(GOLDEN):
        ln = ln.strip()
        if ln and not ln.startswith("#"):
            rows.append(tuple(float(x) for x in ln.split()))
    return rows


def test_coefficients_are_the_printed_ones():
    assert list(OM.POLAR_EXPRESS_COEFFS) == _golden_coeffs()


def _svd_reference(g, steps):
    """U p_steps(...p_1(s)) V^T with s the singular values of G / ||G||_F (library SVD and norm)."""
    x = g / torch.linalg.matrix_norm(g, ord="fro", keepdim=True)
    u, s, vh = torch.linalg.svd(x, full_matrices=False)
    for a, b, c in _golden_coeffs()[:steps]:
        s = a * s + b * s ** 3 + c * s ** 5
    return u @ torch.diag_embed(s) @ vh


@pytest.mark.parametrize("shape", [(3, 24, 40), (2, 40, 24), (2, 32, 32), (1, 7, 5)])
@pytest.mark.parametrize("steps", [1, 3, 5])
def test_iteration_acts_on_singular_values(shape, steps):
    g = _rand(shape, 11 + shape[1])
    x = oracle.polar_express(g, steps=steps, eps=0.0)
    assert torch.allclose(x, _svd_reference(g, steps), atol=1e-11)


def test_tall_and_wide_forms_agree_by_transpose():
    g = _rand((2, 48, 20), 5)
    a = oracle.polar_express(g)
    b = oracle.polar_express(g.transpose(-2, -1).contiguous()).transpose(-2, -1)
    assert torch.allclose(a, b, atol=1e-12)


def test_five_steps_bring_singular_values_near_one():
    """Singular values spread over [1e-2, 1] (about [4e-3, 0.4] after the
    Frobenius scaling): after the five printed steps all lie within 0.15 of 1
    (the behaviour the precomputed coefficients are made for; the SVD check
    above is the exact pin)."""
    u, _ = torch.linalg.qr(_rand((64, 64), 1))
    v, _ = torch.linalg.qr(_rand((96, 64), 2))
    s = torch.logspace(-2, 0, 64, dtype=F64)
    g = (u @ torch.diag(s) @ v.T).unsqueeze(0)
    sv = torch.linalg.svdvals(oracle.polar_express(g))
    assert float((sv - 1).abs().max()) < 0.15


def test_zero_matrix_stays_zero():
    assert torch.equal(oracle.polar_express(torch.zeros(1, 8, 12, dtype=F64)), torch.zeros(1, 8, 12, dtype=F64))


# ------------------------------------------------------------------ planted mistakes

def _pins_pass():
    for shape in ((2, 24, 40), (2, 40, 24)):
        g = _rand(shape, 21)
        if not torch.allclose(oracle.polar_express(g, eps=0.0), _svd_reference(g, 5), atol=1e-11):
            return False
    return list(OM.POLAR_EXPRESS_COEFFS) == _golden_coeffs()


def _mut_step_dropped_square(x, a, b, c):
    m, n = x.shape[-2], x.shape[-1]
    A = x.transpose(-2, -1) @ x if m > n else x @ x.transpose(-2, -1)
    B = b * A + c * A  # A instead of A A
    return a * x + (x @ B if m > n else B @ x)


def _mut_normalize_max(g, eps=1e-7):
    g = g.to(F64)
    return g / (g.abs().amax(dim=(-2, -1), keepdim=True) + eps)  # max entry instead of Frobenius norm


@pytest.mark.parametrize("name,mutant", [
    ("polar_step", _mut_step_dropped_square),
    ("normalize", _mut_normalize_max),
    ("POLAR_EXPRESS_COEFFS", tuple(reversed(OM.POLAR_EXPRESS_COEFFS))),
])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant):
    assert _pins_pass()
    monkeypatch.setattr(OM, name, mutant)
    assert not _pins_pass(), f"planted mistake in {name} went unnoticed"


def test_polar_tile_check_catches_one_wrong_tile():
    """The GPU test's per-tile check, exercised on the oracle's own result: a
    copy passes, and one 128 x 128 tile made 25% wrong (as a wrong mirrored
    or split-K tile would be) fails the tile bound although the whole-matrix
    error stays within the per-matrix bound."""
    import sys, os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from gpu_helpers import POLAR_TILE_REL, polar_tile_rel_errors

    g = torch.randn((1, 768, 768), generator=torch.Generator().manual_seed(9), dtype=torch.float64)
    ref = oracle.polar_express(g, steps=1)[0]
    assert float(polar_tile_rel_errors(ref.clone(), ref).max()) == 0.0
    bad = ref.clone()
    bad[256:384, 512:640] *= 1.25
    whole = float((bad - ref).norm() / ref.norm())
    assert whole < 5e-2  # a whole-matrix bound alone would let it through
    assert float(polar_tile_rel_errors(bad, ref).max()) > POLAR_TILE_REL[1]
