"""GPU parity of the polar-express orthogonalisation (sa_polar_express)
against the fp64 oracle on the same seeded bf16 gradients.

The GPU keeps X, A = X X^T and B = b A + c A A in bf16 between products, as
a bf16 optimizer step does, so it is compared with the exact fp64 iteration
through measures that rounding cannot break: the relative Frobenius error of
each matrix and the range of its singular values."""

import pytest
import torch

import oracle
from gpu_helpers import (POLAR_TILE_REL, POLAR_TILE_REL_DEFAULT, log, polar_tile_rel_errors,
                         set_cpu_threads)

pytestmark = pytest.mark.gpu

# Relative Frobenius error bound, per matrix (see the design notes for the
# derivation: bf16 storage of X, A and B at each of the five steps, with the
# first step's coefficients amplifying a relative perturbation by about
# (|a| + |b| + |c|) / |a + b + c| ~ 30 near the top of the spectrum).
POLAR_REL_FRO = 5e-2


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    set_cpu_threads()
    import qk_normed_sliding_amd as pkg
    return pkg


def _grad(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _check(sa, g, steps=5, idx=None):
    out = sa.sa_polar_express(g.cuda(), steps=steps)
    torch.cuda.synchronize()
    out = out.cpu()
    idx = range(g.shape[0]) if idx is None else idx
    worst = worst_tile = 0.0
    tile_bound = POLAR_TILE_REL.get(steps, POLAR_TILE_REL_DEFAULT)
    for i in idx:
        ref = oracle.polar_express(g[i:i + 1], steps=steps)[0]
        got = out[i].double()
        assert torch.isfinite(got).all()
        err = float((got - ref).norm() / ref.norm())
        worst = max(worst, err)
        # every 128 x 128 tile on its own: a wrongly mirrored or split-K tile fails here
        worst_tile = max(worst_tile, float(polar_tile_rel_errors(got, ref).max()))
        if steps == 5:
            sv = torch.linalg.svdvals(got)
            sr = torch.linalg.svdvals(ref)
            assert float(sv.max()) < float(sr.max()) + 0.1 and float(sv.min()) > float(sr.min()) - 0.1
    log(f"  {tuple(g.shape)} steps {steps}: worst rel-Frobenius {worst:.3e}, worst 128x128 tile {worst_tile:.3e}")
    assert worst <= POLAR_REL_FRO
    assert worst_tile <= tile_bound, f"a tile is off by {worst_tile:.3e} (bound {tile_bound})"
    return out


# K is split in ranges of at least 1024: (1, 128, 2048): one tile, the
# Gram's K split in 2; (1, 256, 2048): split in 2 with a mirrored
# off-diagonal tile; (2, 512, 3072): Gram split in 3; (1, 2048, 2048): the
# Gram and A A both split in 2, with mirrored tiles; (1, 384, 640) and
# (2, 1152, 384): B X in 96-row tiles (m = 384)
@pytest.mark.parametrize("shape", [(3, 256, 384), (2, 384, 256), (2, 256, 256), (1, 128, 2048), (1, 256, 2048),
                                   (2, 512, 3072), (1, 2048, 2048), (1, 384, 640), (2, 1152, 384)])
def test_polar_express_small(sa, shape):
    log(f"[polar] {shape}")
    _check(sa, _grad(shape, 300 + shape[1]))


@pytest.mark.parametrize("shape", [(1, 2048, 2048), (2, 512, 3072), (1, 256, 2048), (2, 384, 256), (1, 384, 640)])
def test_polar_express_one_step_tiles(sa, shape):
    """One step, where the per-tile bound is tight (1e-2): the symmetric
    products' mirrored tiles and the split-K reductions (K = 2048: A = X X^T
    and A A both split in two, with mirrored tiles; K = 3072: the Gram in
    three) against the exact iteration, tile by tile."""
    log(f"[polar, 1 step] {shape}")
    _check(sa, _grad(shape, 350 + shape[1]), steps=1)


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_polar_express_steps(sa, steps):
    log(f"[polar] steps {steps}")
    _check(sa, _grad((2, 256, 512), 400), steps=steps)


@pytest.mark.parametrize("shape", [(32, 768, 768), (8, 768, 3072), (8, 3072, 768)])
def test_polar_express_model_shape_groups(sa, shape):
    """The trainer's Muon groups at n_embd 768: attention projections and the
    MLP's two matrices, every matrix of the stack computed, two compared."""
    log(f"[polar] model group {shape}")
    g = _grad(shape, 500 + shape[2])
    _check(sa, g, idx=[0, shape[0] - 1])
    # one step, tile by tile, on more matrices of the stack
    _check(sa, g, steps=1, idx=sorted({0, 1, shape[0] // 2, shape[0] - 2, shape[0] - 1}))


def test_polar_express_transpose_symmetry(sa):
    """The iteration commutes with transposition, and a tall stack and its
    transpose go through different products (Y^T Y and Y B + a Y on the tall
    matrix, X X^T and B X + a X on the wide one), so the results agree up to
    bf16 rounding: each against the oracle, and the two against each other
    within the same relative-Frobenius bound."""
    g = _grad((2, 512, 256), 77)
    gt = g.transpose(-2, -1).contiguous()
    _check(sa, g)
    _check(sa, gt)
    a = sa.sa_polar_express(g.cuda()).cpu().double()
    b = sa.sa_polar_express(gt.cuda()).cpu().double().transpose(-2, -1)
    for i in range(g.shape[0]):
        rel = float((a[i] - b[i]).norm() / b[i].norm())
        log(f"  tall vs wide, matrix {i}: rel-Frobenius {rel:.3e}")
        assert rel <= POLAR_REL_FRO


def test_polar_express_matrices_are_independent(sa):
    g = _grad((3, 256, 384), 81)
    full = sa.sa_polar_express(g.cuda())
    one = sa.sa_polar_express(g[1:2].contiguous().cuda())
    assert torch.equal(full[1:2], one)
