"""fp64 CPU oracle for Muon's polar-express orthogonalisation.

TEST INFRASTRUCTURE ONLY (same rules as oracle/attention.py): only the tests,
the smoke check and the benchmark's CPU-baseline leg may use it; it shares no
code with the HIP path.

Source: "autoresearch Administrator & Developer Guide", section 8.2.3 (Muon
step internals): five (a, b, c) coefficient triples applied in order; each
step forms A = X^T X or X X^T (whichever is the smaller square), then
B = b A + c A A and X <- a X + X B (or a X + B X for the X X^T side).

Reading where the guide is silent: the iteration starts from the gradient
divided by its Frobenius norm (plus a tiny guard), which bounds every
singular value by 1, the range the coefficients are made for.

In exact arithmetic a step maps X = U diag(s) V^T to U diag(a s + b s^3 + c s^5) V^T:
A = V diag(s^2) V^T (or U diag(s^2) U^T), and both update forms give the
same odd polynomial of X. The pins use exactly this.
"""

from __future__ import annotations

import torch

F64 = torch.float64

# [guide] 8.2.3, the printed coefficient list, in order.
POLAR_EXPRESS_COEFFS = (
    (8.156554524902461, -22.48329292557795, 15.878769915207462),
    (4.042929935166739, -2.808917465908714, 0.5000178451051316),
    (3.8916678022926607, -2.772484153217685, 0.5060648178503393),
    (3.285753657755655, -2.3681294933425376, 0.46449024233003106),
    (2.3465413258596377, -1.7097828382687081, 0.42323551169305323),
)


def normalize(g: torch.Tensor, eps: float = 1e-7) -> torch.Tensor:
    """X0 = G / (||G||_F + eps), per matrix of a [..., m, n] stack (float64)."""
    g = g.to(F64)
    nrm = torch.sqrt((g * g).sum(dim=(-2, -1), keepdim=True))
    return g / (nrm + eps)


def polar_step(x: torch.Tensor, a: float, b: float, c: float) -> torch.Tensor:
    """One step on a [..., m, n] stack: the smaller Gram matrix, then the update."""
    m, n = x.shape[-2], x.shape[-1]
    if m > n:  # tall: A = X^T X (n x n), X <- a X + X B
        A = x.transpose(-2, -1) @ x
        B = b * A + c * (A @ A)
        return a * x + x @ B
    A = x @ x.transpose(-2, -1)  # wide or square: A = X X^T (m x m), X <- a X + B X
    B = b * A + c * (A @ A)
    return a * x + B @ x


def polar_express(g: torch.Tensor, steps: int = 5, eps: float = 1e-7) -> torch.Tensor:
    """Muon's orthogonalisation of a [..., m, n] stack of gradients (float64)."""
    if not 1 <= steps <= len(POLAR_EXPRESS_COEFFS):
        raise ValueError(f"steps must be in [1, {len(POLAR_EXPRESS_COEFFS)}]")
    x = normalize(g, eps)
    for a, b, c in POLAR_EXPRESS_COEFFS[:steps]:
        x = polar_step(x, a, b, c)
    return x
