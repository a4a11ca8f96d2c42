"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the HIP runtime
(so these run on a machine without a GPU; no kernel is launched here)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa_attn.h")
LIB = os.path.join(ROOT, "qk_normed_sliding_amd", "libsa_attn.so")

SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_ALIGN, SA_ERR_WORKSPACE, SA_ERR_HIP = range(7)


@pytest.fixture(scope="module")
def sa():
    if not os.path.exists(LIB):
        subprocess.run(["python", os.path.join(ROOT, "qk_normed_sliding_amd", "build.py")], check=True)
    import qk_normed_sliding_amd as pkg
    return pkg


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("sa_qknorm", "sa_attn_fwd", "sa_attn_fwd_workspace_bytes", "sa_attn_bwd", "sa_attn_bwd_workspace_bytes",
              "sa_status_string", "sa_abi_version", "sa_attn_fwd_rope", "sa_attn_bwd_rope",
              "sa_polar_express", "sa_polar_express_workspace_bytes", "sa_attn_fwd_ex", "sa_attn_bwd_ex",
              "sa_attn_ve_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(sa):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, missing
    # nothing else leaks out under an sa_ name
    extra = sorted(n for n in exported if n.startswith("sa_") and n not in _declared_functions())
    assert not extra, extra


def test_version_and_status_strings(sa):
    lib = sa.library()
    assert lib.sa_abi_version() == sa.ABI_VERSION
    for code in range(7):
        assert lib.sa_status_string(code)
    assert b"unknown" in lib.sa_status_string(99)


def _fwd(lib, q=16, k=16, v=16, o=16, lse=16, ws=256, ws_bytes=None, B=1, T=8, Hq=4, Hkv=2, D=64, W=-1,
         scale=0.125, norm=1, eps=1e-6):
    P = ctypes.c_void_p
    if ws_bytes is None:
        ws_bytes = lib.sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, D)
    return lib.sa_attn_fwd(P(q), P(k), P(v), P(o), P(lse), P(ws), ws_bytes, B, T, Hq, Hkv, D, W, scale, norm, eps,
                           None)


def test_forward_validation_paths(sa):
    lib = sa.library()
    assert _fwd(lib, q=0) == SA_ERR_NULL
    assert _fwd(lib, lse=0) == SA_ERR_NULL
    assert _fwd(lib, B=0) == SA_ERR_SHAPE
    assert _fwd(lib, T=-1) == SA_ERR_SHAPE
    assert _fwd(lib, Hq=3, Hkv=2) == SA_ERR_SHAPE
    assert _fwd(lib, Hkv=0) == SA_ERR_SHAPE
    assert _fwd(lib, W=-2) == SA_ERR_SHAPE
    assert _fwd(lib, scale=float("nan")) == SA_ERR_SHAPE
    assert _fwd(lib, eps=-1.0) == SA_ERR_SHAPE
    assert _fwd(lib, D=96) == SA_ERR_UNSUPPORTED
    assert _fwd(lib, D=256) == SA_ERR_UNSUPPORTED
    assert _fwd(lib, q=24) == SA_ERR_ALIGN
    assert _fwd(lib, o=8) == SA_ERR_ALIGN
    assert _fwd(lib, lse=2) == SA_ERR_ALIGN
    assert _fwd(lib, ws=0) == SA_ERR_WORKSPACE
    assert _fwd(lib, ws_bytes=16) == SA_ERR_WORKSPACE
    assert _fwd(lib, ws=128) == SA_ERR_WORKSPACE


def _bwd(lib, ws=256, ws_bytes=None, B=1, T=8, Hq=4, Hkv=2, D=64, W=-1, dq=16, null_lse=False):
    P = ctypes.c_void_p
    need = lib.sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, D)
    ws_bytes = need if ws_bytes is None else ws_bytes
    lse = 0 if null_lse else 16
    return lib.sa_attn_bwd(P(16), P(16), P(16), P(16), P(lse), P(16), P(dq), P(16), P(16), P(ws), ws_bytes,
                           B, T, Hq, Hkv, D, W, 0.125, 1, 1e-6, None)


def test_backward_validation_paths(sa):
    lib = sa.library()
    assert _bwd(lib, null_lse=True) == SA_ERR_NULL
    assert _bwd(lib, dq=0) == SA_ERR_NULL
    assert _bwd(lib, Hq=5, Hkv=2) == SA_ERR_SHAPE
    assert _bwd(lib, D=32) == SA_ERR_UNSUPPORTED
    assert _bwd(lib, ws=0) == SA_ERR_WORKSPACE
    assert _bwd(lib, ws_bytes=16) == SA_ERR_WORKSPACE
    assert _bwd(lib, ws=128) == SA_ERR_WORKSPACE  # not 256-byte aligned
    assert _bwd(lib, dq=8) == SA_ERR_ALIGN


def _fwd_rope(lib, cos=1024, sin=2048, stride=64, D=128, norm=1, scale=0.125, q=16, T=8):
    P = ctypes.c_void_p
    ws_bytes = lib.sa_attn_fwd_workspace_bytes(1, T, 4, 2, D)
    return lib.sa_attn_fwd_rope(P(q), P(16), P(16), P(16), P(16), P(256), ws_bytes, 1, T, 4, 2, D, -1, scale, norm,
                                1e-6, P(cos), P(sin), stride, None)


def _bwd_rope(lib, cos=1024, sin=2048, stride=64, D=128, norm=1):
    P = ctypes.c_void_p
    need = lib.sa_attn_bwd_workspace_bytes(1, 8, 4, 2, D)
    return lib.sa_attn_bwd_rope(P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(256), need,
                                1, 8, 4, 2, D, -1, 0.125, norm, 1e-6, P(cos), P(sin), stride, None)


def test_rope_validation_paths(sa):
    lib = sa.library()
    for call in (_fwd_rope, _bwd_rope):
        assert call(lib, cos=0) == SA_ERR_NULL
        assert call(lib, sin=0) == SA_ERR_NULL
        assert call(lib, stride=60) == SA_ERR_SHAPE     # fewer than D/2 entries per row
        assert call(lib, stride=66) == SA_ERR_SHAPE     # rows not 16-byte aligned
        assert call(lib, D=64, stride=30) == SA_ERR_SHAPE
        assert call(lib, cos=1028) == SA_ERR_ALIGN
        assert call(lib, sin=8) == SA_ERR_ALIGN
        assert call(lib, norm=0) == SA_ERR_UNSUPPORTED  # the fused turn rides on the QK-norm kernels
        assert call(lib, D=80) == SA_ERR_UNSUPPORTED
    # the logits of the fixed-maximum kernels must stay bounded
    assert _fwd_rope(lib, scale=2.0) == SA_ERR_UNSUPPORTED
    assert _fwd_rope(lib, q=0) == SA_ERR_NULL
    assert _fwd_rope(lib, T=0) == SA_ERR_SHAPE


def test_workspace_size(sa):
    lib = sa.library()
    # k_hat and v' (bf16 rows), 1/rms and gate (fp32 per row and KV head), each rounded to 256 B
    assert lib.sa_attn_fwd_workspace_bytes(16, 2048, 6, 3, 128) == 2 * (16 * 2048 * 3 * 128 * 2) + 2 * (
        16 * 2048 * 3 * 4)
    assert lib.sa_attn_fwd_workspace_bytes(1, 5, 4, 2, 64) == 2 * 1280 + 2 * 256
    assert lib.sa_attn_fwd_workspace_bytes(1, 5, 4, 3, 64) == 0
    B, T, Hq, Hkv, D = 16, 2048, 6, 3, 128
    rows = B * T * Hq
    r256 = lambda x: (x + 255) // 256 * 256
    # normed q rows, Delta, base-2 LSE, normed k rows, 1/rms of the k rows
    assert lib.sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, D) == r256(rows * D * 2) + 2 * r256(rows * 4) + r256(
        B * T * Hkv * D * 2) + r256(B * T * Hkv * 4)
    assert lib.sa_attn_bwd_workspace_bytes(B, T, 5, Hkv, D) == 0
    assert lib.sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, 80) == 0


def test_timing_hook_validation(sa):
    lib = sa.library()
    P = ctypes.c_void_p
    assert lib.sa_set_timing_events(5, None, None) == SA_ERR_SHAPE
    assert lib.sa_set_timing_events(-1, None, None) == SA_ERR_SHAPE
    assert lib.sa_set_timing_events(0, P(16), None) == SA_ERR_NULL
    assert lib.sa_set_max_workgroups(-1) == SA_ERR_SHAPE
    assert lib.sa_set_max_workgroups(3) == SA_OK
    assert lib.sa_set_max_workgroups(0) == SA_OK
    for k in (sa.SA_KERNEL_FWD, sa.SA_KERNEL_BWD_DQ, sa.SA_KERNEL_BWD_DKDV, sa.SA_KERNEL_FWD_KNORM,
              sa.SA_KERNEL_BWD_KNORM):
        assert lib.sa_set_timing_events(k, None, None) == SA_OK


def test_qknorm_validation_paths(sa):
    lib = sa.library()
    P = ctypes.c_void_p
    assert lib.sa_qknorm(P(16), P(16), None, 0, 128, 1e-6, None) == SA_OK  # empty: nothing to do
    assert lib.sa_qknorm(None, P(16), None, 4, 128, 1e-6, None) == SA_ERR_NULL
    assert lib.sa_qknorm(P(16), P(16), None, -1, 128, 1e-6, None) == SA_ERR_SHAPE
    assert lib.sa_qknorm(P(16), P(16), None, 4, 100, 1e-6, None) == SA_ERR_UNSUPPORTED
    assert lib.sa_qknorm(P(16), P(20), None, 4, 128, 1e-6, None) == SA_ERR_ALIGN
    assert lib.sa_qknorm(P(16), P(16), P(6), 4, 128, 1e-6, None) == SA_ERR_ALIGN


def test_sssl_windows_host_helper_matches_pages(sa):
    golden = os.path.join(ROOT, "tests", "golden", "sssl_8layer_map.txt")
    kinds = [ln.split()[1] for ln in open(golden) if ln.strip() and not ln.startswith("#")]
    w = sa.sssl_windows(8, 2048)
    assert ["global" if x == -1 else "local" for x in w] == kinds
    assert all(x == 1024 for x in w if x != -1)
    assert sa.sssl_windows(6, 8192)[-1] == -1
    assert sa.sssl_windows(8, 8192) == [4096, 4096, 4096, -1, 4096, 4096, 4096, -1]
    with pytest.raises(ValueError):
        sa.sssl_windows(4, 64, "SQ")


def test_binding_rejects_cpu_tensors(sa):
    import torch
    q = torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sa.sa_attn_fwd(q, k, k)


def test_polar_express_executed_flops_count_upper_tiles(sa):
    """The executed MFMA count: the symmetric products X X^T and A A compute
    their tiles on and above the diagonal only (21 of 36 at m = 768 in
    128 x 128 tiles, the tiles used without a device), the update the full
    product. (8, 768, 3072): m = 768, n = 3072, five steps."""
    m, n, b = 768, 3072, 8
    per_step = 21 * 128 * 128 * 2 * n + 21 * 128 * 128 * 2 * m + 2 * m * m * n
    got = sa.sa_polar_express_executed_flops(b, m, n, 5)
    assert got == b * 5 * per_step
    assert got < b * 5 * (4 * m * m * n + 2 * m ** 3)
    assert sa.sa_polar_express_executed_flops(b, n, m, 5) == got  # tall: the same products
    assert sa.sa_polar_express_executed_flops(1, 100, 128, 5) == 0.0


def test_polar_express_validation_paths(sa):
    lib = sa.library()
    P = ctypes.c_void_p
    r256 = lambda x: (x + 255) // 256 * 256
    # two X buffers on the wide side, A and B, the partial sums of the first
    # Gram product's diagonal (4 per 128 rows: 24 per matrix at m = 768), and
    # split-K partial tiles: the Gram X X^T (K = 3072) of 8 matrices has 21
    # upper tiles each, 168 workgroups; ranges are at least 1024 long, so its K
    # is split in 3 (504 workgroups, the most ranges allowed); A A (K = 768) is
    # not split: 3 x 168 fp32 tiles of 128 x 128
    assert lib.sa_polar_express_workspace_bytes(8, 768, 3072) == 2 * r256(8 * 768 * 3072 * 2) + 2 * r256(
        8 * 768 * 768 * 2) + r256(8 * 24 * 4) + r256(3 * 168 * 128 * 128 * 4)
    # 32 matrices of 768 x 768: 672 workgroups per Gram, no split, no partials
    assert lib.sa_polar_express_workspace_bytes(32, 768, 768) == 2 * r256(32 * 768 * 768 * 2) + 2 * r256(
        32 * 768 * 768 * 2) + r256(32 * 24 * 4)
    assert lib.sa_polar_express_workspace_bytes(8, 3072, 768) == lib.sa_polar_express_workspace_bytes(8, 768, 3072)
    assert lib.sa_polar_express_workspace_bytes(1, 100, 128) == 0
    # the GEMM grids are one-dimensional: batch x 128-tiles stays below 2^20
    assert lib.sa_polar_express_workspace_bytes(4096, 2048, 2048) == 0
    assert lib.sa_polar_express_workspace_bytes(4095, 2048, 2048) > 0

    def call(g=16, out=32, ws=256, ws_bytes=None, batch=2, rows=256, cols=384, steps=5, eps=1e-7):
        need = lib.sa_polar_express_workspace_bytes(batch, rows, cols)
        return lib.sa_polar_express(P(g), P(out), P(ws), need if ws_bytes is None else ws_bytes, batch, rows, cols,
                                    steps, eps, None)

    assert call(g=0) == SA_ERR_NULL
    assert call(out=0) == SA_ERR_NULL
    assert call(g=8) == SA_ERR_ALIGN
    assert call(rows=200) == SA_ERR_UNSUPPORTED
    assert call(cols=64) == SA_ERR_UNSUPPORTED
    assert call(batch=0) == SA_ERR_SHAPE
    assert call(steps=0) == SA_ERR_SHAPE
    assert call(steps=6) == SA_ERR_SHAPE
    assert call(eps=-1.0) == SA_ERR_SHAPE
    assert call(rows=32768, cols=32768) == SA_ERR_SHAPE
    assert call(ws=0) == SA_ERR_WORKSPACE
    assert call(ws_bytes=100) == SA_ERR_WORKSPACE
    assert call(ws=128) == SA_ERR_WORKSPACE


def test_value_embedding_validation_paths(sa):
    lib = sa.library()
    P = ctypes.c_void_p
    B, T, Hq, Hkv, D = 1, 8, 4, 2, 64
    r256 = lambda x: (x + 255) // 256 * 256
    rh = B * T * Hkv
    assert lib.sa_attn_ve_workspace_bytes(B, T, Hkv, D) == r256(rh * D * 2) + r256(rh * 4) + r256(1 * Hkv * 32 * 4)

    def fwd(x=4096, xs=768, w=8192, ids=12288, tab=16384, vocab=100, norm=1):
        ws = lib.sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, D)
        return lib.sa_attn_fwd_ex(P(16), P(16), P(16), P(16), P(16), P(256), ws, B, T, Hq, Hkv, D, -1, 0.125, norm,
                                  1e-6, None, None, 0, P(x), xs, P(w), P(ids), P(tab), vocab, None)

    def bwd(dve=20480, dw=24576, dx=28672, vws=32768, vws_bytes=None, ids=12288, fws=0, fws_bytes=None, norm=1,
            scale=0.125):
        ws = lib.sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, D)
        need = lib.sa_attn_ve_workspace_bytes(B, T, Hkv, D) if vws_bytes is None else vws_bytes
        fneed = lib.sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, D) if fws_bytes is None else fws_bytes
        return lib.sa_attn_bwd_ex(P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(16), P(256), ws,
                                  P(fws) if fws else None, fneed if fws else 0,
                                  B, T, Hq, Hkv, D, -1, scale, norm, 1e-6, None, None, 0,
                                  P(4096), 768, P(8192), P(ids), P(16384), 100,
                                  P(dve), P(dw), P(dx), P(vws), need, None)

    assert fwd(ids=0) == SA_ERR_NULL            # a partial group
    assert fwd(tab=0) == SA_ERR_NULL
    assert fwd(xs=16) == SA_ERR_SHAPE           # fewer than 32 channels
    assert fwd(xs=100) == SA_ERR_SHAPE          # rows not 16-byte aligned
    assert fwd(vocab=0) == SA_ERR_SHAPE
    assert fwd(vocab=1 << 24) == SA_ERR_SHAPE   # table past 32-bit offsets
    assert fwd(x=4100) == SA_ERR_ALIGN
    assert fwd(ids=12290) == SA_ERR_ALIGN
    assert fwd(norm=0) == SA_ERR_UNSUPPORTED
    assert bwd(dve=0) == SA_ERR_NULL
    assert bwd(dw=0) == SA_ERR_NULL
    assert bwd(dve=20488) == SA_ERR_ALIGN
    assert bwd(vws=0) == SA_ERR_WORKSPACE
    assert bwd(vws_bytes=64) == SA_ERR_WORKSPACE
    assert bwd(vws=32768 + 128) == SA_ERR_WORKSPACE
    # the forward's workspace handed back to the backward
    assert bwd(fws=65536, fws_bytes=64) == SA_ERR_WORKSPACE          # too small
    assert bwd(fws=65536 + 128) == SA_ERR_WORKSPACE                  # not 256-byte aligned
    assert bwd(fws=65536, scale=2.0) == SA_ERR_UNSUPPORTED           # beyond the fixed row maximum


def test_rope_tables_helper_matches_the_oracle(sa):
    """The binding's rotary-table helper (the angle ladder t * base^(-2i/D)
    the GPU tests hand to both sides) is pinned to the oracle's tables, so a
    wrong frequency ladder cannot pass the GPU parity tests unnoticed."""
    import torch

    import oracle

    for n_pos, D in ((20480, 128), (4096, 64), (7, 16)):
        cos, sin = sa.rope_tables(n_pos, D)
        rc, rs = oracle.rope_tables(n_pos, D)
        assert cos.dtype == torch.float32 and tuple(cos.shape) == (n_pos, D // 2)
        # fp32 storage of values in [-1, 1]: within half an ulp of 1.0
        assert float((cos.double() - rc).abs().max()) <= 6e-8
        assert float((sin.double() - rs).abs().max()) <= 6e-8
    # a different ladder (base 1000) is far from the oracle's tables
    cos, _ = sa.rope_tables(2048, 128, base=1000.0)
    rc, _ = oracle.rope_tables(2048, 128)
    assert float((cos.double() - rc).abs().max()) > 0.5


def _bwd_noalloc(lib, B=1, T=8, Hq=4, Hkv=2, D=64, W=-1, dq=16, null_lse=False, eps=1e-6):
    P = ctypes.c_void_p
    lse = 0 if null_lse else 16
    return lib.sa_attn_bwd_noalloc(P(16), P(16), P(16), P(16), P(lse), P(16), P(dq), P(16), P(16),
                                   B, T, Hq, Hkv, D, W, 0.125, 1, eps, None)


def test_backward_noalloc_validation_paths(sa):
    """The no-allocation backward checks everything, including that the sizes
    fit its fixed scratch, before touching the HIP runtime."""
    lib = sa.library()
    assert lib.sa_attn_bwd_noalloc_max_bytes() == 80 << 20
    assert _bwd_noalloc(lib, null_lse=True) == SA_ERR_NULL
    assert _bwd_noalloc(lib, dq=0) == SA_ERR_NULL
    assert _bwd_noalloc(lib, Hq=5, Hkv=2) == SA_ERR_SHAPE
    assert _bwd_noalloc(lib, W=-2) == SA_ERR_SHAPE
    assert _bwd_noalloc(lib, eps=-1.0) == SA_ERR_SHAPE
    assert _bwd_noalloc(lib, D=32) == SA_ERR_UNSUPPORTED
    assert _bwd_noalloc(lib, dq=8) == SA_ERR_ALIGN
    # the 8-layer workload's shape fits; the pages' device batch of 128 (multi-head) does not
    assert lib.sa_attn_bwd_workspace_bytes(16, 2048, 6, 3, 128) <= lib.sa_attn_bwd_noalloc_max_bytes()
    assert lib.sa_attn_bwd_workspace_bytes(4, 8192, 6, 3, 128) <= lib.sa_attn_bwd_noalloc_max_bytes()
    assert _bwd_noalloc(lib, B=128, T=2048, Hq=6, Hkv=6, D=128) == SA_ERR_WORKSPACE
    assert _bwd_noalloc(lib, B=19, T=2048, Hq=6, Hkv=3, D=128) == SA_ERR_WORKSPACE
