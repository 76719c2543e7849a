"""The measured-ceiling kernels (libkda_probe, include/kda_probe.h).

CPU: the library exports every declared entry point and validation turns bad
calls into status 1 before anything is enqueued.  GPU: each streaming mode
moves exactly the bytes it claims (checked element by element on small
buffers), and the matrix-core loop computes the products it is credited with
(its output checked against the same sum formed on the host)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from kda_gated_delta_amd import ceilings

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda_probe.h")
P, P2, P_MIS = ctypes.c_void_p(4096), ctypes.c_void_p(1 << 20), ctypes.c_void_p(4096 + 4)


def test_probe_exports_every_declared_symbol():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", src)))
    assert set(declared) == set(ceilings.EXPORTED), declared
    L = ceilings.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_probe_validation():
    L = ceilings.lib()
    assert L.kda_probe_hbm(4, P, P2, 64, None) == 1          # unknown mode
    assert L.kda_probe_hbm(-1, P, P2, 64, None) == 1
    assert L.kda_probe_hbm(0, P, P2, 0, None) == 1           # nothing to move
    assert L.kda_probe_hbm(0, P, P2, 96, None) == 1          # not a multiple of 64
    assert L.kda_probe_hbm(0, None, P2, 64, None) == 1       # copy needs a source
    assert L.kda_probe_hbm(2, None, P2, 64, None) == 1       # read needs a source
    assert L.kda_probe_hbm(1, None, None, 64, None) == 1     # no destination
    assert L.kda_probe_hbm(0, P_MIS, P2, 64, None) == 1      # misaligned
    assert L.kda_probe_hbm(3, None, P_MIS, 64, None) == 1
    assert L.kda_probe_hbm(0, P, ctypes.c_void_p(4096 + 32), 128, None) == 1  # overlap
    for shape in (0, 1):
        assert L.kda_probe_mfma_bf16(shape, 0, 1, P, None) == 1
        assert L.kda_probe_mfma_bf16(shape, 65537, 1, P, None) == 1
        assert L.kda_probe_mfma_bf16(shape, 1, 0, P, None) == 1
        assert L.kda_probe_mfma_bf16(shape, 1, (1 << 24) + 1, P, None) == 1
        assert L.kda_probe_mfma_bf16(shape, 1, 1, None, None) == 1
    assert L.kda_probe_mfma_bf16(2, 1, 1, P, None) == 1       # unknown shape
    assert L.kda_probe_mfma_bf16(-1, 1, 1, P, None) == 1


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [64, 4096 + 64, (1 << 22) + 192])
def test_probe_streams_move_every_byte(nbytes):
    n = nbytes // 4
    src = torch.randn(n, device="cuda")
    dst = torch.full((n,), -7.0, device="cuda")
    ceilings.hbm("copy", src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    ceilings.hbm("rmw", None, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst, 0.5 * src + 1.0)
    ceilings.hbm("write", None, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst, torch.ones_like(dst))
    part = torch.zeros(ceilings.read_partials(nbytes), device="cuda")
    ceilings.hbm("read", src, part, nbytes)
    torch.cuda.synchronize()
    got = part.double().sum().item()
    want = src.double().sum().item()
    assert abs(got - want) <= 1e-4 * src.double().abs().sum().item() + 1e-6


@pytest.mark.gpu
@pytest.mark.parametrize("shape,rows,chains", [("32x32x16", 32, 8), ("16x16x32", 16, 8)])
def test_probe_mfma_loop_computes_its_products(shape, rows, chains):
    blocks, iters = 3, 5
    out = torch.zeros(4 * blocks, device="cuda")
    ceilings.mfma_bf16(shape, blocks, iters, out)
    torch.cuda.synchronize()
    # lane l holds A[r][8 g + j] = a_l[j] and B[8 g + j][r] = b_l[j] with
    # r = l % rows and g = l / rows; every entry of the product lands in
    # exactly one lane, so a wave's output is chains x iters x the sum of A B.
    bf = lambda x: float(torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).double())
    inner = 512 // rows
    A = np.zeros((rows, inner))
    B = np.zeros((inner, rows))
    for l in range(64):
        g, r = divmod(l, rows)
        for j in range(8):
            A[r, 8 * g + j] = bf(0.001 * ((l + j) & 7))
            B[8 * g + j, r] = bf(0.001 * ((l * 3 + j) & 7))
    want = chains * iters * (A @ B).sum()
    np.testing.assert_allclose(out.double().cpu().numpy(), np.full(4 * blocks, want), rtol=1e-5)
