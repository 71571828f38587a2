"""qt_linear_noalloc (the allocation-free projection entry point) against
qt_debug_linear, the entry point it is a variant of, on the same inputs:
bit-identical outputs on two calls in a row (the second smaller, so it runs
over what the first left in the shared static scratch), both within the
projection tolerance of a float64 reference; and a projection whose scratch
need exceeds the static array is refused before any device work."""
import sys

import numpy as np
import pytest

from codec_lm_autoregressive_amd import binding, synth

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


def _case(torch, g, M, N, K, epi, norm):
    W = synth.bf16_round((g.standard_normal((N, K)) * 0.02).astype(np.float32))
    X = g.standard_normal((M, K)).astype(np.float32)
    gain = (1.0 + 0.02 * g.standard_normal(K)).astype(np.float32) if norm else None
    Y0 = (g.standard_normal((M, N // 2 if epi == 2 else N)) * 0.1).astype(np.float32)
    return W, X, gain, Y0


def _reference(W, X, gain, Y0, epi, eps=1e-6):
    x = X.astype(np.float64)
    if gain is not None:
        x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps) * gain.astype(np.float64)
    y = x @ W.astype(np.float64).T
    if epi == 0:
        return y
    if epi == 1:
        return Y0.astype(np.float64) + y
    gt, up = y[:, 0::2], y[:, 1::2]
    return gt / (1.0 + np.exp(-gt)) * up


@pytest.mark.parametrize("shapes", [
    # (M, N, K, epilogue, gain): split-activation GEMM (300 rows), then the row-block GEMM with K ranges (40 rows)
    [(300, 2048, 1024, 0, True), (40, 1024, 3072, 1, False)],
    # row-block GEMM (64 rows, SwiGLU), then the 8-row matrix-core GEMV (5 rows, residual)
    [(64, 6144, 1024, 2, True), (5, 1024, 2048, 1, False)],
])
def test_noalloc_equals_debug_linear(shapes):
    torch = _torch()
    g = np.random.default_rng(17)
    for M, N, K, epi, norm in shapes:
        print(f"noalloc case M={M} N={N} K={K} epilogue={epi} gain={norm}", flush=True)
        W, X, gain, Y0 = _case(torch, g, M, N, K, epi, norm)
        Wd = binding.to_device_weight(W, "bf16")
        Xd = torch.from_numpy(X).cuda()
        gd = torch.from_numpy(gain).cuda() if gain is not None else None
        ya = torch.from_numpy(Y0).cuda()
        yb = torch.from_numpy(Y0).cuda()
        binding.debug_linear(Wd, Xd, gd, 1e-6, epi, ya)
        binding.linear_noalloc(Wd, Xd, gd, 1e-6, epi, yb)
        torch.cuda.synchronize()
        a, b = ya.cpu().numpy(), yb.cpu().numpy()
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
        ref = _reference(W, X, gain, Y0, epi)
        err = float(np.max(np.abs(b - ref)))
        print(f"  bit-identical to qt_debug_linear; max|d| vs float64 {err:.2e}", flush=True)
        assert err < 1e-3 * max(1.0, float(np.max(np.abs(ref))))


def test_noalloc_rejects_oversized_scratch():
    torch = _torch()
    M, N, K = 4096, 2048, 3072          # hi/lo planes of 4096 x 3072 floats > 8 Mi
    W = torch.zeros((N, K), dtype=torch.int16, device="cuda")
    X = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    Y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(binding.QtError) as e:
        binding.linear_noalloc(W, X, None, 1e-6, 0, Y)
    assert e.value.status == binding.QT_E_CAPACITY
    torch.cuda.synchronize()
    assert bool(torch.all(Y == 7.0))     # nothing was written
