"""GPU parity of the matrix-core projection kernel (y = x w^T + b) used by the
DCNv4 layer, against the float64 product, element by element:
    |gpu - ref| <= rtol |ref| + (K + 32) 2^-24 S,   S = |x| |w|^T + |b|
(binary32 accumulation of K exact products, one rounding to the dtype)."""
import random
import sys

import numpy as np
import pytest
import torch

import deformable_convolution_core_amd as dcn
from deformable_convolution_core_amd import inputs
from tests import tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


CASES = [  # M, N, K, bias
    (1000, 64, 64, True),      # the layer's value / output projections
    (777, 108, 64, True),      # merged offset+mask projection, G = 4 (N not a multiple of 16)
    (513, 4, 64, True),        # centre-gate logits
    (300, 864, 512, True),     # offset+mask projection at the 7x7 stage (G = 32, C = 512)
    (100, 70, 36, False),      # N % 4 != 0 (element stores), K % 16 != 0 (a partial last step)
    (16, 16, 16, False),
    (33, 64, 1208, True),      # the widest K a half-precision call takes
]


def check_linear(M, N, K, has_bias, dt, seed):
    x = inputs.normal((M, K), seed, 1.0, dt)
    w = inputs.normal((N, K), seed + 1, 1.0 / np.sqrt(K), dt)
    b = inputs.normal((N,), seed + 2, 0.5, dt) if has_bias else None
    y = dcn.linear(x.to(DEV), w.to(DEV), None if b is None else b.to(DEV))
    torch.cuda.synchronize()
    X, Wm = inputs.to_f64(x), inputs.to_f64(w)
    B = inputs.to_f64(b) if has_bias else np.zeros(N)
    ref = X @ Wm.T + B
    S = np.abs(X) @ np.abs(Wm).T + np.abs(B)
    st = tolerance.compare(y.float().cpu().numpy(), ref, S, K + 1, dt)
    assert st["ok"], ((M, N, K, has_bias, dt), st)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"M{c[0]}_N{c[1]}_K{c[2]}")
def test_linear_matches_float64(case, dt):
    M, N, K, has_bias = case
    if dt == "f32" and K > 636:
        pytest.skip("binary32 takes K <= 636")
    check_linear(M, N, K, has_bias, dt, 7000 + M + N + K)


def draw_linear(case):
    """Seeded random shape: rows around the 16-row tile and 64-row block
    edges or anywhere up to 4000, any N up to 300, K a multiple of 4 up to
    320, with or without bias."""
    r = random.Random(5150 + 131 * case)
    dt = r.choice(["f32", "f16", "bf16"])
    M = r.choice([1, 2, 15, 16, 17, 63, 64, 65, 129]) if r.random() < 0.3 else r.randint(1, 4000)
    return M, r.randint(1, 300), 4 * r.randint(1, 80), r.random() < 0.6, dt


@pytest.mark.parametrize("case", range(40))
def test_linear_random_shapes(case):
    M, N, K, has_bias, dt = draw_linear(case)
    check_linear(M, N, K, has_bias, dt, 7500 + 17 * case)


def test_linear_batched_rows_and_empty():
    x = torch.randn(2, 7, 9, 64, device=DEV)
    w = torch.randn(32, 64, device=DEV)
    y = dcn.linear(x, w)
    torch.cuda.synchronize()
    ref = x.double().reshape(-1, 64) @ w.double().t()
    assert y.shape == (2, 7, 9, 32)
    assert torch.allclose(y.double().reshape(-1, 32), ref, rtol=1e-5, atol=1e-4)
    e = dcn.linear(torch.empty(0, 64, device=DEV), w)
    assert e.shape == (0, 32)


def test_linear_unsupported_shapes_say_so():
    w = torch.randn(8, 6, device=DEV)
    with pytest.raises(dcn.DCNError) as e:
        dcn.linear(torch.randn(10, 6, device=DEV), w)          # K not a multiple of 4
    assert e.value.status == 2
    base = torch.randn(10 * 64 + 1, device=DEV)
    with pytest.raises(dcn.DCNError) as e:
        dcn.linear(base[1:].view(10, 64), torch.randn(8, 64, device=DEV))   # x off a 16-byte boundary
    assert e.value.status == 2
