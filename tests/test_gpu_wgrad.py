"""GPU parity of the matrix-core weight-gradient reduction used by the DCNv4
layer's projections, against the float64 sums, element by element:
    dw[o, i] = sum_m g[m, o] x[m, i],   db[o] = sum_m g[m, o]
    |gpu - ref| <= 1e-5 |ref| + (M + 32) 2^-24 S,   S = |g|^T |x|  (or sum |g|)
(binary32 sums of M products, exact for half-precision operands; M bounds the
length of any chain of additions).  The result is binary32 for every input
dtype.  The chunked sum is added in a fixed order, so repeated calls agree
bit for bit."""
import ctypes
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


CASES = [  # M, O, I
    (1000, 64, 64),       # value / output projection
    (777, 108, 64),       # merged offset+mask projection, G = 4 (216-byte rows in half precision)
    (513, 4, 64),         # centre-gate logits
    (130, 864, 72),       # seven 128-row blocks of dw, two column blocks, a ragged last one
    (64, 7, 3),           # odd widths: element staging reads
    (1, 16, 16),          # one row
    (20000, 33, 130),     # many chunks
]


def check(g, x, dw, db, dt):
    G, X = inputs.to_f64(g), inputs.to_f64(x)
    M = G.shape[0]
    ref, S = G.T @ X, np.abs(G).T @ np.abs(X)
    st = tolerance.compare(dw.cpu().numpy(), ref, S, M, "f32")
    assert st["ok"], ("dw", st)
    if db is not None:
        st = tolerance.compare(db.cpu().numpy(), G.sum(0), np.abs(G).sum(0), M, "f32")
        assert st["ok"], ("db", st)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"M{c[0]}_O{c[1]}_I{c[2]}")
def test_weight_grad_matches_float64(case, dt):
    M, O, I = case
    seed = 8100 + M + O + I
    g = inputs.normal((M, O), seed, 1.0, dt)
    x = inputs.normal((M, I), seed + 1, 1.0, dt)
    dw, db = dcn.linear_weight_grad(g.to(DEV), x.to(DEV))
    torch.cuda.synchronize()
    check(g, x, dw, db, dt)


def draw_wgrad(case):
    """Seeded random shape: rows around the 64-row chunk edges or anywhere up
    to 20000, O up to 260 (several 128-row blocks of dw), I up to 200, with or
    without the bias sum."""
    r = random.Random(6160 + 137 * case)
    dt = r.choice(["f32", "f16", "bf16"])
    M = r.choice([1, 3, 63, 64, 65, 127, 128, 129]) if r.random() < 0.3 else r.randint(1, 20000)
    return M, r.randint(1, 260), r.randint(1, 200), r.random() < 0.7, dt


@pytest.mark.parametrize("case", range(40))
def test_weight_grad_random_shapes(case):
    M, O, I, bias, dt = draw_wgrad(case)
    g = inputs.normal((M, O), 8300 + 17 * case, 1.0, dt)
    x = inputs.normal((M, I), 8301 + 17 * case, 1.0, dt)
    dw, db = dcn.linear_weight_grad(g.to(DEV), x.to(DEV), bias=bias)
    torch.cuda.synchronize()
    assert (db is None) == (not bias)
    check(g, x, dw, db, dt)


@pytest.mark.parametrize("out", ["f16", "bf16"])
@pytest.mark.parametrize("case", [(777, 108, 64), (130, 864, 72), (64, 7, 3), (1, 16, 16)],
                         ids=lambda c: f"M{c[0]}_O{c[1]}_I{c[2]}")
def test_weight_grad_in_half_precision_is_the_binary32_sum_rounded(case, out):
    """dw and db stored in a half-precision type are the binary32 sums rounded
    once to nearest even: bit for bit what the binary32 call gives, converted."""
    M, O, I = case
    odt = inputs.DTYPES[out]
    g = inputs.normal((M, O), 8400 + M + O, 1.0, out).to(DEV)
    x = inputs.normal((M, I), 8401 + M + I, 1.0, out).to(DEV)
    dw32, db32 = dcn.linear_weight_grad(g, x)
    dwh, dbh = dcn.linear_weight_grad(g, x, out_dtype=odt)
    zw, zb = dcn.linear_weight_grad(g[:0], x[:0], out_dtype=odt)
    torch.cuda.synchronize()
    assert dwh.dtype == odt and dbh.dtype == odt
    assert torch.equal(dwh, dw32.to(odt)) and torch.equal(dbh, db32.to(odt))
    assert torch.equal(zw, torch.zeros(O, I, dtype=odt, device=DEV)) and torch.equal(zb, torch.zeros(O, dtype=odt, device=DEV))


def test_weight_grad_at_the_layer_shape_is_deterministic():
    """The headline layer's offset+mask projection (200,704 rows): within the
    bound, and two calls give the same bits."""
    M, O, I = 64 * 56 * 56, 108, 64
    g = inputs.normal((M, O), 8201, 1.0, "f16")
    x = inputs.normal((M, I), 8202, 1.0, "f16")
    gd, xd = g.to(DEV), x.to(DEV)
    dw1, db1 = dcn.linear_weight_grad(gd, xd)
    dw2, db2 = dcn.linear_weight_grad(gd, xd)
    torch.cuda.synchronize()
    assert torch.equal(dw1, dw2) and torch.equal(db1, db2)
    check(g, x, dw1, db1, "f16")


def test_weight_grad_without_bias_and_batched_rows():
    g = torch.randn(3, 5, 7, 24, device=DEV)
    x = torch.randn(3, 5, 7, 40, device=DEV)
    dw, db = dcn.linear_weight_grad(g, x, bias=False)
    torch.cuda.synchronize()
    assert db is None
    check(g.reshape(-1, 24).cpu(), x.reshape(-1, 40).cpu(), dw, None, "f32")


def test_weight_grad_of_no_rows_is_zero():
    g = torch.empty(0, 12, device=DEV, dtype=torch.float16)
    x = torch.empty(0, 8, device=DEV, dtype=torch.float16)
    dw, db = dcn.linear_weight_grad(g, x)
    torch.cuda.synchronize()
    assert torch.equal(dw, torch.zeros(12, 8, device=DEV)) and torch.equal(db, torch.zeros(12, device=DEV))


def test_weight_grad_rejects_a_small_workspace():
    lib = dcn.load_library()
    g = torch.randn(256, 16, device=DEV)
    x = torch.randn(256, 16, device=DEV)
    dw = torch.empty(16, 16, device=DEV)
    need = lib.dcn_linear_weight_grad_workspace_size(256, 16, 16)
    ws = torch.empty(need // 4, device=DEV)
    vp = ctypes.c_void_p
    rc = lib.dcn_linear_weight_grad(vp(g.data_ptr()), vp(x.data_ptr()), vp(dw.data_ptr()), None, 256, 16, 16, 0, 0,
                                    vp(ws.data_ptr()), need - 4, None)
    assert rc == 1
