"""GPU parity: the HIP path (through the C ABI) against the binary64 oracle.

Every workload of the benchmark family is compared element by element at its
full size (the oracle finishes each in seconds), plus a sweep of geometries,
dtypes, channel counts and alignments that exercises every kernel variant,
bit-exact invariants, edge cases and the backward pass.  Tolerances are the
ones tests/tolerance.py derives (1e-5 relative for fp32, 2e-2 for fp16/bf16,
with a binary32 summation floor where terms cancel).
"""
import math
import sys

import numpy as np
import pytest
import torch

import deformable_convolution_core_amd as dcn
import oracle
from deformable_convolution_core_amd import inputs
from tests import tolerance

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def cfg_of(w):
    return dict(kernel_size=w.K, stride=w.stride, pad=w.pad, dilation=w.dilation,
                offset_scale=w.offset_scale, softmax=w.softmax, group=w.G,
                remove_center=w.remove_center)


def oracle_fwd(t, w):
    return oracle.forward(inputs.to_f64(t["input"]), inputs.to_f64(t["offset"]), inputs.to_f64(t["mask"]),
                          K=w.K, stride=w.stride, pad=w.pad, dilation=w.dilation,
                          offset_scale=w.offset_scale, softmax=w.softmax, group=w.G,
                          coord_mode=oracle.COORD_BINARY32, remove_center=w.remove_center)


def gpu_fwd(t, w):
    d = {k: v.to(DEV) for k, v in t.items()}
    return dcn.forward(d["input"], d["offset"], d["mask"], **cfg_of(w))


def check_forward(w, t=None):
    t = t if t is not None else inputs.make(w, with_grad=False)
    out = gpu_fwd(t, w)
    torch.cuda.synchronize()
    ref, S = oracle_fwd(t, w)
    st = tolerance.compare(out.float().cpu().numpy(), ref, S, 4 * w.P, w.dtype)
    assert st["ok"], (w.name, st)
    return st


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_forward_full_size(name):
    check_forward(inputs.WORKLOADS[name])


def test_forward_is_deterministic():
    w = inputs.scaled(inputs.WORKLOADS["c3a_dcnv4_bf16_56"], N=4)
    t = {k: v.to(DEV) for k, v in inputs.make(w).items()}
    a = dcn.forward(t["input"], t["offset"], t["mask"], **cfg_of(w))
    b = dcn.forward(t["input"], t["offset"], t["mask"], **cfg_of(w))
    assert torch.equal(a, b)


SWEEP = [  # name, N, H, W, G, Cg, K, stride, pad, dil, alpha, softmax, dtype
    ("k1", 2, 9, 13, 3, 4, 1, 1, 0, 1, 1.0, False, "f32"),
    ("k2_even", 1, 10, 7, 2, 8, 2, 1, 1, 1, 1.0, True, "bf16"),
    ("k5_runtime", 2, 11, 9, 2, 16, 5, 1, 2, 1, 0.7, True, "f16"),
    ("k3_s2_d2", 1, 17, 15, 4, 8, 3, 2, 2, 2, 1.3, False, "f32"),
    ("k3_s3_pad0", 2, 16, 19, 1, 32, 3, 3, 0, 1, 0.5, True, "bf16"),
    ("cg1_f16", 1, 12, 12, 8, 1, 3, 1, 1, 1, 1.0, False, "f16"),
    ("cg1_f32", 1, 12, 12, 8, 1, 3, 1, 1, 1, 1.0, True, "f32"),
    ("cg2_bf16", 3, 9, 9, 5, 2, 3, 1, 1, 1, 1.0, True, "bf16"),
    ("cg3_odd", 2, 8, 11, 3, 3, 3, 1, 1, 1, 1.0, False, "bf16"),
    ("cg6_f32", 1, 7, 9, 2, 6, 3, 2, 1, 1, 1.0, True, "f32"),
    ("cg12_f16", 1, 9, 8, 2, 12, 3, 1, 1, 1, 1.0, False, "f16"),
    ("cg24_bf16", 2, 6, 10, 2, 24, 3, 1, 1, 1, 1.0, True, "bf16"),
    ("cg64_f32", 1, 8, 8, 2, 64, 3, 1, 1, 1, 1.0, False, "f32"),
    ("cg64_bf16", 1, 9, 7, 3, 64, 3, 1, 1, 1, 1.0, True, "bf16"),
    ("ragged_tail", 3, 5, 7, 3, 8, 3, 1, 1, 1, 1.0, False, "f16"),
    ("wide_map", 1, 3, 130, 2, 16, 3, 1, 1, 1, 1.0, True, "bf16"),
    ("tall_map", 1, 131, 3, 2, 16, 3, 1, 1, 1, 1.0, False, "f32"),
    ("one_pixel", 1, 1, 1, 2, 16, 3, 1, 1, 1, 1.0, True, "bf16"),
    # shapes the LDS-tiled kernel takes (group rows of 32/64/128 bytes, channel
    # rows a multiple of 128 bytes): ragged tiles, several slabs, stride and
    # dilation, runtime K, and offsets that leave the staged region
    ("tiled_f16_k5", 2, 19, 23, 4, 16, 5, 1, 2, 1, 0.8, True, "f16"),
    ("tiled_bf16_s2_d2", 1, 33, 30, 8, 16, 3, 2, 1, 2, 1.2, False, "bf16"),
    ("tiled_f32_cg32", 1, 17, 13, 4, 32, 3, 1, 1, 1, 1.0, True, "f32"),
    ("tiled_f32_cg16", 2, 21, 18, 4, 16, 3, 1, 1, 1, 1.0, False, "f32"),
    ("tiled_bf16_cg32", 1, 20, 9, 8, 32, 3, 1, 1, 1, 1.0, True, "bf16"),
    ("tiled_bf16_cg64", 1, 11, 12, 2, 64, 3, 1, 1, 1, 1.0, False, "bf16"),
    ("tiled_f16_k1", 1, 10, 37, 4, 16, 1, 1, 0, 1, 1.0, False, "f16"),
    ("tiled_bf16_s3_pad0", 2, 26, 25, 4, 16, 3, 3, 0, 1, 1.0, True, "bf16"),
    ("tiled_neg_alpha", 1, 16, 16, 4, 16, 3, 1, 1, 1, -0.9, False, "f16"),
]


@pytest.mark.parametrize("sigma", [0.25, 6.0, 40.0])
def test_tiled_offset_spread(sigma):
    """Small offsets stay in the staged region; large ones take the global
    gather fallback, very large ones fall off the map."""
    w = inputs.Workload(name="spread", N=2, H=24, W=20, G=4, Cg=16, Ho=24, Wo=20, dtype="bf16",
                        offset_sigma=sigma, mask_sigma=0.5, seed_base=93000 + int(sigma * 10))
    check_forward(w)


@pytest.mark.parametrize("sigma", [0.25, 6.0, 40.0])
def test_tall_offset_spread(sigma):
    """The same on a taller map with several tiles in each direction."""
    w = inputs.Workload(name="spread_tall", N=1, H=40, W=32, G=4, Cg=16, Ho=40, Wo=32, dtype="f16",
                        offset_sigma=sigma, mask_sigma=0.5, seed_base=93500 + int(sigma * 10))
    check_forward(w)


# taller maps (32 rows or more, several tiles in each direction): ragged
# tiles, runtime K, every group width, dilation, negative offset_scale
TALL_SWEEP = [  # name, N, H, W, G, Cg, K, stride, pad, dil, alpha, softmax, dtype
    ("tall_f16_ragged", 2, 37, 57, 4, 16, 3, 1, 1, 1, 1.0, False, "f16"),
    ("tall_bf16_k5", 1, 40, 33, 8, 16, 5, 1, 2, 1, 0.8, True, "bf16"),
    ("tall_f32_cg16", 1, 48, 30, 4, 16, 3, 1, 1, 1, 1.0, True, "f32"),
    ("tall_f32_cg8", 1, 33, 26, 8, 8, 3, 1, 1, 1, 1.0, False, "f32"),
    ("tall_bf16_cg64", 1, 35, 28, 2, 64, 3, 1, 1, 1, 1.0, False, "bf16"),
    ("tall_f16_k1", 1, 32, 40, 4, 16, 1, 1, 0, 1, 1.0, False, "f16"),
    ("tall_bf16_d2", 1, 44, 36, 4, 16, 3, 1, 2, 2, 1.0, True, "bf16"),
    ("tall_neg_alpha", 1, 34, 31, 4, 16, 3, 1, 1, 1, -1.1, False, "f16"),
    ("tall_f16_k7", 1, 40, 30, 4, 16, 7, 1, 3, 1, 1.0, False, "f16"),
]


@pytest.mark.parametrize("case", SWEEP + TALL_SWEEP, ids=lambda c: c[0])
def test_geometry_sweep(case):
    name, N, H, W, G, Cg, K, s, p, d, a, sm, dt = case
    Ho, Wo = oracle.out_size(H, K, s, p, d), oracle.out_size(W, K, s, p, d)
    w = inputs.Workload(name=name, N=N, H=H, W=W, G=G, Cg=Cg, Ho=Ho, Wo=Wo, K=K, stride=s, pad=p,
                        dilation=d, offset_scale=a, softmax=sm, dtype=dt, offset_sigma=2.5,
                        mask_sigma=1.0 if sm else 0.5, seed_base=90000 + 17 * len(name))
    check_forward(w)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_misaligned_tensors_use_narrower_loads(dtype):
    """Views whose data starts one element into a buffer: the library picks
    a narrower gather and must still match."""
    w = inputs.Workload(name="misaligned", N=2, H=9, W=10, G=2, Cg=16, Ho=9, Wo=10,
                        dtype=dtype, softmax=True, mask_sigma=1.0, seed_base=91000)
    t = inputs.make(w)
    td = {}
    for k, v in t.items():
        buf = torch.empty(v.numel() + 2, dtype=v.dtype, device=DEV)
        # keep offset pairs element-pair aligned, shift the others by one element
        sh = 2 if k == "offset" else 1
        td[k] = buf[sh:sh + v.numel()].view(v.shape).copy_(v.to(DEV))
    outbuf = torch.empty(int(np.prod(w.shapes()["output"])) + 1, dtype=td["input"].dtype, device=DEV)
    out = outbuf[1:].view(w.shapes()["output"])
    dcn.forward(td["input"], td["offset"], td["mask"], out=out, **cfg_of(w))
    torch.cuda.synchronize()
    ref, S = oracle_fwd(t, w)
    st = tolerance.compare(out.float().cpu().numpy(), ref, S, 4 * w.P, dtype)
    assert st["ok"], st


def test_empty_batch():
    x = torch.zeros(0, 8, 8, 16, device=DEV, dtype=torch.bfloat16)
    off = torch.zeros(0, 8, 8, 2 * 18, device=DEV, dtype=torch.bfloat16)
    m = torch.zeros(0, 8, 8, 2 * 9, device=DEV, dtype=torch.bfloat16)
    out = dcn.forward(x, off, m, group=2)
    assert out.shape == (0, 8, 8, 16)


# ---------------------------------------------------------------- invariants
def identity_inputs(N, H, W, G, Cg, dtype, softmax, seed):
    x = inputs.normal((N, H, W, G * Cg), seed, 1.0, dtype)
    off = torch.zeros(N, H, W, G * 18, dtype=inputs.DTYPES[dtype])
    m = torch.full((N, H, W, G, 9), -1e4 if softmax else 0.0)
    m[..., 4] = 0.0 if softmax else 1.0
    return x, off, m.reshape(N, H, W, G * 9).to(inputs.DTYPES[dtype])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("softmax", [False, True])
def test_identity_bit_exact(dtype, softmax):
    x, off, m = identity_inputs(2, 13, 11, 4, 16, dtype, softmax, 5)
    out = dcn.forward(x.to(DEV), off.to(DEV), m.to(DEV), group=4, softmax=softmax)
    assert torch.equal(out.cpu(), x)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_integer_offsets_are_exact_shifts(dtype):
    N, H, W, G, Cg = 1, 12, 10, 2, 8
    x = inputs.normal((N, H, W, G * Cg), 6, 1.0, dtype)
    for (p, dx, dy) in [(4, 1, 0), (4, -2, 3), (0, 0, 0), (8, -3, -1), (5, 4, -4)]:
        i, j = divmod(p, 3)
        off = torch.zeros(N, H, W, G, 9, 2)
        off[..., p, 0] = dx
        off[..., p, 1] = dy
        m = torch.zeros(N, H, W, G, 9)
        m[..., p] = 1.0
        T = inputs.DTYPES[dtype]
        out = dcn.forward(x.to(DEV), off.reshape(N, H, W, -1).to(T).to(DEV),
                          m.reshape(N, H, W, -1).to(T).to(DEV), group=G).cpu()
        exp = torch.zeros_like(x)
        sx, sy = (i - 1) + dx, (j - 1) + dy
        ys = slice(max(0, -sy), min(H, H - sy))
        xs = slice(max(0, -sx), min(W, W - sx))
        exp[:, ys, xs] = x[:, ys.start + sy:ys.stop + sy, xs.start + sx:xs.stop + sx]
        assert torch.equal(out, exp), (p, dx, dy)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_far_outside_and_nan_offsets_give_zero(dtype):
    N, H, W, G, Cg = 1, 6, 7, 2, 16
    T = inputs.DTYPES[dtype]
    x = inputs.normal((N, H, W, G * Cg), 7, 1.0, dtype).to(DEV)
    m = inputs.normal((N, H, W, G * 9), 8, 1.0, dtype).to(DEV)
    for big in (1e4, -1e4, float("inf"), float("-inf"), float("nan")):
        off = torch.full((N, H, W, G * 18), big, dtype=T, device=DEV)
        for sm in (False, True):
            out = dcn.forward(x, off, m, group=G, softmax=sm)
            assert torch.equal(out, torch.zeros_like(out)), (big, sm)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_input_does_not_leak_tiled(dtype):
    """Same check on a shape the tiled kernel serves (channel row of 128
    bytes or more): off-map corners read the staged zeros, not a wrapped
    neighbour."""
    N, H, W, G, Cg = 1, 12, 12, 4, 16
    T = inputs.DTYPES[dtype]
    x = torch.randn(N, H, W, G * Cg, generator=torch.Generator().manual_seed(2)).to(T)
    x[0, 0, 11] = float("nan")
    off = torch.zeros(N, H, W, G, 2)
    off[..., 0] = -0.5
    m = torch.ones(N, H, W, G)
    out = dcn.forward(x.to(DEV), off.reshape(N, H, W, -1).to(T).to(DEV), m.reshape(N, H, W, -1).to(T).to(DEV),
                      kernel_size=1, pad=0, group=G).cpu()
    nan_pix = torch.isnan(out.float()).any(-1)
    assert nan_pix[0, 0, 11] and nan_pix.sum() == 1


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_nan_input_does_not_leak_tall(dtype):
    """Same check on a taller map with several tiles."""
    N, H, W, G, Cg = 1, 32, 32, 4, 16
    T = inputs.DTYPES[dtype]
    x = torch.randn(N, H, W, G * Cg, generator=torch.Generator().manual_seed(3)).to(T)
    x[0, 0, 31] = float("nan")
    off = torch.zeros(N, H, W, G, 2)
    off[..., 0] = -0.5
    m = torch.ones(N, H, W, G)
    out = dcn.forward(x.to(DEV), off.reshape(N, H, W, -1).to(T).to(DEV), m.reshape(N, H, W, -1).to(T).to(DEV),
                      kernel_size=1, pad=0, group=G).cpu()
    nan_pix = torch.isnan(out.float()).any(-1)
    assert nan_pix[0, 0, 31] and nan_pix.sum() == 1


@pytest.mark.parametrize("shape", [(14, 14, 16), (7, 7, 32), (28, 28, 8)])
def test_off_map_samples_never_read_nan(shape):
    """Small maps (the staged region is the whole map plus its border):
    samples that miss the map read nothing, even with NaN in every corner
    pixel of the map; samples that land on it see the NaN."""
    H, W, G = shape
    Cg, N = 16, 2
    x = torch.randn(N, H, W, G * Cg, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    for yy, xx in ((0, 0), (0, W - 1), (H - 1, 0), (H - 1, W - 1)):
        x[:, yy, xx] = float("nan")
    off = torch.full((N, H, W, G, 9, 2), -60.0)   # every sample far off the map
    off[1] = 0.0                                    # image 1: every sample on the map
    m = torch.ones(N, H, W, G, 9)
    out = dcn.forward(x.to(DEV), off.reshape(N, H, W, -1).to(torch.bfloat16).to(DEV),
                      m.reshape(N, H, W, -1).to(torch.bfloat16).to(DEV), group=G).cpu().float()
    assert torch.all(out[0] == 0)
    assert torch.isnan(out[1]).any()


def test_nan_input_does_not_leak_to_other_pixels():
    """A NaN at one pixel reaches only outputs whose sample has a corner on
    that pixel; an off-map corner whose address would wrap onto it reads 0."""
    N, H, W, G, Cg = 1, 10, 10, 1, 16
    x = torch.randn(N, H, W, G * Cg, generator=torch.Generator().manual_seed(1))
    x[0, 0, 9] = float("nan")                   # right end of row 0
    off = torch.zeros(N, H, W, 2)               # K = 1: one sample per pixel
    off[..., 0] = -0.5                          # half a pixel left of each pixel
    m = torch.ones(N, H, W, 1)
    out = dcn.forward(x.to(DEV), off.to(DEV), m.to(DEV), kernel_size=1, pad=0, group=1).cpu()
    # only (0, 9) samples x = 8.5 between pixels 8 and 9 of row 0; (1, 0) samples
    # x = -0.5, whose left corner is off the map (its flat address is pixel (0, 9))
    nan_pix = torch.isnan(out).any(-1)
    assert nan_pix[0, 0, 9] and nan_pix.sum() == 1
    assert torch.equal(out[0, 1, 0], (0.5 * x[0, 1, 0]).float())


# ---------------------------------------------------------------- backward
def oracle_bwd(t, w):
    return oracle.backward(inputs.to_f64(t["input"]), inputs.to_f64(t["offset"]),
                           inputs.to_f64(t["mask"]), inputs.to_f64(t["grad_out"]),
                           K=w.K, stride=w.stride, pad=w.pad, dilation=w.dilation,
                           offset_scale=w.offset_scale, softmax=w.softmax, group=w.G,
                           coord_mode=oracle.COORD_BINARY32, remove_center=w.remove_center)


def check_backward(w):
    """Every gradient, element by element; half precision included: its
    grad_input is a binary32 sum rounded once, which rtol covers."""
    t = inputs.make(w, with_grad=True)
    d = {k: v.to(DEV) for k, v in t.items()}
    gi, goff, gm = dcn.backward(d["input"], d["offset"], d["mask"], d["grad_out"], **cfg_of(w))
    torch.cuda.synchronize()
    r = oracle_bwd(t, w)
    Cg, P = w.Cg, w.P
    stats = {}
    for key, got, S, n in (("grad_input", gi, r["gi_abs"], r["gi_cnt"]),
                           ("grad_offset", goff, r["goff_abs"], 4 * Cg),
                           ("grad_mask", gm, r["gmask_abs"], 4 * Cg * (P + 1) if w.softmax else 4 * Cg)):
        st = tolerance.compare(got.float().cpu().numpy().reshape(r[key].shape), r[key], S, n, w.dtype)
        assert st["ok"], (w.name, key, st)
        stats[key] = st
    return stats


def test_workload_backward_full_size():
    check_backward(inputs.WORKLOADS["c5_dcnv4_f32_56_fwdbwd"])


BWD_SWEEP = [  # name, N, H, W, G, Cg, K, stride, pad, dil, alpha, softmax
    ("softmax_k3", 2, 9, 11, 2, 16, 3, 1, 1, 1, 1.0, True),
    ("cg4_L1", 1, 8, 8, 3, 4, 3, 1, 1, 1, 1.0, False),
    ("cg8_s2_d2", 1, 13, 12, 2, 8, 3, 2, 2, 2, 0.75, True),
    ("cg32", 1, 7, 9, 2, 32, 3, 1, 1, 1, 1.0, False),
    ("cg64_L16", 1, 6, 6, 1, 64, 3, 1, 1, 1, 1.0, True),
    ("cg1_scalar", 2, 8, 9, 4, 1, 3, 1, 1, 1, 1.0, False),
    ("cg2_scalar", 1, 9, 8, 3, 2, 3, 1, 1, 1, 1.3, True),
    ("k5_runtime", 1, 10, 10, 2, 16, 5, 1, 2, 1, 1.0, True),
    ("k1_runtime", 1, 9, 9, 2, 8, 1, 1, 0, 1, 1.0, False),
    ("ragged", 3, 5, 7, 3, 16, 3, 1, 1, 1, 1.0, False),
]


@pytest.mark.parametrize("case", BWD_SWEEP, ids=lambda c: c[0])
def test_backward_sweep(case):
    name, N, H, W, G, Cg, K, s, p, d, a, sm = case
    Ho, Wo = oracle.out_size(H, K, s, p, d), oracle.out_size(W, K, s, p, d)
    w = inputs.Workload(name=name, N=N, H=H, W=W, G=G, Cg=Cg, Ho=Ho, Wo=Wo, K=K, stride=s, pad=p,
                        dilation=d, offset_scale=a, softmax=sm, dtype="f32", offset_sigma=2.0,
                        mask_sigma=1.0 if sm else 0.5, seed_base=92000 + 31 * len(name), backward=True)
    check_backward(w)


# Shapes the owner-tiled grad_input path takes (Cg a multiple of 8, C a
# multiple of 32): strides, dilation, negative offset_scale, tiles that do not
# divide the map, and offset spreads that put many corners beyond the owners'
# reach (those are added by the gradient kernel's atomics).
OWNER_SWEEP = [  # name, N, H, W, G, Cg, K, stride, pad, dil, alpha, softmax, sigma
    ("own_s2_d2", 1, 21, 19, 4, 8, 3, 2, 2, 2, 0.75, True, 2.0),
    ("own_ragged", 2, 37, 29, 4, 8, 3, 1, 1, 1, 1.0, False, 1.5),
    ("own_neg_alpha", 1, 17, 23, 2, 16, 3, 1, 1, 1, -1.25, False, 2.0),
    ("own_k1", 1, 15, 14, 4, 8, 1, 1, 0, 1, 1.0, False, 2.0),
    ("own_k7_s3", 1, 26, 24, 1, 32, 7, 3, 3, 1, 1.0, True, 1.5),
    ("own_far_6", 1, 19, 21, 2, 16, 3, 1, 1, 1, 1.0, False, 6.0),
    ("own_far_40", 1, 19, 21, 2, 16, 3, 1, 1, 1, 1.0, True, 40.0),
    ("own_cg64", 2, 11, 13, 2, 64, 3, 1, 1, 1, 1.0, False, 3.0),
    ("big_alpha_atomic", 1, 12, 12, 4, 8, 3, 1, 1, 1, 9.0, False, 1.0),
    # visited windows of one to three rows (row phases left empty) and of one column
    ("own_h1", 2, 1, 40, 4, 8, 3, 1, 1, 1, 1.0, False, 1.5),
    ("own_h2", 1, 2, 33, 2, 16, 3, 1, 1, 1, 1.0, True, 1.5),
    ("own_h3_s2", 1, 5, 30, 4, 8, 3, 2, 1, 1, 1.0, False, 1.5),
    ("own_w1", 2, 29, 1, 4, 8, 3, 1, 1, 1, 1.0, False, 1.5),
]


@pytest.mark.parametrize("case", OWNER_SWEEP, ids=lambda c: c[0])
def test_backward_owner_sweep(case):
    name, N, H, W, G, Cg, K, s, p, d, a, sm, sigma = case
    Ho, Wo = oracle.out_size(H, K, s, p, d), oracle.out_size(W, K, s, p, d)
    w = inputs.Workload(name=name, N=N, H=H, W=W, G=G, Cg=Cg, Ho=Ho, Wo=Wo, K=K, stride=s, pad=p,
                        dilation=d, offset_scale=a, softmax=sm, dtype="f32", offset_sigma=sigma,
                        mask_sigma=1.0 if sm else 0.5, seed_base=93000 + 37 * len(name), backward=True)
    check_backward(w)


# Half-precision backward on the tiled shapes: binary32 arithmetic, every
# gradient rounded once to the dtype; corners beyond the owners' reach are
# summed in the binary32 workspace before the owners round each element.
HALF_BWD = [  # name, N, H, W, G, Cg, K, stride, pad, dil, alpha, softmax, dtype, sigma
    ("h_c5_f16", 4, 56, 56, 4, 16, 3, 1, 1, 1, 1.0, False, "f16", 1.5),
    ("h_c5_bf16", 4, 56, 56, 4, 16, 3, 1, 1, 1, 1.0, False, "bf16", 1.5),
    ("h_softmax_bf16", 2, 23, 29, 4, 16, 3, 1, 1, 1, 1.0, True, "bf16", 2.0),
    ("h_k5_f16", 1, 21, 19, 2, 32, 5, 1, 2, 1, 0.8, True, "f16", 2.0),
    ("h_s2_d2_f16", 1, 25, 23, 4, 16, 3, 2, 2, 2, 1.2, False, "f16", 2.0),
    ("h_cg32_bf16", 2, 17, 20, 4, 32, 3, 1, 1, 1, -1.1, True, "bf16", 1.5),
    # offsets far beyond the owners' reach: many corners go through the workspace
    ("h_far_f16", 1, 19, 21, 4, 16, 3, 1, 1, 1, 1.0, False, "f16", 6.0),
    ("h_far_bf16", 2, 24, 20, 4, 16, 3, 1, 1, 1, 1.0, True, "bf16", 8.0),
]


@pytest.mark.parametrize("case", HALF_BWD, ids=lambda c: c[0])
def test_backward_half_precision(case):
    name, N, H, W, G, Cg, K, s, p, d, a, sm, dt, sigma = case
    Ho, Wo = oracle.out_size(H, K, s, p, d), oracle.out_size(W, K, s, p, d)
    w = inputs.Workload(name=name, N=N, H=H, W=W, G=G, Cg=Cg, Ho=Ho, Wo=Wo, K=K, stride=s, pad=p,
                        dilation=d, offset_scale=a, softmax=sm, dtype=dt, offset_sigma=sigma,
                        mask_sigma=1.0 if sm else 0.5, seed_base=94000 + 41 * len(name), backward=True)
    check_backward(w)


def test_half_backward_full_size_c5_shape():
    """The c5 shape (N=32, 56x56, C=64) in fp16 and bf16 at full size."""
    for dt in ("f16", "bf16"):
        check_backward(inputs.scaled(inputs.WORKLOADS["c5_dcnv4_f32_56_fwdbwd"], dtype=dt))


def test_backward_half_needs_the_workspace():
    """dcn_core_backward (no workspace argument) declines half precision; the
    binding runs it through dcn_core_backward_ws with a binary32 workspace
    (parity of that path: test_backward_half_generic and the tiled cases)."""
    import ctypes
    x = torch.randn(1, 8, 8, 16, device=DEV, dtype=torch.float16)
    off = torch.zeros(1, 8, 8, 2 * 9 * 2, device=DEV, dtype=torch.float16)
    m = torch.ones(1, 8, 8, 2 * 9, device=DEV, dtype=torch.float16)
    g = torch.ones(1, 8, 8, 16, device=DEV, dtype=torch.float16)
    gi, goff, gm = torch.empty_like(x), torch.empty_like(off), torch.empty_like(m)
    lib = dcn.load_library()
    vp = ctypes.c_void_p
    rc = lib.dcn_core_backward(*(vp(t.data_ptr()) for t in (x, off, m, g, gi, goff, gm)), 1, 8, 8, 2, 8, 3, 1, 1, 1,
                               ctypes.c_float(1.0), 0, 1, None)
    assert rc == 2
    need = lib.dcn_core_backward_workspace_size(vp(x.data_ptr()), vp(g.data_ptr()), vp(gi.data_ptr()), 1, 8, 8, 2, 8,
                                                3, 1, 1, 1, ctypes.c_float(1.0), 0, 1)
    assert need == 1 * 8 * 8 * 16 * 4
    gi2, _, _ = dcn.backward(x, off, m, g, group=2)
    torch.cuda.synchronize()
    assert torch.isfinite(gi2.float()).all()


# Half precision outside the tiled shapes: binary32 atomics into a workspace,
# one rounding into grad_input (grad_mask of a softmax carries one more: the
# raw gm is stored, then reread for the Jacobian).
HALF_GENERIC = [  # name, N, H, W, G, Cg, K, stride, pad, dil, alpha, softmax, dtype
    ("g_cg8_f16", 2, 13, 11, 2, 8, 3, 1, 1, 1, 1.0, False, "f16"),
    ("g_cg4_bf16_softmax", 1, 12, 9, 3, 4, 3, 1, 1, 1, 0.9, True, "bf16"),
    ("g_cg2_f16_k5", 1, 11, 10, 4, 2, 5, 1, 2, 1, 1.0, False, "f16"),
    ("g_stride5_bf16", 1, 23, 21, 4, 16, 3, 5, 1, 1, 1.0, False, "bf16"),
    ("g_k9_f16_softmax", 1, 14, 15, 2, 16, 9, 1, 4, 1, 1.0, True, "f16"),
    ("g_cg1_bf16", 1, 7, 8, 8, 1, 3, 1, 1, 2, 1.3, False, "bf16"),
]


@pytest.mark.parametrize("case", HALF_GENERIC, ids=lambda c: c[0])
def test_backward_half_generic(case):
    name, N, H, W, G, Cg, K, s, p, d, a, sm, dt = case
    Ho, Wo = oracle.out_size(H, K, s, p, d), oracle.out_size(W, K, s, p, d)
    w = inputs.Workload(name=name, N=N, H=H, W=W, G=G, Cg=Cg, Ho=Ho, Wo=Wo, K=K, stride=s, pad=p, dilation=d,
                        offset_scale=a, softmax=sm, dtype=dt, offset_sigma=2.0, mask_sigma=1.0 if sm else 0.5,
                        seed_base=98000 + 13 * len(name), backward=True)
    t = inputs.make(w, with_grad=True)
    dd = {k: v.to(DEV) for k, v in t.items()}
    gi, goff, gm = dcn.backward(dd["input"], dd["offset"], dd["mask"], dd["grad_out"], **cfg_of(w))
    torch.cuda.synchronize()
    r = oracle_bwd(t, w)
    for key, got, S, n, extra in (("grad_input", gi, r["gi_abs"], r["gi_cnt"], 0),
                                  ("grad_offset", goff, r["goff_abs"], 4 * Cg, 0),
                                  ("grad_mask", gm, r["gmask_abs"], 4 * Cg * (w.P + 1) if sm else 4 * Cg,
                                   1 if sm else 0)):
        st = tolerance.compare(got.float().cpu().numpy().reshape(r[key].shape), r[key], S, n, dt,
                               store_roundings=extra)
        assert st["ok"], (name, key, st)


@pytest.mark.parametrize("shape", [(4, 16, "f32"), (4, 16, "f16"), (2, 8, "bf16"), (3, 8, "f32")],
                         ids=["tiled_f32", "tiled_f16", "workspace_bf16", "untiled_f32"])
def test_backward_of_far_inf_and_nan_offsets_is_zero(shape):
    """Samples whose coordinates are far off the map, infinite or NaN are
    skipped by the definition: every gradient is zero (no NaN leaks), on the
    tiled, the half-precision workspace and the untiled paths."""
    G, Cg, dt = shape
    N, H, W = 1, 9, 10
    T = inputs.DTYPES[dt]
    x = inputs.normal((N, H, W, G * Cg), 31, 1.0, dt).to(DEV)
    g = inputs.normal((N, H, W, G * Cg), 32, 1.0, dt).to(DEV)
    m = inputs.normal((N, H, W, G * 9), 33, 1.0, dt).to(DEV)
    for big in (1e4, -1e4, float("inf"), float("-inf"), float("nan")):
        off = torch.full((N, H, W, G * 18), big, dtype=T, device=DEV)
        for sm in (False, True):
            gi, goff, gm = dcn.backward(x, off, m, g, group=G, softmax=sm)
            torch.cuda.synchronize()
            for name, t in (("grad_input", gi), ("grad_offset", goff), ("grad_mask", gm)):
                assert torch.equal(t, torch.zeros_like(t)), (big, sm, name)


def test_backward_repeat_within_tolerance_and_autograd():
    w = inputs.scaled(inputs.WORKLOADS["c5_dcnv4_f32_56_fwdbwd"], N=2)
    t = {k: v.to(DEV) for k, v in inputs.make(w, with_grad=True).items()}
    a = dcn.backward(t["input"], t["offset"], t["mask"], t["grad_out"], **cfg_of(w))
    b = dcn.backward(t["input"], t["offset"], t["mask"], t["grad_out"], **cfg_of(w))
    for x, y in zip(a, b):
        assert torch.allclose(x, y, rtol=1e-5, atol=1e-5)
    xi = t["input"].clone().requires_grad_(True)
    oi = t["offset"].clone().requires_grad_(True)
    mi = t["mask"].clone().requires_grad_(True)
    out = dcn.dcn_core(xi, oi, mi, w.K, w.stride, w.pad, w.dilation, w.offset_scale, w.softmax, w.G)
    out.backward(t["grad_out"])
    for got, want in zip((xi.grad, oi.grad, mi.grad), a):
        assert torch.allclose(got, want, rtol=1e-5, atol=1e-5)


def test_backward_unsupported_group_width_raises():
    x = torch.zeros(1, 4, 4, 12, device=DEV)
    off = torch.zeros(1, 4, 4, 18, device=DEV)
    m = torch.zeros(1, 4, 4, 9, device=DEV)
    with pytest.raises(dcn.DCNError) as e:
        dcn.backward(x, off, m, torch.zeros_like(x), group=1)
    assert e.value.status == 2
