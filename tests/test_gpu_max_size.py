"""GPU checks at the largest supported image: one bf16 image of 1448 x 1448
pixels x 512 channels, 2,147,024,896 bytes, just under the 2^31 - 4096-byte
limit of one image (larger images return DCN_ERR_UNSUPPORTED).  Here the
kernels' 32-bit byte offsets within an image are closest to overflowing.

The oracle cannot finish this size, so the checks are properties that hold
exactly at any size:
* zero offsets and a one-hot centre mask (raw, or softmax logits of -1e4
  around a 0) give the input itself, bit for bit;
* an integer offset on the centre tap gives the shifted input, zeros past
  the border;
* the backward of the identity gives grad_input = grad_output bit for bit,
  and grad_mask and grad_offset of the centre point equal the channel sums
  sum_c g*x and sum_c g*(x[right or below] - x) (right-sided derivative at an
  integer coordinate), formed here in float32 from the same tensors.
Inputs are drawn on the GPU from a seeded generator.
"""
import sys

import pytest
import torch

import deformable_convolution_core_amd as dcn

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N, H, W, G, Cg, K = 1, 1448, 1448, 16, 32, 3
P = K * K


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_image_is_at_the_limit():
    assert N * H * W * G * Cg * 2 == 2_147_024_896
    assert N * H * W * G * Cg * 2 <= 2 ** 31 - 4096 < (H + 1) * (W + 1) * G * Cg * 2


def big_input(seed):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(N, H, W, G * Cg, device=DEV, dtype=torch.float32, generator=gen).to(torch.bfloat16)


def centre_records(dx=0, dy=0, softmax=False):
    off = torch.zeros(N, H, W, G, P, 2, device=DEV, dtype=torch.bfloat16)
    off[..., 4, 0] = dx
    off[..., 4, 1] = dy
    m = torch.full((N, H, W, G, P), -1e4 if softmax else 0.0, device=DEV, dtype=torch.bfloat16)
    m[..., 4] = 0.0 if softmax else 1.0
    return off.reshape(N, H, W, G * P * 2), m.reshape(N, H, W, G * P)


@pytest.mark.parametrize("softmax", [False, True])
def test_identity_at_the_largest_image(softmax):
    x = big_input(11)
    off, m = centre_records(softmax=softmax)
    out = dcn.forward(x, off, m, kernel_size=K, pad=1, group=G, softmax=softmax)
    torch.cuda.synchronize()
    assert torch.equal(out, x)


def test_integer_shift_at_the_largest_image():
    x = big_input(12)
    dx, dy = 1, -2
    off, m = centre_records(dx, dy)
    out = dcn.forward(x, off, m, kernel_size=K, pad=1, group=G)
    exp = torch.zeros_like(x)
    # out[h, w] = x[h + dy, w + dx] where that pixel exists
    exp[:, -dy:, :W - dx] = x[:, :H + dy, dx:]
    torch.cuda.synchronize()
    assert torch.equal(out, exp)


def test_backward_of_identity_at_the_largest_image():
    x = big_input(13)
    go = big_input(14)
    off, m = centre_records()
    gi, goff, gm = dcn.backward(x, off, m, go, kernel_size=K, pad=1, group=G)
    torch.cuda.synchronize()
    assert torch.equal(gi, go)
    xf = x.float().view(N, H, W, G, Cg)
    gf = go.float().view(N, H, W, G, Cg)
    want_m = (gf * xf).sum(-1)                                        # (N, H, W, G)
    got_m = gm.float().view(N, H, W, G, P)[..., 4]
    S_m = (gf.abs() * xf.abs()).sum(-1)
    # binary32 sum of Cg products, one rounding to bfloat16
    assert torch.all((got_m - want_m).abs() <= 2.0 ** -8 * want_m.abs() + (Cg + 32) * 2.0 ** -24 * S_m)
    right = torch.zeros_like(xf)
    right[:, :, :-1] = xf[:, :, 1:]
    below = torch.zeros_like(xf)
    below[:, :-1] = xf[:, 1:]
    want_x = (gf * (right - xf)).sum(-1)
    want_y = (gf * (below - xf)).sum(-1)
    S_x = (gf.abs() * (right.abs() + xf.abs())).sum(-1)
    S_y = (gf.abs() * (below.abs() + xf.abs())).sum(-1)
    got = goff.float().view(N, H, W, G, P, 2)[..., 4, :]
    for k, want, S in ((0, want_x, S_x), (1, want_y, S_y)):
        err = (got[..., k] - want).abs()
        assert torch.all(err <= 2.0 ** -8 * want.abs() + (2 * Cg + 32) * 2.0 ** -24 * S), k
