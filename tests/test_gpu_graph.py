"""The entry points under HIP graph capture: forward, backward (tiled, half
precision, and the half-precision workspace path), the forward with the
fused gate and the projections' weight gradient are captured once and
replayed several times, with unrelated eager work and synchronisations
between the replays.  Every replay must overwrite every output and reproduce
the eager result: bit for bit where the arithmetic order is fixed, and to a
few dozen units in the last place of the dtype for grad_input, whose adds
(LDS compare-and-swap, binary32 or half-precision atomics) have no fixed
order.
The library clears its buffers with kernels, not memset nodes, so nothing in
a captured call depends on state left by an earlier replay."""
import sys

import pytest
import torch

import deformable_convolution_core_amd as dcn
from deformable_convolution_core_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def announce(request):
    print(f"\n[gpu-case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def capture(fn):
    """A graph of fn() (after two warm-up calls on a side stream) and the
    tensors it returns (owned by the graph's memory pool)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


# unit roundoff of each dtype: an unordered sum may land a few of these away
ULP = {torch.float32: 2.0 ** -24, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}


def replay_and_check(g, got, want, close=()):
    noise = torch.randn(1 << 20, device=DEV)
    for r in range(3):
        noise.mul_(1.0001).add_(0.5)          # unrelated eager work between replays
        torch.cuda.synchronize()
        for t in got:
            if t is not None:
                t.fill_(float("nan"))          # a replay must overwrite every element
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, want)):
            if a is None:
                assert b is None
            elif i in close:
                assert torch.isfinite(a).all(), (r, i, "not overwritten")
                u = ULP[a.dtype]
                scale = float(b.float().abs().max())
                assert torch.allclose(a.float(), b.float(), rtol=64 * u, atol=64 * u * scale), (r, i)
            else:
                assert torch.equal(a, b), (r, i)


CASES = [  # N, H, W, G, Cg, dtype, softmax  (C = 64 / 128: tiled; C = 16 half: workspace path)
    (2, 20, 18, 4, 16, "f32", True),
    (2, 20, 18, 4, 16, "f16", False),
    (1, 15, 17, 2, 8, "bf16", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[5]}_G{c[3]}_Cg{c[4]}")
def test_forward_and_backward_replay(case):
    N, H, W, G, Cg, dt, sm = case
    w = inputs.Workload(name="graph", N=N, H=H, W=W, G=G, Cg=Cg, Ho=H, Wo=W, softmax=sm, dtype=dt,
                        mask_sigma=1.0 if sm else 0.5, seed_base=88100 + G * Cg, backward=True)
    t = {k: v.to(DEV) for k, v in inputs.make(w, with_grad=True).items()}
    kw = dict(group=G, softmax=sm)
    fwd = lambda: (dcn.forward(t["input"], t["offset"], t["mask"], **kw),)
    bwd = lambda: dcn.backward(t["input"], t["offset"], t["mask"], t["grad_out"], **kw)
    want_f, want_b = fwd(), bwd()
    torch.cuda.synchronize()
    g, got = capture(fwd)
    replay_and_check(g, got, want_f)
    g, got = capture(bwd)
    replay_and_check(g, got, want_b, close=(0,))


def test_gated_forward_and_weight_grad_replay():
    N, H, W, G, Cg, K = 2, 16, 16, 4, 16, 3
    P = K * K
    x = inputs.normal((N, H, W, G * Cg), 88201, 1.0, "f16").to(DEV)
    om = inputs.normal((N, H, W, G * 3 * P), 88202, 1.0, "f16").to(DEV)
    z = inputs.normal((N, H, W, G), 88203, 1.0, "f16").to(DEV)
    gated = lambda: dcn.forward_packed_gated(x, om, z, kernel_size=K, group=G, keep_core_output=True)
    want = gated()
    torch.cuda.synchronize()
    g, got = capture(gated)
    replay_and_check(g, got, want)
    gy = inputs.normal((N * H * W, 108), 88204, 1.0, "f16").to(DEV)
    xs = x.reshape(-1, G * Cg)
    wg = lambda: dcn.linear_weight_grad(gy, xs)
    want = wg()
    torch.cuda.synchronize()
    g, got = capture(wg)
    replay_and_check(g, got, want)


def test_concurrent_threads_on_their_own_streams():
    """The library keeps no state: two host threads, each on a stream of its
    own (default priority), run forward and backward on different inputs at
    the same time; every result equals the same call made alone."""
    import threading
    cases = []
    for k in range(2):
        w = inputs.Workload(name=f"thread{k}", N=2, H=24, W=22, G=4, Cg=16, Ho=24, Wo=22, dtype="f32",
                            seed_base=88300 + 17 * k, backward=True)
        cases.append({n: v.to(DEV) for n, v in inputs.make(w, with_grad=True).items()})
    want = []
    for t in cases:
        out = dcn.forward(t["input"], t["offset"], t["mask"], group=4)
        _, goff, gm = dcn.backward(t["input"], t["offset"], t["mask"], t["grad_out"], group=4)
        want.append((out, goff, gm))
    torch.cuda.synchronize()
    got = [[] for _ in cases]
    errors = []

    def work(k):
        try:
            s = torch.cuda.Stream()
            t = cases[k]
            with torch.cuda.stream(s):
                for _ in range(10):
                    out = dcn.forward(t["input"], t["offset"], t["mask"], group=4)
                    _, goff, gm = dcn.backward(t["input"], t["offset"], t["mask"], t["grad_out"], group=4)
                    got[k].append((out, goff, gm))
            s.synchronize()
        except Exception as e:          # reported on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(k,)) for k in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k in range(len(cases)):
        assert len(got[k]) == 10
        for res in got[k]:
            for a, b in zip(res, want[k]):
                assert torch.equal(a, b), k
