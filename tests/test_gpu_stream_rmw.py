"""la_stream_rmw, the in-place streaming pass that bounds a decode step: x <- a x over fp32
data, each element read once and written once. One fp32 multiply per element, so the
result is compared bit for bit with numpy's fp32 product (IEEE round to nearest even), on
lengths with a ragged last tile, on a decode-sized buffer (8,192 states of 128 x 128), and
on two calls in a row."""
import ctypes

import numpy as np
import pytest
import torch

from gated_delta_rule_linear_amd import binding as bd
from gpu_util import banner

pytestmark = pytest.mark.gpu


def run(x, a):
    lib = bd.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.la_stream_rmw(ctypes.c_void_p(x.data_ptr()), x.numel(), ctypes.c_float(a), stream)
    assert rc == 0, bd.status_str(rc)


@pytest.mark.parametrize("n", [4, 4096, 4096 * 3 + 12, 1 << 20, 4096 * 1000 + 2044])
@pytest.mark.parametrize("a", [0.5, 1.0001])
def test_stream_rmw_exact(n, a):
    banner(f"stream rmw n={n} a={a}")
    rng = np.random.default_rng(n)
    h = rng.standard_normal(n).astype(np.float32)
    x = torch.from_numpy(h.copy()).cuda()
    run(x, a)
    torch.cuda.synchronize()
    want = h * np.float32(a)
    assert np.array_equal(x.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_stream_rmw_decode_size_twice():
    n = 8192 * 128 * 128
    banner(f"stream rmw decode-sized buffer n={n}, two calls")
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn(n, device="cuda", generator=g)
    ref = x.clone()
    run(x, 0.5)
    run(x, 2.0)
    torch.cuda.synchronize()
    assert torch.equal(x, ref)   # both products are exact
    run(x, 1.0001)
    torch.cuda.synchronize()
    assert torch.equal(x, ref * 1.0001)
