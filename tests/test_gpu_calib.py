"""The measurement kernels of libkda_calib.so do exactly what their byte counts
assume: the copy copies every byte, the fill writes every value, and the state
read-modify-write touches every value of every state once (so their traffic is
the known size that the byte counters are checked against)."""
import pytest
import torch

import gated_delta_rule_short_amd as kda

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.load_calib_library()


@pytest.mark.parametrize("n", [4, 1000, 4096 * 256 + 12, 3 * 2 ** 20 + 4])
def test_copy_and_fill_cover_every_value(n):
    g = torch.Generator(device=DEV).manual_seed(n)
    src = torch.randn(n, generator=g, device=DEV)
    dst = torch.full((n + 4,), -7.0, device=DEV)
    kda.calib_copy(dst[:n], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src) and (dst[n:] == -7.0).all()
    kda.calib_fill(dst[:n], 2.5)
    torch.cuda.synchronize()
    assert (dst[:n] == 2.5).all() and (dst[n:] == -7.0).all()


def test_state_rmw_scales_every_value_once():
    g = torch.Generator(device=DEV).manual_seed(3)
    st = torch.randn((37, 128, 128), generator=g, device=DEV)
    guard = torch.randn((2, 128, 128), generator=g, device=DEV)
    buf = torch.cat([st, guard])
    kda.calib_state_rmw(buf[:37], 0.5)
    torch.cuda.synchronize()
    assert torch.equal(buf[:37], st * 0.5) and torch.equal(buf[37:], guard)
