"""GPU parity of patchify / unpatchify (through the C ABI) against oracle.patchify, bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.patchify as pf
import workloads
from tests import oracle_full

pytestmark = pytest.mark.gpu

rla = pytest.importorskip("rope_ltx3drope_amd")
from rope_ltx3drope_amd import _lib  # noqa: E402

DEV = "cuda:0"
TORCH_INT = {1: torch.uint8, 2: torch.int16, 4: torch.int32, 8: torch.int64}
NP_SIGNED = {1: np.uint8, 2: np.int16, 4: np.int32, 8: np.int64}


@pytest.fixture(autouse=True)
def fresh():
    assert torch.cuda.is_available()
    _lib.lib()
    rla.set_option(rla.OPT_PATH, 0)
    rla.stats_reset()
    yield
    rla.set_option(rla.OPT_PATH, 0)
    torch.cuda.synchronize()


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(NP_SIGNED[x.dtype.itemsize])).to(DEV)


def to_host(t, like):
    return t.cpu().numpy().view(like.dtype)



@pytest.mark.parametrize("key", ["p1", "p2", "p3", "p4", "p5", "p7", "p8", "p9", "p10", "p11", "p13", "p14", "p15",
                                 "p16", "p17", "p18", "p19", "p20", "p21"])
@pytest.mark.parametrize("path", [0, 2], ids=["fast", "plain"])
def test_patchify_and_inverse_full(key, path):
    shape, p, eb = workloads.PATCH_WORKLOADS[key]
    x = workloads.generate_patch(shape, eb, seed=len(key) + p)
    rla.set_option(rla.OPT_PATH, path)
    # the library's rule for its fast kernels
    fast = path == 0 and p in (2, 4, 8, 16) and shape[4] % (p * 16 // eb) == 0
    y = rla.patchify(to_dev(x), p)
    torch.cuda.synchronize()
    want = pf.patchify(x, p)
    np.testing.assert_array_equal(to_host(y, want), want)
    back = rla.unpatchify(y, p)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(back, x), x)
    yy = workloads.generate_patch(want.shape, eb, seed=7)
    np.testing.assert_array_equal(to_host(rla.unpatchify(to_dev(yy), p), x), pf.unpatchify(yy, p))
    st = rla.stats()
    assert (st["fast_launches"], st["plain_launches"]) == ((3, 0) if fast else (0, 3))


@pytest.mark.parametrize("eb", [1, 2, 4, 8])
def test_patch_sizes_other_than_2_4_8_16_use_the_plain_kernel(eb):
    shape, p = (2, 3, 2, 12, 18), 3
    x = workloads.generate_patch(shape, eb, seed=eb)
    y = rla.patchify(to_dev(x), p)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(y, x), pf.patchify(x, p))
    assert rla.stats()["plain_launches"] == 1 and rla.stats()["fast_launches"] == 0


def test_full_clip_patchify_round_trip_in_full():
    shape, p, eb = workloads.PATCH_WORKLOADS["p6"]
    x = workloads.generate_patch(shape, eb, seed=6)
    dx = to_dev(x)
    y = rla.patchify(dx, p)
    torch.cuda.synchronize()
    want = pf.patchify(x, p)
    assert np.array_equal(to_host(y, want), want)
    del want
    back = rla.unpatchify(y, p)
    torch.cuda.synchronize()
    assert torch.equal(back, dx)
    assert rla.stats()["fast_launches"] == 2


def test_refusals():
    x = torch.zeros((1, 2, 1, 8, 8), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        rla.patchify(x, 3)
    L = _lib.lib()
    y = torch.empty((1, 8, 1, 4, 4), dtype=torch.bfloat16, device=DEV)
    assert L.ltx3drope_patchify(y.data_ptr(), x.data_ptr(), 3, 1, 2, 1, 8, 8, 2, None) == _lib.E_INVALID
    assert L.ltx3drope_patchify(y.data_ptr(), x.data_ptr(), 2, 1, 2, 1, 8, -8, 2, None) == _lib.E_INVALID
    assert L.ltx3drope_patchify(x.data_ptr() + 2, x.data_ptr(), 2, 1, 2, 1, 8, 8, 2, None) == _lib.E_UNSUPPORTED
    small = torch.empty(16, dtype=torch.bfloat16, device=DEV)
    assert L.ltx3drope_patchify(y.data_ptr(), small.data_ptr(), 2, 1, 2, 1, 800, 800, 2, None) == _lib.E_UNSUPPORTED
    host = torch.zeros((1, 2, 1, 8, 8), dtype=torch.bfloat16).pin_memory()
    assert L.ltx3drope_patchify(y.data_ptr(), host.data_ptr(), 2, 1, 2, 1, 8, 8, 2, None) == _lib.E_UNSUPPORTED
    assert rla.stats()["fast_launches"] == 0 and rla.stats()["plain_launches"] == 0


def test_empty_tensors():
    """An empty batch (or frame count) gives an empty result of the right shape; nothing launches."""
    for shape in ((0, 3, 5, 8, 8), (2, 3, 0, 8, 8)):
        x = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        y = rla.patchify(x, 4)
        assert tuple(y.shape) == (shape[0], 48, shape[2], 2, 2)
        back = rla.unpatchify(y, 4)
        assert tuple(back.shape) == shape
    assert rla.stats()["fast_launches"] == 0 and rla.stats()["plain_launches"] == 0


def test_output_of_2_gib_or_more():
    """An output of 2^31 bytes or more (the LDS kernels then store with 64-bit addresses instead of
    32-bit offsets from the output's base): whole-tensor fast == plain and round trip on the
    device, every element against the oracle."""
    shape, p = (1, 8, 129, 1088, 960), 4
    B, C, F, H, W = shape
    assert B * C * F * H * W * 2 >= 2 ** 31 and B * C * F * H * W < 2 ** 31
    x = workloads.generate_patch_device(shape, 2, 123, DEV)
    y = rla.patchify(x, p)
    rla.set_option(rla.OPT_PATH, 2)
    y_plain = rla.patchify(x, p)
    rla.set_option(rla.OPT_PATH, 0)
    torch.cuda.synchronize()
    assert torch.equal(y, y_plain)
    del y_plain
    back = rla.unpatchify(y, p)
    torch.cuda.synchronize()
    assert torch.equal(back, x)
    del back
    assert oracle_full.compare_full_patchify(x.cpu().numpy(), y.cpu().numpy(), p) == 0
    st = rla.stats()
    assert st["fast_launches"] == 2 and st["plain_launches"] == 1


def test_4k_clip_of_more_than_2_to_the_31_elements():
    """A 121-frame 2160 x 3840 RGB clip in bf16 with p = 4: 3,010,560,000 elements (between 2^31 and
    2^32, 6 GB per tensor), drawn on the device.  The LDS kernels against the plain kernel over the
    whole output, the round trip, and every element against the oracle."""
    shape, p = (1, 3, 121, 2160, 3840), 4
    B, C, F, H, W = shape
    assert 2 ** 31 < B * C * F * H * W < 2 ** 32
    x = workloads.generate_patch_device(shape, 2, 4096, DEV)
    y = rla.patchify(x, p)
    rla.set_option(rla.OPT_PATH, 2)
    y_plain = rla.patchify(x, p)
    rla.set_option(rla.OPT_PATH, 0)
    torch.cuda.synchronize()
    assert torch.equal(y, y_plain)
    del y_plain
    back = rla.unpatchify(y, p)
    torch.cuda.synchronize()
    assert torch.equal(back, x)
    del back
    assert oracle_full.compare_full_patchify(x.cpu().numpy(), y.cpu().numpy(), p) == 0
    st = rla.stats()
    assert st["fast_launches"] == 2 and st["plain_launches"] == 1


@pytest.mark.parametrize("seed", [5, 6])
def test_random_configurations(seed):
    """Twenty seeded random configurations per seed: element sizes 1/2/4/8, p in {2, 3, 4, 8, 16},
    widths that do or do not allow the LDS kernels, both directions, against the oracle."""
    rng = np.random.default_rng(seed)
    for i in range(20):
        eb = int(rng.choice([1, 2, 4, 8]))
        p = int(rng.choice([2, 3, 4, 8, 16]))
        E = 16 // eb
        unit = p * E if (rng.random() < 0.7 and p != 3) else p  # W a multiple of p*E: LDS kernels
        W = unit * int(rng.integers(1, max(2, 512 // unit) + 1))
        H = p * int(rng.integers(1, 5))
        shape = (int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 4)), H, W)
        x = workloads.generate_patch(shape, eb, seed=seed * 100 + i)
        rla.stats_reset()
        y = rla.patchify(to_dev(x), p)
        back = rla.unpatchify(y, p)
        torch.cuda.synchronize()
        want = pf.patchify(x, p)
        np.testing.assert_array_equal(to_host(y, want), want, err_msg=f"{shape} p={p} eb={eb}")
        np.testing.assert_array_equal(to_host(back, x), x, err_msg=f"{shape} p={p} eb={eb} inverse")
        fast = p in (2, 4, 8, 16) and W % (p * E) == 0
        st = rla.stats()
        assert (st["fast_launches"], st["plain_launches"]) == ((2, 0) if fast else (0, 2)), (shape, p, eb)
