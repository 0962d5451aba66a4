"""The library's launches inside a HIP graph (torch.cuda.graph capture) and its replays.

Each entry point is called once eagerly (the first call of a configuration runs the gate's
verification, which synchronizes, and allocates the per-device counter; the DiT grid needs no
such call), then captured; the
graph is replayed several times with fresh inputs copied in by eager work between replays, and
every replay is compared bit for bit with the oracle.  The captured work is one kernel launch
per call: nothing in it clears memory with hipMemsetAsync.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.neox as nx
import oracle.patchify as pf
import workloads

pytestmark = pytest.mark.gpu

rla = pytest.importorskip("rope_ltx3drope_amd")
from rope_ltx3drope_amd import _lib  # noqa: E402

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def fresh():
    assert torch.cuda.is_available()
    _lib.lib()
    rla.set_option(rla.OPT_PATH, 0)
    rla.set_option(rla.OPT_GATE, 1)
    rla.gate_reset()
    rla.stats_reset()
    yield
    torch.cuda.synchronize()


def bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_host(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def test_rope3d_graph_replays():
    shape, split = (1, 4, 8, 8, 16, 128), (32, 48, 48)
    sets = [workloads.generate_custom(shape, oracle.BF16, seed=50 + i) for i in range(3)]
    dq, dk = bf16_dev(sets[0][0]), bf16_dev(sets[0][1])
    qo, ko = torch.empty_like(dq), torch.empty_like(dk)
    with rla.tables_build(*shape[1:4], split) as tab:
        rla.apply_qk(dq, dk, tab, qo, ko)  # eager: the gate's verification
        torch.cuda.synchronize()
        assert rla.gate_state(0, rla.DTYPE_BF16, shape, split) == "TRUSTED"
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rla.apply_qk(dq, dk, tab, qo, ko)
        for q, k in sets[1:] + sets[:1]:
            dq.copy_(bf16_dev(q))
            dk.copy_(bf16_dev(k))
            qo.zero_()
            ko.zero_()
            g.replay()
            torch.cuda.synchronize()
            want_q, want_k = oracle.rope3d_qk(q, k, oracle.BF16, split)
            np.testing.assert_array_equal(bf16_host(qo), want_q)
            np.testing.assert_array_equal(bf16_host(ko), want_k)
    st = rla.stats()
    assert st["gate_verifications"] == 1 and st["plain_launches"] == 0


def test_neox_graph_replays():
    w = workloads.NeoxWorkload("g", oracle.BF16, 257, 8, 4, 128, 512, oracle.F32, "random", 60)
    sets = [workloads.generate_neox(workloads.NeoxWorkload(w.key, w.dtype, w.tokens, w.q_heads, w.k_heads,
                                                           w.head_dim, w.max_position, w.cache_dtype,
                                                           w.positions, 60 + i)) for i in range(3)]
    q0, k0, pos0, cache = sets[0]
    dq, dk = bf16_dev(q0), bf16_dev(k0)
    dpos, dcache = torch.from_numpy(pos0).to(DEV), torch.from_numpy(cache).to(DEV)
    qo, ko = torch.empty_like(dq), torch.empty_like(dk)
    rla.neox_apply_qk(dq, dk, dpos, dcache, qo, ko)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rla.neox_apply_qk(dq, dk, dpos, dcache, qo, ko)
    for q, k, pos, _ in sets[1:] + sets[:1]:
        dq.copy_(bf16_dev(q))
        dk.copy_(bf16_dev(k))
        dpos.copy_(torch.from_numpy(pos))
        qo.zero_()
        ko.zero_()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bf16_host(qo), nx.neox_rope(q, oracle.BF16, pos, cache, oracle.F32))
        np.testing.assert_array_equal(bf16_host(ko), nx.neox_rope(k, oracle.BF16, pos, cache, oracle.F32))
    assert rla.neox_position_errors(0) == 0


def test_patchify_graph_replays():
    shape, p = (1, 3, 5, 32, 64), 4
    sets = [workloads.generate_patch(shape, 2, seed=70 + i) for i in range(3)]
    x = torch.from_numpy(sets[0].view(np.int16)).to(DEV)
    y = rla.patchify(x, p)
    back = rla.unpatchify(y, p)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rla.patchify(x, p, out=y)
        rla.unpatchify(y, p, out=back)
    for h in sets[1:] + sets[:1]:
        x.copy_(torch.from_numpy(h.view(np.int16)))
        y.zero_()
        back.zero_()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint16), pf.patchify(h, p))
        np.testing.assert_array_equal(back.cpu().numpy().view(np.uint16), h)


def test_dit_freq_grid_graph_replays():
    """Both recipes of the DiT frequency grid captured through the C ABI into fixed outputs; every
    replay, after the outputs are cleared by eager work, equals the oracle."""
    import ctypes

    import oracle.dit_freqs as df

    theta, dim, ne = 10000.0, 4096, 6
    outs = {d: torch.empty(dim // ne, dtype=torch.float32, device=DEV) for d in (1, 0)}
    n = ctypes.c_int64(0)
    L = _lib.lib()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sp = torch.cuda.current_stream().cuda_stream
        for d, out in outs.items():
            assert L.ltx3drope_dit_freq_grid(theta, dim, ne, d, out.data_ptr(), sp, ctypes.byref(n)) == _lib.OK
    want = {d: df.freq_grid(theta, dim, ne, bool(d)).view(np.uint32) for d in outs}
    for _ in range(3):
        for out in outs.values():
            out.zero_()
        g.replay()
        torch.cuda.synchronize()
        for d, out in outs.items():
            np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want[d])


@pytest.mark.parametrize("entry", ["apply_qk", "apply_qk_noalloc"])
def test_unverified_configuration_under_capture_runs_the_plain_kernel(entry):
    """A configuration's first call made under graph capture cannot run the gate's verification
    (it waits for a count on the host): the captured call is the plain kernel and the gate stays
    UNSEEN.  Its replays are bit-exact; a later eager call verifies and trusts the fast kernel."""
    shape, split = (1, 3, 8, 8, 12, 64), (16, 24, 24)
    sets = [workloads.generate_custom(shape, oracle.BF16, seed=80 + i) for i in range(3)]
    dq, dk = bf16_dev(sets[0][0]), bf16_dev(sets[0][1])
    qo, ko = torch.empty_like(dq), torch.empty_like(dk)
    call = getattr(rla, entry)
    with rla.tables_build(*shape[1:4], split) as tab:  # built eagerly: the build allocates and waits
        torch.cuda.synchronize()
        assert rla.gate_state(0, rla.DTYPE_BF16, shape, split) == "UNSEEN"
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            call(dq, dk, tab, qo, ko)
        st = rla.stats()
        assert st["gate_verifications"] == 0 and st["plain_launches"] == 1 and st["fast_launches"] == 0
        assert rla.gate_state(0, rla.DTYPE_BF16, shape, split) == "UNSEEN"
        for q, k in sets[1:] + sets[:1]:
            dq.copy_(bf16_dev(q))
            dk.copy_(bf16_dev(k))
            qo.zero_()
            ko.zero_()
            g.replay()
            torch.cuda.synchronize()
            want_q, want_k = oracle.rope3d_qk(q, k, oracle.BF16, split)
            np.testing.assert_array_equal(bf16_host(qo), want_q)
            np.testing.assert_array_equal(bf16_host(ko), want_k)
        call(dq, dk, tab, qo, ko)  # eager now: verified, trusted
        torch.cuda.synchronize()
        assert rla.gate_state(0, rla.DTYPE_BF16, shape, split) == "TRUSTED"
        assert rla.stats()["gate_verifications"] == 1
