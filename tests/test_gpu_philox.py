"""The device random-number functions against the oracle, directly (GPU).

The sampling kernels' Philox4x32-10 block, the word layout of a draw, u24 and
the Gumbel transform are called through a test-only probe built from the same
device header (tests/device_probe.hip) and compared with oracle/philox.py:
10^6 (counter, key) blocks bit for bit, draw words bit for bit, u24 exactly,
and Gumbel variates within their binary32 error bound."""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import philox
from tests.gpu_support import device, log

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "libss_device_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(PROBE)
    vp, i32, u32, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64
    lib.ss_probe_philox.argtypes = [vp, vp, i32, vp]
    lib.ss_probe_words.argtypes = [u64, u32, u32, u32, vp, i32, vp]
    lib.ss_probe_transforms.argtypes = [vp, vp, vp, i32, vp]
    for f in (lib.ss_probe_philox, lib.ss_probe_words, lib.ss_probe_transforms):
        f.restype = i32
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_philox_blocks_bit_exact(probe):
    # 1000 keys x 1000 counters: random words, plus keys and counters at 0 and
    # at 2^32 - 1 (the Weyl additions and the products wrap there)
    rng = np.random.default_rng(11)
    nk, nc = 1000, 1000
    keys = rng.integers(0, 2 ** 32, (nk, 2), dtype=np.uint64).astype(np.uint32)
    keys[0] = 0
    keys[1] = 0xFFFFFFFF
    ctrs = rng.integers(0, 2 ** 32, (nk, nc, 4), dtype=np.uint64).astype(np.uint32)
    ctrs[:, 0] = 0
    ctrs[:, 1] = 0xFFFFFFFF
    ctrs[:, 2] = np.arange(4, dtype=np.uint32)  # a counter of the form (request, position, block, domain)
    inp = np.concatenate([ctrs, np.broadcast_to(keys[:, None, :], (nk, nc, 2))], axis=2)
    n = nk * nc
    log(f"[philox] {n} blocks")
    dinp = torch.from_numpy(np.ascontiguousarray(inp).reshape(n, 6).view(np.int32)).to(device())
    dout = torch.empty(n, 4, dtype=torch.int32, device=device())
    assert probe.ss_probe_philox(_p(dinp), _p(dout), n, _stream()) == 0
    torch.cuda.synchronize()
    got = dout.cpu().numpy().view(np.uint32).reshape(nk, nc, 4)
    for k in range(nk):
        c = ctrs[k]
        want = philox.philox4x32_10_np(c[:, 0], c[:, 1], c[:, 2], c[:, 3],
                                       int(keys[k, 0]), int(keys[k, 1]))
        for j in range(4):
            bad = np.nonzero(got[k, :, j] != want[j])[0]
            assert bad.size == 0, (k, j, bad[:4].tolist())


@pytest.mark.parametrize("seed,req,position,domain", [
    (0, 0, 0, philox.SAMPLE), (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, philox.GUMBEL),
    (0x0123456789ABCDEF, 5, 7, philox.RESIDUAL), (12345, 1 << 30, 3, philox.ACCEPT)])
def test_draw_words_bit_exact(probe, seed, req, position, domain):
    n = 128256 + 3  # a ragged count of draws: the last block is partly used
    out = torch.empty(n, dtype=torch.int32, device=device())
    assert probe.ss_probe_words(seed, req, position, domain, _p(out), n, _stream()) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    want = philox.words_np(seed, req, position, np.arange(n), domain).astype(np.uint32)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, bad[:4].tolist()


def test_u24_exact_and_gumbel_within_binary32_bounds(probe):
    rng = np.random.default_rng(12)
    w = rng.integers(0, 2 ** 32, 10 ** 6, dtype=np.uint64).astype(np.uint32)
    # both ends of the word range and both sides of the branch at 2^31
    w[:8] = [0, 1, 255, 256, 0x7FFFFFFF, 0x80000000, 0xFFFFFFFE, 0xFFFFFFFF]
    dw = torch.from_numpy(w.view(np.int32)).to(device())
    du = torch.empty(w.size, dtype=torch.float32, device=device())
    dg = torch.empty(w.size, dtype=torch.float32, device=device())
    assert probe.ss_probe_transforms(_p(dw), _p(du), _p(dg), w.size, _stream()) == 0
    torch.cuda.synchronize()
    u = du.cpu().numpy().astype(np.float64)
    g = dg.cpu().numpy().astype(np.float64)
    assert np.array_equal(u, philox.u24_np(w))
    want = philox.gumbel_np(w)
    # binary32 evaluation: the word rounded to 24 bits, log1p / log and the
    # outer log each within a few units in the last place; 2^-20 (1 + |g|)
    # bounds the sum, far below the 1e-5 gap at which a Gumbel-max draw is
    # treated as a boundary case
    err = np.abs(g - want)
    bound = 2.0 ** -20 * (1.0 + np.abs(want))
    log(f"[gumbel] max |err| {err.max():.3e}, max err/bound {(err / bound).max():.3f}")
    assert np.all(np.isfinite(g))
    assert np.all(err <= bound), np.nonzero(err > bound)[0][:4].tolist()
