"""Byte offsets beyond 4 GiB: a batch's field bases are 64-bit (the lanes add
only a small 32-bit offset), so a mesh whose arrays span more than 2^32 bytes
per field must give, tile by tile, the bitwise result of the small mesh it is
tiled from.  The volume term is element-local and the whole right-hand side
of a tiled mesh whose tiles keep their own connectivity is the tiled result;
the kernels are deterministic."""
import math

import numpy as np
import pytest

from entropy_stable_dg_amd import esdg
from entropy_stable_dg_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def tiles_for(nelem: int, Np: int, itemsize: int, field: int) -> int:
    """Tiles so that field `field` of a [fields][nelem][Np] array starts beyond 2^32 bytes."""
    return math.ceil(2 ** 32 / (field * Np * itemsize) / nelem) + 1


def tiled_nbr(nbr: np.ndarray, reps: int) -> np.ndarray:
    nelem = nbr.shape[0]
    off = (np.arange(reps, dtype=np.int64) * nelem)[:, None, None]
    big = np.where(nbr[None] >= 0, nbr[None].astype(np.int64) + off, -1).reshape(reps * nelem, 6)
    assert big.max() < 2 ** 31
    return big.astype(np.int32)


def check_tiles(big, small, reps, nelem, label):
    for r in sorted({0, 1, reps // 2, reps - 1}):
        got = big[:, r * nelem:(r + 1) * nelem]
        assert torch.equal(got, small), (label, r)
    print(f"[large] {label}: {reps} tiles, {reps * nelem} elements, tiles 0, 1, {reps // 2}, {reps - 1} bitwise equal",
          flush=True)


@pytest.mark.parametrize("name", ["bubble", "bubble_f32"])
def test_volume_term_beyond_4gib(name):
    wl = I.make(name)
    tq, tp, tg, tD = (torch.from_numpy(np.ascontiguousarray(a)).to(dev()) for a in (wl.q, wl.phi, wl.geom, wl.D))
    small = esdg.volume_rhs(tq, tp, tg, tD)
    itemsize = wl.q.dtype.itemsize
    # the rhs's (and q's) last field starts beyond 4 GiB in fp64, geom's last in both
    reps = tiles_for(wl.nelem, wl.q.shape[2], itemsize, 4 if itemsize == 8 else 9)
    big_q, big_p, big_g = tq.repeat(1, reps, 1), tp.repeat(reps, 1), tg.repeat(1, reps, 1)
    fstride_bytes = reps * wl.nelem * wl.q.shape[2] * itemsize
    assert 9 * fstride_bytes > 2 ** 32
    out = esdg.volume_rhs(big_q, big_p, big_g, tD)
    torch.cuda.synchronize()
    check_tiles(out, small, reps, wl.nelem, f"volume term {name}")
    del big_q, big_p, big_g, out
    torch.cuda.empty_cache()


def test_whole_rhs_beyond_4gib():
    wl = I.make("bubble")
    tq, tp, tg, tD = (torch.from_numpy(np.ascontiguousarray(a)).to(dev()) for a in (wl.q, wl.phi, wl.geom, wl.D))
    tn = torch.from_numpy(np.ascontiguousarray(wl.nbr, dtype=np.int32)).to(dev())
    small = esdg.rhs(tq, tp, tg, tD, tn)
    reps = tiles_for(wl.nelem, wl.q.shape[2], 8, 4)
    big_q, big_p, big_g = tq.repeat(1, reps, 1), tp.repeat(reps, 1), tg.repeat(1, reps, 1)
    big_n = torch.from_numpy(tiled_nbr(wl.nbr, reps)).to(dev())
    assert 4 * reps * wl.nelem * wl.q.shape[2] * 8 > 2 ** 32
    out = esdg.rhs(big_q, big_p, big_g, tD, big_n)
    torch.cuda.synchronize()
    check_tiles(out, small, reps, wl.nelem, "whole rhs bubble")
    del big_q, big_p, big_g, big_n, out
    torch.cuda.empty_cache()
