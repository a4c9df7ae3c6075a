"""Host-side check of the volume kernel's launch geometry: the index arithmetic
of every phase, replayed on the CPU for every compiled order, stays inside the
buffers it touches, and each (direction, node) partial-sum slot in LDS is
written by exactly one line thread.  Mirrors entropy_stable_dg_amd/csrc
(volume_kernel.hpp and the launch table in launch_table.hpp)."""
import re

import numpy as np
import pytest

import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
API = os.path.join(ROOT, "entropy_stable_dg_amd", "csrc", "launch_table.hpp")
KERNEL = os.path.join(ROOT, "entropy_stable_dg_amd", "csrc", "volume_kernel.hpp")

NODE_VALUES = 19     # staged values per node (10 state values + 9 metric terms)
PARTIAL_VALUES = 15  # 3 directions x 5 fields


def launch_table():
    """{(dtype, N): (EPB, NT, metric_in_lds, line order, finish_in_line)} from launch_table.hpp;
    line order 0 element-major, 1 direction-major, 2 direction-major with each
    direction on a 32-lane boundary."""
    text = open(API).read()
    rows = re.findall(r"struct Launch<(double|float), (\d+)>\s*\{\s*using C = LaunchCfg<([^>]*)>;", text)
    table = {}
    for dt, n, args in rows:
        parts = [a.strip() for a in args.split(",")]
        epb, nt = int(parts[0]), int(parts[1])
        metric = parts[3] != "false" if len(parts) > 3 else True
        kmajor = {"true": 1, "false": 0}.get(parts[5], None) if len(parts) > 5 else 0
        if kmajor is None:
            kmajor = int(parts[5])
        fin = parts[6] == "true" if len(parts) > 6 else False
        table[(dt, int(n))] = (epb, nt, metric, kmajor, fin)
    return table


def line_task(task, EPB, Nq2, kmajor):
    """(element in batch, direction, line) of a line thread, as LineTask maps it;
    returns the number of task threads too (threads at or past it are idle)."""
    lines = 3 * EPB * Nq2
    if kmajor:
        stride = (EPB * Nq2 + 31) // 32 * 32 if kmajor == 2 else EPB * Nq2
        k, r = divmod(task, stride)
        eb, line = divmod(r, Nq2)   # r past the direction's lines gives eb >= EPB: idle
        if k > 2:
            k, eb = 2, EPB
        return eb, k, line, 3 * stride
    eb, r3 = divmod(task, 3 * Nq2)
    k, line = divmod(r3, Nq2)
    return eb, k, line, lines


def test_launch_table_covers_orders():
    t = launch_table()
    assert sorted(n for d, n in t if d == "double") == list(range(1, 9))
    assert sorted(n for d, n in t if d == "float") == list(range(1, 9))


def test_staged_value_count_matches_kernel():
    text = open(KERNEL).read()
    m = re.search(r"enum NodeValue \{(.*?)\};", text, flags=re.S)
    body = m.group(1)
    assert "kJa + 9" in body
    names = [x.strip().split("=")[0].strip() for x in body.split(",")]
    assert names.index("kJa") + 9 == NODE_VALUES


@pytest.mark.parametrize("dtype", ["double", "float"])
@pytest.mark.parametrize("N", range(1, 9))
@pytest.mark.parametrize("nelem", [1, 2, 5, 13])
def test_indices_in_bounds(dtype, N, nelem):
    EPB, NT, metric_in_lds, kmajor, fin = launch_table()[(dtype, N)]
    Nq = N + 1
    Nq2, Np = Nq * Nq, Nq ** 3
    NODES = EPB * Np
    staged = NODE_VALUES if metric_in_lds else 10
    partials = 10 if fin else PARTIAL_VALUES
    region = max(staged, partials)
    lds_values = (region + (1 if fin else 0)) * NODES
    lines = 3 * EPB * Nq2
    assert lines <= NT
    node_iters = (NODES + NT - 1) // NT
    blocks = (nelem + EPB - 1) // EPB
    fstride = nelem * Np
    written = np.zeros((3, nelem * Np), dtype=int)
    out_written = np.zeros(nelem * Np, dtype=int)
    for blk in range(blocks):
        e0 = blk * EPB
        nvalid = min(EPB, nelem - e0) * Np
        g0 = e0 * Np
        # phase A / D: node threads, node_iters nodes each
        for t in range(NT):
            for it in range(node_iters):
                tt = t + it * NT
                # every lane loads, one past the batch's nodes the last one
                gl = g0 + min(tt, nvalid - 1)
                assert 0 <= gl and 9 * fstride + gl < 10 * fstride
                pnode = (N // 2) * (1 + Nq + Nq2)
                assert fstride + g0 + (min(tt, nvalid - 1) // Np) * Np + pnode < 2 * fstride
                if tt >= nvalid:
                    continue
                g = g0 + tt
                assert 0 <= g and 4 * fstride + g < 5 * fstride and 9 * fstride + g < 10 * fstride
                assert (staged - 1) * NODES + tt < lds_values
                if fin:
                    assert region * NODES + tt < lds_values          # staged -1/J
                else:
                    assert (10 + 4) * NODES + tt < lds_values    # phase D reads
                    out_written[g] += 1
        # phase B / C: line threads
        for task in range(NT):
            eb, k, line, task_threads = line_task(task, EPB, Nq2, kmajor)
            assert task_threads <= NT
            p1, p2 = line % Nq, line // Nq
            base = [Nq * (p1 + Nq * p2), p1 + Nq2 * p2, p1 + Nq * p2][k]
            step = [1, Nq, Nq2][k]
            active = task < task_threads and eb * Np < nvalid
            # phase A loads every lane issues, an idle lane for its element
            # clamped to the batch's last one: the line metric and (fp32 on
            # perturbation variables) the element's reference pressure
            own = blk * EPB + min(eb, nvalid // Np - 1)
            if not metric_in_lds:
                for a in range(Nq):
                    for j in range(3):
                        gm = (3 * k + j) * fstride + own * Np + base + a * step
                        assert 0 <= gm < 9 * fstride
            pnode = (N // 2) * (1 + Nq + Nq2)
            assert 0 <= fstride + own * Np + pnode < 2 * fstride
            if not active:
                continue
            nb = eb * Np + base
            for a in range(Nq):
                s = nb + a * step
                assert eb * Np <= s < (eb + 1) * Np <= NODES
                if metric_in_lds:
                    assert (10 + 3 * k + 2) * NODES + s < lds_values   # staged reads
                else:
                    assert (3 * k + 2) * fstride + g0 + s < 9 * fstride  # direct metric loads
                assert 9 * NODES + s < lds_values
                if fin and k == 2:
                    assert region * NODES + s < lds_values and 9 * NODES + s < lds_values
                    assert 4 * fstride + g0 + s < 5 * fstride        # direct store
                    out_written[g0 + s] += 1
                else:
                    assert (k * 5 + 4) * NODES + s < (region if fin else lds_values // NODES) * NODES
                written[k, g0 + s] += 1
                for l in range(a + 1, Nq):
                    assert a * Nq + l < Nq2 and l * Nq + a < Nq2    # D reads
    assert np.all(written == 1)
    assert np.all(out_written == 1)


@pytest.mark.parametrize("dtype", ["double", "float"])
@pytest.mark.parametrize("N", range(1, 9))
@pytest.mark.parametrize("K,periodic", [((1, 1, 1), (True, True, True)),
                                        ((3, 2, 1), (True, False, True)),
                                        ((2, 3, 2), (False, False, False))])
def test_face_partner_indices(dtype, N, K, periodic):
    """Surface term of the whole right-hand side: each line thread's two ends
    read the neighbour index of faces 2k and 2k+1 of its own element and load
    the matching node of that neighbour, the other end of the same line:
    in bounds, on the opposite face, same tangential indices; every
    (element, face, face node) is handled by exactly one line end."""
    from entropy_stable_dg_amd import inputs as I

    EPB, NT, _, kmajor, _ = launch_table()[(dtype, N)]
    Nq = N + 1
    Nq2, Np = Nq * Nq, Nq ** 3
    nbr = I.box_connectivity(K, periodic)
    nelem = nbr.shape[0]
    blocks = (nelem + EPB - 1) // EPB
    seen = np.zeros((nelem, 6, Nq2), dtype=int)

    def abc(n):
        return n % Nq, (n // Nq) % Nq, n // Nq2

    for blk in range(blocks):
        nvalid = min(EPB, nelem - blk * EPB) * Np
        for task in range(NT):
            eb, k, line, task_threads = line_task(task, EPB, Nq2, kmajor)
            p1, p2 = line % Nq, line // Nq
            base = [Nq * (p1 + Nq * p2), p1 + Nq2 * p2, p1 + Nq * p2][k]
            step = [1, Nq, Nq2][k]
            # every lane loads its neighbour indices and both partner nodes,
            # an idle lane for its element clamped to the batch's last one, a wall or
            # an invalid index from the lane's own element (in bounds, unused)
            own_e = blk * EPB + min(eb, nvalid // Np - 1)
            assert 0 <= 6 * own_e + 2 * k and 6 * own_e + 2 * k + 1 < 6 * nelem
            for end in (0, 1):
                nbe = nbr[own_e, 2 * k + end]
                src = nbe if 0 <= nbe < nelem else own_e
                g = src * Np + base + (N if end == 0 else 0) * step
                assert 0 <= g < nelem * Np
            if not (task < task_threads and eb * Np < nvalid):
                continue
            e = blk * EPB + eb
            assert 0 <= 6 * e + 2 * k + 1 < 6 * nelem
            for end in (0, 1):
                a = N if end else 0
                own = base + a * step
                face = 2 * k + end
                nb = nbr[e, face]
                tang = [x for i, x in enumerate(abc(own)) if i != k]
                seen[e, face, tang[0] + Nq * tang[1]] += 1
                if nb < 0:
                    continue
                partner = base + (N if end == 0 else 0) * step
                g = nb * Np + partner
                assert 0 <= g < nelem * Np and 4 * nelem * Np + g < 5 * nelem * Np
                pa = abc(partner)
                assert pa[k] == N - abc(own)[k]
                assert [x for i, x in enumerate(pa) if i != k] == tang
    assert np.all(seen == 1)


def test_xcd_batch_order_is_a_bijection():
    """The whole right-hand side maps workgroup b to batch xcd_batch(b, nb):
    every batch is taken exactly once, for any grid size."""
    text = open(KERNEL).read()
    assert "const int64_t x = block % kXcds, i = block / kXcds;" in text
    assert "return x * q + (x < r ? x : r) + i;" in text
    X = int(re.search(r"constexpr int kXcds = (\d+);", text).group(1))

    def xcd_batch(block, nb):
        x, i = block % X, block // X
        q, r = nb // X, nb % X
        return x * q + (x if x < r else r) + i

    for nb in list(range(1, 200)) + [1366, 3414, 4609, 87382]:
        assert sorted(xcd_batch(b, nb) for b in range(nb)) == list(range(nb))
