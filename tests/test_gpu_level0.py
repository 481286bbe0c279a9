"""Level 0 in the init kernel: on sorted rows, a source of at most 512 entries
(one per thread of a workgroup) whose level is top-down has its distinct
out-neighbours written as level 0's winners by the init launch (the first
level launch starts at level 1).  The cases around it: exactly 512 entries
(taken there) and 513 (a level launch takes level 0), a row with a
self-loop and repeated entries, a neighbour of degree over 2,048 (its queue
pieces), a source with no out-edges, and unsorted rows (never taken there);
each bit-exact against the oracle, with the default fill of dist and with
the finishing pass.  Graphs of at least 3,585 vertices, so that the
multi-workgroup path runs."""
import contextlib
import os

import numpy as np
import pytest

import graphgen as gg
from gpu_util import check_graph, is_symmetric

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def finish_from(n):
    os.environ["FBFS_FINISH_MIN_N"] = str(n)
    try:
        yield
    finally:
        del os.environ["FBFS_FINISH_MIN_N"]


def _graph(name, n, edges, symmetric_closure, sources):
    """CSR with every row sorted; duplicates and self-loops kept."""
    adj = [[] for _ in range(n)]
    for u, v in edges:
        adj[u].append(v)
        if symmetric_closure and u != v:
            adj[v].append(u)
    adj = [sorted(a) for a in adj]
    row_ptr, col = gg.csr_from_lists(n, adj)
    g = gg.Graph(name, row_ptr, col, False, np.asarray(sources, dtype=np.int32))
    g.symmetric = is_symmetric(g)
    return g


def _level0_graph():
    n = 6000
    e = []
    e += [(0, v) for v in range(1, 513)]            # source 0: 512 distinct neighbours
    e += [(1000, v) for v in range(1001, 1514)]     # source 1000: 513
    e += [(2000, 2000)]                             # source 2000: a self-loop ...
    e += [(2000, v) for v in range(2001, 2011)]
    e += [(2000, v) for v in (2001, 2002, 2003)]    # ... and repeated entries
    e += [(1, v) for v in range(3000, 6000)]        # neighbour 1 of source 0: 3,000 edges
    e += [(5999, 2500)] + [(2500 + i, 2501 + i) for i in range(50)]   # a tail of levels
    e += [(2010, 3000), (1513, 4000)]
    return _graph("level0", n, e, True, [0, 1000, 2000, 1, 5, 2500, 4500])


@pytest.mark.parametrize("finish", [False, True])
def test_level0_in_init(finish):
    g = _level0_graph()
    assert g.symmetric
    assert np.diff(g.row_ptr)[0] == 512 and np.diff(g.row_ptr)[1000] == 513
    ctx = finish_from(0) if finish else contextlib.nullcontext()
    with ctx:
        check_graph(g, label=f"level0 finish={finish}")


@pytest.mark.parametrize("finish", [False, True])
def test_level0_directed(finish):
    """Sorted directed rows: a source without out-edges (one level), and
    sources whose neighbours' in-lists come from the transpose."""
    rng = np.random.default_rng(7)
    n = 5000
    src = rng.integers(0, n, 30000)
    dst = rng.integers(0, n, 30000)
    keep = src % 7 != 0          # every seventh vertex has no out-edges
    edges = list(zip(src[keep].tolist(), dst[keep].tolist()))
    deg_in = np.bincount(dst[keep], minlength=n)
    sink = int(np.nonzero((np.arange(n) % 7 == 0) & (deg_in > 0))[0][0])
    g = _graph("level0 directed", n, edges, False, [sink, 1, 2, 3])
    assert not g.symmetric and np.diff(g.row_ptr)[sink] == 0
    ctx = finish_from(0) if finish else contextlib.nullcontext()
    with ctx:
        check_graph(g, label=f"level0 directed finish={finish}")


def test_level0_unsorted_rows():
    """Unsorted rows: level 0 stays with the level launches."""
    g = _level0_graph()
    col = g.col_idx.copy()
    rng = np.random.default_rng(3)
    for u in (0, 2000, 5):
        a, b = g.row_ptr[u], g.row_ptr[u + 1]
        col[a:b] = rng.permutation(col[a:b])
    h = gg.Graph("level0 unsorted", g.row_ptr, col, False, g.sources)
    check_graph(h, label="level0 unsorted")
