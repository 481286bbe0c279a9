"""The algorithmic byte model on hand-counted cases."""
import numpy as np

import graphgen as gg
from frontier_bfs_csr_amd import bytemodel


def test_topdown_chapter22():
    g = gg.chapter22_graph()
    dist = np.array([0, 1, 1, 2, 2, 3], np.int32)
    init, lv = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.zeros(4, np.int8))
    # init: 4n dist + 4n parent + ceil(n/8) visited
    assert init == 24 + 24 + 1
    # level k: 12|F_k| + 4 sum deg(F_k) + 12 |F_k+1|
    assert lv.tolist() == [12 + 8 + 24, 24 + 16 + 24, 24 + 12 + 12, 12]
    init, lv = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.zeros(4, np.int8), with_parent=False)
    assert init == 25 and lv.tolist() == [12 + 8 + 16, 24 + 16 + 16, 24 + 12 + 8, 12]


def test_bottomup_pmpp():
    g = gg.pmpp_graph()
    dist = np.array([0, 1, 1, 2], np.int32)
    init, lv = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.ones(3, np.int8))
    assert init == 16 + 16 + 1
    # level 0: bitmaps 1+1, U={1,2,3}: 24, scans 1+1+1 entries: 12, 2 found: 16
    # level 1: U={3}: 8, scan of adj(3)=[2] hits at once: 4, 1 found: 8
    # level 2: nothing left
    assert lv.tolist() == [2 + 24 + 12 + 16, 2 + 8 + 4 + 8, 2]


def test_isolated_vertices_not_counted_in_bottom_up():
    g = gg.disjoint_union(gg.pmpp_graph(), gg.path_graph(1))   # vertex 4 isolated
    dist = np.array([0, 1, 1, 2, -1], np.int32)
    _, lv = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.ones(3, np.int8))
    assert lv.tolist() == [2 + 24 + 12 + 16, 2 + 8 + 4 + 8, 2]
