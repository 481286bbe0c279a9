"""The algorithmic byte model on hand-counted cases."""
import numpy as np

import graphgen as gg
from frontier_bfs_csr_amd import bytemodel


def test_topdown_chapter22():
    g = gg.chapter22_graph()
    dist = np.array([0, 1, 1, 2, 2, 3], np.int32)
    init, lv, _ = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.zeros(4, np.int8))
    # init: 4n dist + 4n parent + ceil(n/8) visited
    assert init == 24 + 24 + 1
    # level k: 12|F_k| + 4 sum deg(F_k) + 12 |F_k+1|
    assert lv.tolist() == [12 + 8 + 24, 24 + 16 + 24, 24 + 12 + 12, 12]
    init, lv, _ = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.zeros(4, np.int8), with_parent=False)
    assert init == 25 and lv.tolist() == [12 + 8 + 16, 24 + 16 + 16, 24 + 12 + 8, 12]


def test_bottomup_pmpp():
    g = gg.pmpp_graph()
    dist = np.array([0, 1, 1, 2], np.int32)
    init, lv, _ = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.ones(3, np.int8))
    assert init == 16 + 16 + 1
    # level 0: bitmaps 1+1, U={1,2,3}: 24, scans 1+1+1 entries: 12, 2 found: 16
    # level 1: U={3}: 8, scan of adj(3)=[2] hits at once: 4, 1 found: 8
    # level 2: nothing left
    assert lv.tolist() == [2 + 24 + 12 + 16, 2 + 8 + 4 + 8, 2]


def test_isolated_vertices_not_counted_in_bottom_up():
    g = gg.disjoint_union(gg.pmpp_graph(), gg.path_graph(1))   # vertex 4 isolated
    dist = np.array([0, 1, 1, 2, -1], np.int32)
    _, lv, _ = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.ones(3, np.int8))
    assert lv.tolist() == [2 + 24 + 12 + 16, 2 + 8 + 4 + 8, 2]


def test_bottomup_directed_uses_in_edges():
    """P5's directed graph pulled over its in-edges: in-lists 1:[0] 2:[0,1]
    3:[1,2] 4:[2,3] 5:[3,4], counted by hand."""
    g = gg.chapter22_graph()
    dist = np.array([0, 1, 1, 2, 2, 3], np.int32)
    in_csr = bytemodel.transpose(g.row_ptr, g.col_idx)
    assert in_csr[0].tolist() == [0, 0, 1, 3, 5, 7, 9]
    assert in_csr[1].tolist() == [0, 0, 1, 1, 2, 2, 3, 3, 4]
    _, lv, _ = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.ones(4, np.int8), in_csr=in_csr)
    # level 0: U={1..5} 40, scans 1+1+2+2+2 = 8 entries 32, 2 found 16, bitmaps 2
    # level 1: U={3,4,5} 24, scans 1+1+2 16, 2 found 16, bitmaps 2
    # level 2: U={5} 8, scan 1 entry 4, 1 found 8, bitmaps 2
    assert lv.tolist() == [90, 58, 22, 2]



def test_level_flags_move_dist_bytes():
    """Where a level's dist stores went, counted by hand on the worked graphs.
    Chapter 22 pushed: level 0 queue-free (2 new vertices cost their parent,
    4 each, plus the next bitmap, 1 byte, instead of 12 each); level 1 writes
    its frontier's dist (+4 per frontier vertex)."""
    g = gg.chapter22_graph()
    dist = np.array([0, 1, 1, 2, 2, 3], np.int32)
    init, lv, fin = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.zeros(4, np.int8),
                                        flags=np.array([1, 8, 0, 0], np.uint8))
    assert init == 24 + 24 + 1 and fin == 0
    assert lv.tolist() == [12 + 8 + 4 * 2 + 1, 24 + 16 + 24 + 4 * 2, 24 + 12 + 12, 12]


def test_level_flags_finishing_pass():
    """PMPP's graph pulled, levels 0 and 1 keeping their finds as bitmaps and
    the finishing pass writing dist: the init writes parent and visited only
    (16 + 1); a kept level writes parents (4 per find) and its bitmap (1 byte)
    beside the two bitmaps every bottom-up level moves; the finishing pass
    reads the visited bitmap, the template and the 2 kept bitmaps (1 byte
    each) and writes dist of the 3 kept vertices (12 bytes)."""
    g = gg.pmpp_graph()
    dist = np.array([0, 1, 1, 2], np.int32)
    init, lv, fin = bytemodel.alg_bytes(g.row_ptr, g.col_idx, dist, np.ones(3, np.int8),
                                        flags=np.array([16 | 2, 2, 0], np.uint8))
    assert init == 16 + 1
    assert lv.tolist() == [1 + 24 + 12 + 4 * 2 + 1 + 1, 1 + 8 + 4 + 4 * 1 + 1 + 1, 2]
    assert fin == 1 + 1 + 2 + 4 * 3
    # an unreached isolated vertex: the finishing pass writes its -1 too
    h = gg.disjoint_union(gg.pmpp_graph(), gg.path_graph(1))
    d2 = np.array([0, 1, 1, 2, -1], np.int32)
    _, _, fin2 = bytemodel.alg_bytes(h.row_ptr, h.col_idx, d2, np.ones(3, np.int8),
                                     flags=np.array([16 | 2, 2, 0], np.uint8))
    assert fin2 == 1 + 1 + 2 + 4 * 4
