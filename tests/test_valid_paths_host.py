"""Host-side valid-path tables (xattn_trie_build), checked on the CPU.

The tables are decoded here from their documented layout and compared with
the oracle's brute-force item membership: every node's children are exactly
the valid next tokens of its prefix, in ascending order, nodes are numbered
in lexicographic prefix order, and the dense rows hold the same sets.
"""
import ctypes

import numpy as np
import pytest

import oracle
from generative_recommendation_beam_xattn_amd import binding as B
from generative_recommendation_beam_xattn_amd import workloads as W


def decode(lay, table):
    """prefixes[d][n] and children[d][n] (token list) for every node."""
    i32 = table.view(np.int32)
    prefixes = [[()]]
    children = []
    for d in range(lay.levels):
        n_d, n_next = lay.nodes[d], lay.nodes[d + 1]
        rp = i32[lay.row_ptr_off[d] // 4: lay.row_ptr_off[d] // 4 + n_d + 1]
        ct = i32[lay.child_tok_off[d] // 4: lay.child_tok_off[d] // 4 + n_next]
        assert rp[0] == 0 and rp[-1] == n_next and np.all(np.diff(rp) >= 0)
        kids, nxt = [], [None] * n_next
        for n in range(n_d):
            toks = ct[rp[n]: rp[n + 1]].tolist()
            kids.append(toks)
            for e in range(rp[n], rp[n + 1]):
                nxt[e] = prefixes[d][n] + (int(ct[e]),)
        children.append(kids)
        prefixes.append(nxt)
    return prefixes, children


@pytest.mark.parametrize("seed,n,L,V,dense", [(0, 500, 3, 40, 2), (1, 3000, 3, 256, 1),
                                              (2, 200, 4, 16, 0), (3, 50, 1, 8, 1),
                                              (4, 1000, 2, 33, 2)])
def test_tables_match_brute_force(seed, n, L, V, dense):
    items = W.valid_items(seed, n_items=n, levels=L, vocab=V)
    lay, table = B.trie_build(items, V, dense)
    assert (lay.vocab, lay.levels, lay.dense_levels, lay.words) == (V, L, dense, (V + 31) // 32)
    prefixes, children = decode(lay, table)
    for d in range(L):
        # lexicographic numbering
        assert prefixes[d] == sorted(prefixes[d])
        assert len(set(prefixes[d + 1])) == len(prefixes[d + 1])
        for nd, p in enumerate(prefixes[d]):
            want = oracle.valid_next_tokens(items, list(p)).tolist()
            assert children[d][nd] == want, (d, p)
    assert len(prefixes[L]) == len(np.unique(items, axis=0))
    words = lay.words
    u32 = table.view(np.uint32)
    for d in range(dense):
        m = u32[lay.mask_off[d] // 4: lay.mask_off[d] // 4 + lay.nodes[d] * words]
        m = m.reshape(lay.nodes[d], words)
        for nd in range(lay.nodes[d]):
            bits = [j for j in range(V) if (m[nd, j >> 5] >> (j & 31)) & 1]
            assert bits == children[d][nd]


def test_sections_are_aligned_and_within_the_buffer():
    items = W.valid_items(9, n_items=777, levels=3, vocab=100)
    lay, table = B.trie_build(items, 100, 2)
    offs = [lay.row_ptr_off[d] for d in range(3)] + [lay.child_tok_off[d] for d in range(3)] + \
        [lay.mask_off[d] for d in range(2)]
    assert all(o % 256 == 0 and 0 < o < lay.total_bytes for o in offs)
    assert table.nbytes == lay.total_bytes


def test_empty_vocabulary_has_a_root_without_children():
    lay, table = B.trie_build(np.zeros((0, 3), np.int32), 10, 1)
    assert list(lay.nodes)[:4] == [1, 0, 0, 0]
    _, children = decode(lay, table)
    assert children[0] == [[]]


def test_build_rejects_bad_input():
    lib = B.load()
    lay = B.Trie()
    items = np.array([[1, 2], [3, 9]], np.int32)
    ptr = items.ctypes.data_as(ctypes.c_void_p)
    assert lib.xattn_trie_build(ptr, 2, 2, 9, 1, ctypes.byref(lay), None, 0) == 1
    assert "outside" in lib.xattn_last_error().decode()
    for levels in (0, 9):
        assert lib.xattn_trie_build(ptr, 1, levels, 10, 0, ctypes.byref(lay), None, 0) == 1
    assert lib.xattn_trie_build(ptr, 2, 2, 10, 3, ctypes.byref(lay), None, 0) == 1
    assert lib.xattn_trie_build(ptr, 2, 2, 10, 1, None, None, 0) == 1
    assert lib.xattn_trie_build(ptr, 2, 2, 10, 1, ctypes.byref(lay), None, 0) == 0
    small = np.zeros(16, np.uint8)
    assert lib.xattn_trie_build(ptr, 2, 2, 10, 1, ctypes.byref(lay),
                                small.ctypes.data_as(ctypes.c_void_p), 16) == 1
    assert "host_bytes" in lib.xattn_last_error().decode()


def test_mask_and_advance_reject_bad_arguments():
    lib = B.load()
    items = W.valid_items(1, n_items=50, levels=3, vocab=64)
    lay, _ = B.trie_build(items, 64, 2)
    fake = ctypes.c_void_p(0x100000)
    assert lib.xattn_valid_mask(ctypes.byref(lay), fake, 3, fake, fake, 1, 1, 64, None) == 1
    assert "depth" in lib.xattn_last_error().decode()
    assert lib.xattn_valid_mask(ctypes.byref(lay), fake, 0, fake, fake, 1, 1, 62, None) == 1
    assert "row_stride" in lib.xattn_last_error().decode()
    assert lib.xattn_valid_mask(None, fake, 0, fake, fake, 1, 1, 64, None) == 1
    assert lib.xattn_valid_mask(ctypes.byref(lay), ctypes.c_void_p(0x100010), 0, fake, fake, 1,
                                1, 64, None) == 1
    assert "256-byte" in lib.xattn_last_error().decode()
    bad = B.Trie()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(lay), ctypes.sizeof(lay))
    bad.words = 7
    assert lib.xattn_valid_mask(ctypes.byref(bad), fake, 0, fake, fake, 1, 1, 64, None) == 1
    assert "layout" in lib.xattn_last_error().decode()
    assert lib.xattn_trie_advance(ctypes.byref(lay), fake, 0, fake, fake, 3, fake, 4, fake, 2, 4,
                                  None) == 1
    assert "stride" in lib.xattn_last_error().decode()
    assert lib.xattn_valid_mask_timed(ctypes.byref(lay), fake, 0, fake, fake, 1, 1, 64, None,
                                      None, fake) == 1
