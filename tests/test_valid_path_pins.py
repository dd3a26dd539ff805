"""Pins of the valid-path oracle (oracle.valid_next_tokens / apply_valid_mask).

xGR summary, section 2.2: a beam may only extend along paths of a pre-built
vocabulary of valid items.  The oracle answers by brute force over the item
list; these tests check it against hand-derived cases and against an
independent trie built from Python dictionaries.
"""
import numpy as np
import pytest

import oracle
from generative_recommendation_beam_xattn_amd import workloads as W

ITEMS = np.array([[1, 2, 3], [1, 2, 4], [1, 7, 0], [5, 0, 0], [5, 0, 0]], np.int32)


def test_hand_derived_masks():
    assert oracle.valid_next_tokens(ITEMS, []).tolist() == [1, 5]
    assert oracle.valid_next_tokens(ITEMS, [1]).tolist() == [2, 7]
    assert oracle.valid_next_tokens(ITEMS, [1, 2]).tolist() == [3, 4]
    assert oracle.valid_next_tokens(ITEMS, [5]).tolist() == [0]
    assert oracle.valid_next_tokens(ITEMS, [5, 0]).tolist() == [0]     # duplicate item
    assert oracle.valid_next_tokens(ITEMS, [3]).tolist() == []         # not a prefix
    assert oracle.valid_next_tokens(ITEMS, [1, 3]).tolist() == []
    assert oracle.valid_next_tokens(ITEMS, None).tolist() == []        # dead beam
    with pytest.raises(ValueError):
        oracle.valid_next_tokens(ITEMS, [1, 2, 3])


def test_masking_keeps_valid_values_only():
    logits = np.arange(2 * 8, dtype=np.float32).reshape(2, 8)
    got = oracle.apply_valid_mask(ITEMS, [[1], [5, 0]], logits)
    ninf = -np.inf
    assert got[0].tolist() == [ninf, ninf, 2.0, ninf, ninf, ninf, ninf, 7.0]
    assert got[1].tolist() == [8.0] + [ninf] * 7


def dict_trie(items):
    root = {}
    for it in items:
        node = root
        for tok in it:
            node = node.setdefault(int(tok), {})
    return root


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_dictionary_trie(seed):
    items = W.valid_items(seed, n_items=300, levels=3, vocab=40)
    trie = dict_trie(items)
    rng = np.random.default_rng(seed)
    # every prefix of every item, plus random (mostly invalid) prefixes
    prefixes = [list(items[i, :d]) for i in range(0, 300, 7) for d in range(3)]
    prefixes += [list(rng.integers(0, 40, size=d)) for d in (0, 1, 2) for _ in range(20)]
    for p in prefixes:
        node = trie
        for tok in p:
            node = node.get(int(tok)) if node is not None else None
        want = sorted(node) if node is not None else []
        assert oracle.valid_next_tokens(items, p).tolist() == want


def test_every_item_path_is_valid_and_counts_match():
    items = W.valid_items(4, n_items=500, levels=3, vocab=32)
    uniq = np.unique(items, axis=0)
    for it in uniq[:50]:
        for d in range(3):
            assert it[d] in oracle.valid_next_tokens(items, list(it[:d]))
    # valid (prefix, token) pairs at depth d = distinct prefixes of length d + 1
    for d in range(3):
        prefixes = np.unique(uniq[:, :d], axis=0) if d else np.zeros((1, 0), np.int32)
        total = sum(len(oracle.valid_next_tokens(items, list(p))) for p in prefixes)
        assert total == len(np.unique(uniq[:, : d + 1], axis=0))
