"""Pins of the oracle's MoE dispatch order (moe_permute).

Rows sorted by expert, stable in the order of the routing table (token t,
slot j: entry t*k + j), shared experts as groups of all tokens after the
routed ones; invalid expert ids in no group (the reading of the page "NVIDIA
NeMo RL erreicht 48% Geschwindigkeitssteigerung ...", sections
"Leistungsgewinne in der Praxis" and "Warum dies fuer die KI-Oekonomie wichtig
ist", which name the MoE models but no dispatch order).  Pinned by a brute
force that appends entries to per-expert lists while scanning the table,
closed forms, and invariants that any correct grouping satisfies.
"""
import numpy as np
import pytest

import oracle


def _brute(ids, E, n_shared):
    """Per-expert lists filled by one scan of the table in entry order."""
    T, k = len(ids), len(ids[0])
    lists = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            e = ids[t][j]
            if 0 <= e < E:
                lists[e].append((t, j))
    rows, offsets = [], [0]
    for e in range(E):
        rows.extend(lists[e])
        offsets.append(len(rows))
    entry_row = [[-1] * k for _ in range(T)]
    for r, (t, j) in enumerate(rows):
        entry_row[t][j] = r
    tokens = [t for t, _ in rows]
    for _ in range(n_shared):
        tokens.extend(range(T))
        offsets.append(len(tokens))
    tokens.extend([-1] * (T * (k + n_shared) - len(tokens)))
    return offsets, tokens, [r for row in entry_row for r in row]


@pytest.mark.parametrize("T,k,E,ns,invalid", [
    (1, 1, 1, 0, False), (7, 2, 5, 0, False), (33, 4, 16, 1, False), (50, 8, 8, 2, False),
    (64, 6, 64, 2, False), (40, 3, 9, 0, True), (25, 5, 7, 1, True),
])
def test_matches_brute_force(T, k, E, ns, invalid):
    rng = np.random.default_rng(T * 100 + k)
    ids = np.stack([rng.permutation(max(E, k))[:k] for _ in range(T)]) % E if k <= E else rng.integers(0, E, (T, k))
    if invalid:
        ids = ids.copy()
        ids[rng.random(ids.shape) < 0.2] = -1
        ids[0, 0] = E          # one past the last expert
    off, rows, er = oracle.moe_permute(ids, E, ns)
    boff, brows, ber = _brute(ids.tolist(), E, ns)
    assert off.tolist() == boff
    assert rows.tolist() == brows
    assert er.tolist() == ber


def test_duplicate_experts_in_one_token_keep_slot_order():
    ids = np.array([[2, 2, 0], [2, 1, 2]])
    off, rows, er = oracle.moe_permute(ids, 3)
    assert off.tolist() == [0, 1, 2, 6]
    assert rows.tolist() == [0, 1, 0, 0, 1, 1]
    assert er.tolist() == [2, 3, 0, 4, 1, 5]


def test_identity_routing_closed_form():
    """k = 1, token t to expert t mod E, T = 12E: group e holds tokens e, e+E,
    e+2E, ... in order, 12 rows each."""
    E, T = 8, 96
    ids = (np.arange(T) % E)[:, None]
    off, rows, er = oracle.moe_permute(ids, E, n_shared=1)
    assert off.tolist() == [12 * e for e in range(E + 1)] + [96 + 96]
    for e in range(E):
        assert rows[12 * e:12 * (e + 1)].tolist() == list(range(e, T, E))
    assert rows[96:].tolist() == list(range(T))
    assert er.tolist() == [12 * (t % E) + t // E for t in range(T)]


@pytest.mark.parametrize("seed", [0, 1])
def test_invariants_on_a_large_table(seed):
    """Qwen3-sized table (8192 tokens, top-8 of 128, Zipf-like load): every
    entry lands in its expert's group exactly once, groups follow the entry
    order, the maps are mutual inverses and the counts are the histogram."""
    rng = np.random.default_rng(seed)
    T, k, E = 8192, 8, 128
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    off, rows, er = oracle.moe_permute(ids, E)
    flat = ids.reshape(-1)
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
    assert np.array_equal(np.sort(er), np.arange(T * k))           # a permutation of the rows
    assert np.array_equal(rows[er], np.arange(T * k) // k)          # row of (t, j) holds token t
    for e in (0, 1, 17, 127):
        ent = np.flatnonzero(flat == e)
        assert np.array_equal(er[ent], np.arange(off[e], off[e + 1]))   # in entry order
