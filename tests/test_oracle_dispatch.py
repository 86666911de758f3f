"""Pins for the oracle's dispatch tables and row recovery.

The tutorial (Example 07, moe_dispatch_contract.py) prints the tables of a
9-token, top_k=2, 4-expert example and states three self-checks; the golden
file holds those printed values. The brute-force checks below build the
padded layout explicitly, row by row, which shares nothing with the prefix
sums and the m_start formula they check.
"""
import json
import os
import random

import numpy as np
import pytest

import oracle
import moe_synth


def _load(golden_dir):
    with open(os.path.join(golden_dir, "dispatch_worked_example.json")) as f:
        return json.load(f)


def test_worked_example_printed_tables(golden_dir):
    g = _load(golden_dir)
    p = g["params"]
    ids = np.array(g["topk_ids"], dtype=np.int32)
    assert ids.shape == (p["tokens"], p["top_k"])
    tab = oracle.dispatch_tables(ids, p["experts"], p["padding_m"], p["block_token"])
    pr = g["printed"]
    assert tab["group_sizes"].tolist() == pr["group_sizes"]
    assert tab["group_offsets"].tolist() == pr["group_offsets"]
    assert tab["group_padded_offsets"].tolist() == pr["group_padded_offsets"]
    lengths = np.diff(np.append(tab["group_padded_offsets"], tab["padded_total"])).tolist()
    assert lengths == pr["padded_lengths"]
    assert tab["group_sum"] == pr["group_sum"]
    assert tab["m_blocks"] == pr["m_blocks"]
    assert tab["waste"] == pr["waste_rows"]
    assert tab["group_idx_for_bx"].tolist() == pr["group_idx_for_bx"]


def _brute_padded_layout(ids, E, padding_m):
    """Explicit padded row list: each expert's pairs (ascending pair index) then -1 padding."""
    flat = np.asarray(ids).reshape(-1).tolist()
    rows, owner = [], []
    for e in range(E):
        mine = [p for p, x in enumerate(flat) if x == e]
        pad = (-len(mine)) % padding_m
        rows += mine + [-1] * pad
        owner += [e] * (len(mine) + pad)
    return rows, owner


def _check_contract(ids, E, padding_m, block_m):
    ids = np.asarray(ids, dtype=np.int32)
    tab = oracle.dispatch_tables(ids, E, padding_m, block_m)
    flat = ids.reshape(-1)
    numel = flat.size
    sp = tab["sorted_pair"].tolist()
    # 1. every (token, slot) pair exactly once, grouped by expert in ascending pair order
    assert sorted(sp) == list(range(numel))
    assert [int(flat[p]) for p in sp] == sorted(flat.tolist())
    for e in range(E):
        lo, n = int(tab["group_offsets"][e]), int(tab["group_sizes"][e])
        seg = sp[lo:lo + n]
        assert seg == sorted(seg) and all(flat[p] == e for p in seg)
    assert all(sp[r] == p for p, r in [(sp[r], r) for r in range(numel)])
    p2r = tab["pair_to_row"]
    assert all(sp[int(p2r[p])] == p for p in range(numel))
    # 2. each padded range covers its compact range, lengths multiples of padding_m
    gpo = tab["group_padded_offsets"].tolist() + [tab["padded_total"]]
    for e in range(E):
        n = int(tab["group_sizes"][e])
        plen = gpo[e + 1] - gpo[e]
        assert plen % padding_m == 0 and n <= plen < n + padding_m + (0 if n else 1)
        if n == 0:
            assert plen == 0
    # 3. per block: the brute-force padded layout's block slice equals the
    #    compact rows [m_start, m_start + actual_rows) recovered by the formula
    rows, owner = _brute_padded_layout(ids, E, padding_m)
    covered = []
    assert tab["m_blocks"] == -(-numel // block_m) + E * (padding_m // block_m)
    assert tab["m_blocks"] * block_m >= len(rows)
    for bx in range(tab["m_blocks"]):
        g, m_start, actual = oracle.block_decode(tab, bx, block_m)
        assert 0 <= actual <= block_m
        sl = rows[bx * block_m:(bx + 1) * block_m]
        real = [p for p in sl if p >= 0]
        assert len(real) == actual
        if actual:
            assert owner[bx * block_m] == g
            assert 0 <= m_start and m_start + actual <= numel
            assert sp[m_start:m_start + actual] == real
            covered += list(range(m_start, m_start + actual))
        if bx * block_m < len(rows) and actual == 0:
            assert all(p < 0 for p in sl)
    assert covered == list(range(numel))
    return tab


def test_worked_example_self_checks(golden_dir):
    g = _load(golden_dir)
    p = g["params"]
    tab = _check_contract(g["topk_ids"], p["experts"], p["padding_m"], p["block_token"])
    decoded = [oracle.block_decode(tab, bx, p["block_token"]) for bx in range(tab["m_blocks"])]
    assert [(m, a) for _, m, a in decoded] == [(0, 8), (8, 4), (12, 3), (15, 3), (143, 0)]


def _random_routing(rng, T, E, k, zero_frac=0.0):
    allowed = [e for e in range(E) if rng.random() >= zero_frac] or [0]
    k = min(k, len(allowed))
    return np.array([rng.sample(allowed, k) for _ in range(T)], dtype=np.int32), k


def test_second_parameter_set(golden_dir):
    s = _load(golden_dir)["second_parameter_set"]
    rng = random.Random(40)
    ids, _ = _random_routing(rng, s["tokens"], s["experts"], s["top_k"])
    _check_contract(ids, s["experts"], s["padding_m"], s["block_token"])


@pytest.mark.parametrize("seed", range(12))
def test_random_routings(seed):
    rng = random.Random(seed)
    E = rng.choice([1, 2, 3, 5, 8, 13])
    T = rng.choice([0, 1, 3, 17, 64, 130])
    k = rng.randint(1, min(E, 4))
    bm = rng.choice([1, 4, 16, 64])
    pm = bm * rng.choice([1, 2, 4])
    ids, k = _random_routing(rng, T, E, k, zero_frac=0.4)
    if T == 0:
        ids = np.zeros((0, k), dtype=np.int32)
    _check_contract(ids, E, pm, bm)


def test_exact_multiples_and_single_expert():
    # every group an exact multiple of padding_m: no extra padding, no waste blocks inside
    ids = np.array([[0], [0], [1], [1], [2], [2], [2], [2]], dtype=np.int32)
    tab = _check_contract(ids, 4, 2, 2)
    assert tab["group_padded_offsets"].tolist() == [0, 2, 4, 8]
    assert tab["group_idx_for_bx"].tolist() == [0, 1, 2, 2, 3, 3, 3, 3]
    # all pairs on one expert
    ids = np.full((50, 1), 3, dtype=np.int32)
    tab = _check_contract(ids, 5, 16, 16)
    assert tab["group_sizes"].tolist() == [0, 0, 0, 50, 0]


@pytest.mark.parametrize("name", ["tiny", "qwen3_decode"])
def test_config_routings(name):
    cfg = moe_synth.CONFIGS[name]
    logits = moe_synth.router_logits(cfg).numpy()
    ids, _ = oracle.route(logits, cfg.top_k)
    _check_contract(ids, cfg.E, cfg.padding_m, cfg.block_m)


def test_invalid_arguments():
    ids = np.array([[0, 1]], dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.dispatch_tables(ids, 2, 96, 64)       # padding not a multiple of the block
    with pytest.raises(ValueError):
        oracle.dispatch_tables(np.array([[0, 2]]), 2, 64, 64)
