"""Host logic of bench.py's quality figures (CPU only).

planted_recall counts the generator's planted blocks that a selection kept; _compare_rows is
the comparison the cpu_baseline leg reports as parity_sample.  Both are checked here against
brute force and constructed cases, with the oracle's own selections standing in for the
device's.
"""
import numpy as np
import pytest
import torch

import bench
import oracle as O
from workloads import SPECS, make_workload


def _oracle_selection(spec, seed):
    """The oracle's block selection of a prefill workload (pool, scores, top-k)."""
    w = make_workload(spec, seed)
    q = w.q.float().numpy()
    pt = w.page_table.numpy()
    cache = O.block_pool(w.k_cache.float().numpy(), pt, w.kv_lens_host, spec.dtype)
    sc = O.group_scores(q, cache, pt, w.kv_lens_host, spec.num_kv_heads, spec.page_size)
    return w, O.select_blocks(sc, w.kv_lens_host, q.shape[2], spec.page_size, spec.top_k)


@pytest.mark.parametrize("spec", [
    SPECS[1].replace(seq_len=64 * 24 + 7, top_k=6),                          # token planting
    SPECS[3].replace(seq_len=128 * 40 + 3, top_k=8, region=1024),             # region planting + recency
], ids=["token", "region"])
def test_planted_recall_matches_brute_force(spec):
    w, sel = _oracle_selection(spec, 5)
    idx = torch.from_numpy(sel)
    got = bench.planted_recall(idx, w)
    hit = tot = 0
    B, Hkv, S, _ = idx.shape
    for b in range(B):
        for g in range(Hkv):
            for t in range(S):
                kept = set(idx[b, g, t].tolist())
                pl = w.planted_for(b, g, t)
                tot += len(pl)
                hit += sum(1 for x in pl if x in kept)
    assert got["planted"] == tot and got["kept"] == hit
    assert tot > 0 and got["recall"] == hit / tot
    # a selection that drops every planted block scores zero
    none = torch.full_like(idx, -1)
    assert bench.planted_recall(none, w)["kept"] == 0


def _rows(scores, k, n_tok):
    """Oracle-style selection of hand-made scores: [1, 1, n_tok, nb] -> block ids."""
    return O.select_blocks(scores, [scores.shape[-1] * 64], n_tok, 64, k)


def test_compare_rows_counts_differences_and_tie_window():
    rng = np.random.default_rng(3)
    nb, k, n_tok = 12, 4, 3
    sc = rng.normal(size=(1, 1, n_tok, nb)) * 10.0
    # every row's own block is the last one, so all 11 earlier blocks are candidates
    for t in range(n_tok):
        sc[0, 0, t, nb - 1] = -np.inf
    ora = _rows(sc, k, n_tok)
    out = rng.normal(size=(1, 4, n_tok, 8))
    c = bench._compare_rows(ora.copy(), out.astype(np.float32), ora, out, sc, k)
    assert c["rows"] == n_tok and c["idx_rows_differing"] == 0 and c["idx_rows_in_tie_window"] == 0
    assert c["out_max_abs_err"] < 1e-6

    # row 1: the (k-1)-th and k-th candidates tie within 1e-4 relative; taking the k-th instead
    # is exempt.  Row 2: swapping in the worst candidate is a real difference.
    order = sorted(range(nb - 1), key=lambda j: -sc[0, 0, 1, j])
    a, b_ = order[k - 2], order[k - 1]
    sc[0, 0, 1, b_] = sc[0, 0, 1, a] * (1 - 1e-6)
    ora = _rows(sc, k, n_tok)
    dev = ora.copy()
    row = [x for x in dev[0, 0, 1] if x != a and x >= 0]
    dev[0, 0, 1] = sorted(row[:-1] + [b_]) + [row[-1]]
    worst = sorted(range(nb - 1), key=lambda j: sc[0, 0, 2, j])[0]
    r2 = list(dev[0, 0, 2])
    r2[0] = worst
    dev[0, 0, 2] = sorted(r2[:-1]) + [r2[-1]]
    out_dev = out.copy()
    out_dev[0, 2, 0, 3] += 0.25
    c = bench._compare_rows(dev, out_dev.astype(np.float32), ora, out, sc, k)
    assert c["idx_rows_differing"] == 2
    assert c["idx_rows_in_tie_window"] == 1
    assert abs(c["out_max_abs_err"] - 0.25) < 1e-6
