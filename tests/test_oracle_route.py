"""Pins for the oracle's router top-k and routing metadata: brute force over every
k-subset, closed forms and special cases of the renormalised gates, the hand-worked
round-robin gates (tests/golden/roundrobin_gates.txt), metadata invariants and a
pure-Python dictionary-of-lists construction of the expert-major row order."""

import itertools
import os

import numpy as np
import pytest

import synth
from oracle import moe


def brute_force_topk_set(row, k):
    """Among all k-subsets, those with the largest logit sum; the lexicographically
    smallest sorted id tuple (ties toward lower expert ids).  Integer logits keep the
    sums exact."""
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(row)), k):
        s = sum(row[i] for i in sub)
        if best_sum is None or s > best_sum or (s == best_sum and sub < best):
            best, best_sum = sub, s
    return best


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (8, 2), (8, 8), (10, 4)])
def test_topk_set_matches_brute_force(E, k):
    rng = np.random.default_rng(E * 100 + k)
    logits = rng.integers(-3, 4, size=(60, E)).astype(np.float64)   # many exact ties
    idx, gate, _ = moe.route_topk(logits, k)
    for t in range(60):
        assert tuple(sorted(idx[t].tolist())) == brute_force_topk_set(logits[t].tolist(), k)
        # slot order: descending logit, ties toward the lower expert id
        keys = [(-logits[t, e], e) for e in idx[t]]
        assert keys == sorted(keys)


def test_gates_closed_form_softmax_of_selected_logits():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((200, 16)) * 3
    idx, gate, probs = moe.route_topk(logits, 5)
    sel = np.take_along_axis(logits, idx.astype(np.int64), axis=1)
    # closed form: exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected logits only
    cf = np.exp(sel - sel[:, :1]) / np.exp(sel - sel[:, :1]).sum(axis=1, keepdims=True)
    assert np.allclose(gate, cf, rtol=1e-13, atol=1e-15)
    assert np.allclose(gate.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(gate, axis=1) <= 0) and np.all(gate > 0) and np.all(gate <= 1)
    assert np.allclose(probs.sum(axis=1), 1.0, atol=1e-14)


def test_special_cases():
    T, E = 20, 7
    eq = np.zeros((T, E))
    idx, gate, _ = moe.route_topk(eq, 3)
    assert np.array_equal(idx, np.tile(np.arange(3), (T, 1))) and np.allclose(gate, 1 / 3)
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((T, E))
    _, g1, _ = moe.route_topk(lg, 1)
    assert np.all(g1 == 1.0)
    idxE, gE, probs = moe.route_topk(lg, E)
    assert np.allclose(gE, np.take_along_axis(probs, idxE.astype(np.int64), axis=1), rtol=1e-14)


def test_roundrobin_gates_golden(golden_dir):
    with open(os.path.join(golden_dir, "roundrobin_gates.txt")) as fh:
        want = np.array([float(l) for l in fh if l.strip() and not l.startswith("#")])
    cfg = synth.CONFIGS["balanced"].with_(T=64)
    _, gate, _ = moe.route_topk(synth.gen_logits(cfg), cfg.k)
    assert np.allclose(gate, want[None, :], atol=5e-7)


def brute_force_metadata(idx, E):
    lists = {e: [] for e in range(E)}
    for t in range(idx.shape[0]):              # tokens in ascending order
        for j in range(idx.shape[1]):
            lists[int(idx[t, j])].append((t, j))
    dest = np.full(idx.shape, -1)
    row_token, r = [], 0
    for e in range(E):
        for t, j in lists[e]:
            dest[t, j] = r
            row_token.append(t)
            r += 1
    return [len(lists[e]) for e in range(E)], dest, row_token


@pytest.mark.parametrize("T,E,k,seed", [(1, 1, 1, 0), (7, 3, 2, 1), (64, 8, 2, 2), (100, 16, 4, 3), (33, 5, 5, 4)])
def test_metadata_matches_dict_of_lists(T, E, k, seed):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E))
    logits[:, E // 2] -= 50.0 if E > k else 0.0    # an expert that is (nearly) never chosen
    idx, _, _ = moe.route_topk(logits, k)
    counts, off, dest, row_token, offp = moe.route_metadata(idx, E, pad=32)
    bc, bdest, brt = brute_force_metadata(idx, E)
    assert counts.tolist() == bc and np.array_equal(dest, bdest) and row_token.tolist() == brt
    assert counts.sum() == T * k and off[0] == 0 and off[E] == T * k
    assert np.array_equal(np.sort(dest.ravel()), np.arange(T * k))           # bijection
    assert np.array_equal(row_token[dest], np.tile(np.arange(T)[:, None], (1, k)))
    for e in range(E):
        seg = row_token[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert offp[e + 1] - offp[e] == -(-counts[e] // 32) * 32


def test_roundrobin_counts_are_exact():
    cfg = synth.CONFIGS["balanced"]
    idx, _, _ = moe.route_topk(synth.gen_logits(cfg), cfg.k)
    counts, *_ = moe.route_metadata(idx, cfg.E)
    assert np.all(counts == cfg.T * cfg.k // cfg.E) and counts[0] == 512


def test_zipf_routing_is_skewed():
    cfg = synth.CONFIGS["skewed"]
    idx, _, _ = moe.route_topk(synth.gen_logits(cfg), cfg.k)
    counts, *_ = moe.route_metadata(idx, cfg.E)
    assert counts[0] == cfg.T                       # the hottest expert takes every token
    assert (counts == 0).sum() > 50                 # many experts get nothing
    assert counts.max() / counts.sum() > 0.10


def test_metadata_invariants_on_generated_ties():
    """Hypothesis-generated logits drawn from a few values (many exact ties): the selection keeps
    the lower expert id on ties, dest is a bijection onto 0..T*k-1, rows run expert-major and
    token-ascending, and counts sum to T*k."""
    from hypothesis import given, settings, strategies as st

    @settings(max_examples=60, deadline=None)
    @given(T=st.integers(1, 24), E=st.integers(1, 10), data=st.data())
    def check(T, E, data):
        k = data.draw(st.integers(1, E))
        vals = data.draw(st.lists(st.sampled_from([-1.0, 0.0, 0.5, 2.0]), min_size=T * E, max_size=T * E))
        logits = np.array(vals).reshape(T, E)
        idx, gate, _ = moe.route_topk(logits, k)
        for t in range(T):
            chosen = list(idx[t])
            # descending logits, ties to the lower id: exactly the first k of a stable sort
            order = sorted(range(E), key=lambda e: (-logits[t, e], e))
            assert chosen == order[:k]
        assert np.allclose(gate.sum(axis=1), 1.0)
        counts, off, dest, row_token, _ = moe.route_metadata(idx, E)
        assert counts.sum() == T * k and off[-1] == T * k
        assert sorted(dest.ravel().tolist()) == list(range(T * k))
        for t in range(T):
            for j in range(k):
                r = dest[t, j]
                assert row_token[r] == t and off[idx[t, j]] <= r < off[idx[t, j] + 1]
        for e in range(E):
            toks = row_token[off[e]:off[e + 1]]
            assert list(toks) == sorted(toks)

    check()
