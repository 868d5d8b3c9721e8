"""Pins of the prefill oracle (``oracle.prefill_ref``).

Causal attention of a chunk reduces, row by row, to single-query attention
over the context up to that row's position: each row is checked against the
pinned decode oracle and against the scalar-loop brute force on such
truncated contexts.  Closed forms (two keys; a zero query averages the
visible values; the first prompt token returns its own value row) and the
causal invariance (rows never see later positions) cover what a reduction
could share with the code under test.
"""

import math

import numpy as np
import pytest

from oracle import decode_bruteforce, decode_ref, prefill_ref


def problem(seed, lens, chunks, hq=4, hkv=2, d=8, bs=4, spare=3):
    """Random caches, shuffled block tables, packed queries."""
    rng = np.random.default_rng(seed)
    need = [-(-L // bs) for L in lens]
    nb = sum(need) + spare
    perm = rng.permutation(nb)
    m = max(need)
    tables = np.full((len(lens), m), -1, dtype=np.int32)
    used = 0
    for s, k in enumerate(need):
        tables[s, :k] = perm[used:used + k]
        used += k
    kc = rng.standard_normal((nb, bs, hkv, d)).astype(np.float16)
    vc = rng.standard_normal((nb, bs, hkv, d)).astype(np.float16)
    starts = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = rng.standard_normal((int(starts[-1]), hq, d)).astype(np.float16)
    return q, kc, vc, tables, np.asarray(lens, dtype=np.int32), starts


def rows(starts, lens):
    """(row, sequence, position) of every packed query row."""
    for s in range(len(lens)):
        n = int(starts[s + 1] - starts[s])
        for j in range(n):
            yield int(starts[s]) + j, s, int(lens[s]) - n + j


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_each_row_is_decode_over_its_prefix(seed):
    lens, chunks = [9, 1, 17, 6], [4, 1, 17, 0]
    q, kc, vc, tables, L, starts = problem(seed, lens, chunks)
    out = prefill_ref(q, kc, vc, tables, L, starts, 0.37)
    for t, s, pos in rows(starts, L):
        ref = decode_ref(q[t:t + 1], kc, vc, tables[s:s + 1], [pos + 1], 0.37)
        np.testing.assert_allclose(out[t], ref[0], rtol=0, atol=1e-12)


def test_rows_match_scalar_bruteforce():
    lens, chunks = [7, 5], [3, 5]
    q, kc, vc, tables, L, starts = problem(5, lens, chunks, hq=6, hkv=3, d=4, bs=2)
    out = prefill_ref(q, kc, vc, tables, L, starts, 0.5)
    for t, s, pos in rows(starts, L):
        bf = decode_bruteforce(q[t:t + 1], kc, vc, tables[s:s + 1], [pos + 1], 0.5)
        np.testing.assert_allclose(out[t], np.asarray(bf[0]), rtol=0, atol=1e-12)


def test_two_keys_closed_form():
    # one head, D = 2, keys e0 and e1, values (1, 0) and (0, 1); the query
    # row at position 1 sees both: weights softmax(scale * q)
    kc = np.zeros((1, 2, 1, 2), dtype=np.float16)
    kc[0, 0, 0] = [1, 0]
    kc[0, 1, 0] = [0, 1]
    vc = kc.copy()
    q = np.array([[[1.5, -0.25]], [[0.75, 2.0]]], dtype=np.float16)
    out = prefill_ref(q, kc, vc, np.array([[0]]), [2], [0, 2], 1.0)
    np.testing.assert_allclose(out[0, 0], [1.0, 0.0], atol=0)       # position 0: only key 0
    w = 1.0 / (1.0 + math.exp(2.0 - 0.75))
    np.testing.assert_allclose(out[1, 0], [w, 1.0 - w], rtol=1e-14)


def test_zero_query_averages_visible_values():
    lens, chunks = [11, 8], [5, 8]
    q, kc, vc, tables, L, starts = problem(7, lens, chunks)
    q[:] = 0
    out = prefill_ref(q, kc, vc, tables, L, starts, 0.9)
    bs = kc.shape[1]
    for t, s, pos in rows(starts, L):
        vis = np.array([vc[tables[s][p // bs], p % bs] for p in range(pos + 1)], dtype=np.float64)
        for h in range(q.shape[1]):
            np.testing.assert_allclose(out[t, h], vis[:, h // 2].mean(0), rtol=0, atol=1e-12)


def test_first_prompt_token_returns_its_value_row():
    lens, chunks = [6], [6]                      # the whole prompt is the chunk
    q, kc, vc, tables, L, starts = problem(3, lens, chunks)
    out = prefill_ref(q, kc, vc, tables, L, starts, 1.3)
    v0 = vc[tables[0][0], 0].astype(np.float64)
    for h in range(q.shape[1]):
        assert np.array_equal(out[0, h], v0[h // 2])


def test_rows_never_see_later_positions():
    lens, chunks = [13], [9]
    q, kc, vc, tables, L, starts = problem(9, lens, chunks)
    base = prefill_ref(q, kc, vc, tables, L, starts, 0.6)
    bs = kc.shape[1]
    cut = 8                                      # perturb position 8 only
    k2, v2 = kc.copy(), vc.copy()
    k2[tables[0][cut // bs], cut % bs] += np.float16(1.0)
    v2[tables[0][cut // bs], cut % bs] -= np.float16(2.0)
    pert = prefill_ref(q, k2, v2, tables, L, starts, 0.6)
    for t, s, pos in rows(starts, L):
        if pos < cut:
            assert np.array_equal(pert[t], base[t])
        else:
            assert not np.allclose(pert[t], base[t])


def test_bad_arguments_raise():
    q, kc, vc, tables, L, starts = problem(1, [4], [4])
    with pytest.raises(ValueError):
        prefill_ref(q, kc, vc, tables, [3], starts, 1.0)          # chunk longer than context
    with pytest.raises(ValueError):
        prefill_ref(q, kc, vc, tables, L, [1, 4], 1.0)             # does not start at 0
    with pytest.raises(ValueError):
        prefill_ref(q, kc, vc, tables, L, [0, 3], 1.0)             # does not end at T
