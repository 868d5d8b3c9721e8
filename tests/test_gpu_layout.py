"""Head-major caches ([num_blocks][num_kv_heads][block_size][head_dim]) on the GPU.

The layout only moves rows inside a block, and every kernel does the same
arithmetic in the same order either way, so decode and prefill over a
head-major copy of a cache must equal the slot-major results bit for bit (for
decode in the same order: given the plain order's workspace, slot-major runs
the plain order that head-major runs; with its own, larger workspace it may
run the head-group order, which is checked against the oracle); the
store must put every head's piece where the oracle's head-major store does; and
the outputs must be within the parity bar of the oracle run on the head-major
arrays themselves.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_382_amd as pa
import workloads as W
from oracle import decode_ref, prefill_ref, store_ref
from tests.gpu_problems import DEV, check_close, host_u16, say

pytestmark = pytest.mark.gpu


def head_major(c):
    return c.transpose(1, 2).contiguous()


def problem(seed, nb, bs, hkv, d, lens):
    """Slot-major caches (NaN sentinel outside the context rows), tables over a
    seeded permutation of the pool, ragged lengths."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(nb)
    m = max(-(-L // bs) for L in lens)
    tables = np.full((len(lens), m), -1, dtype=np.int32)
    k = 0
    for i, L in enumerate(lens):
        n = -(-L // bs)
        tables[i, :n] = order[k:k + n]
        k += n
    assert k <= nb
    shape = (nb, bs, hkv, d)
    kc = W.nan_sentinel_fp16(shape, DEV)
    vc = W.nan_sentinel_fp16(shape, DEV)
    vals_k = W.normal_fp16(shape, seed * 7 + 1, DEV)
    vals_v = W.normal_fp16(shape, seed * 7 + 2, DEV)
    used = np.zeros(nb * bs, dtype=bool)
    for i, L in enumerate(lens):
        blocks = tables[i, :-(-L // bs)].astype(np.int64)
        used[(blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)[:L]] = True
    mask = torch.from_numpy(used).to(DEV)
    kc.view(nb * bs, hkv, d)[mask] = vals_k.view(nb * bs, hkv, d)[mask]
    vc.view(nb * bs, hkv, d)[mask] = vals_v.view(nb * bs, hkv, d)[mask]
    return kc, vc, tables, list(lens)


def test_head_major_store_matches_oracle():
    nb, bs, hkv, d = 40, 16, 4, 128
    shape = (nb, hkv, bs, d)
    kc = W.nan_sentinel_fp16(shape, DEV)
    vc = W.nan_sentinel_fp16(shape, DEV)
    ref_k, ref_v = host_u16(kc), host_u16(vc)
    rng = np.random.default_rng(3)
    slots = [int(s) for s in rng.permutation(nb * bs)[:300]] + [-1, -5]
    k = W.normal_fp16((len(slots), hkv, d), 31, DEV)
    v = W.normal_fp16((len(slots), hkv, d), 32, DEV)
    say("head-major store")
    pa.pa_store_kvcache(k, v, torch.tensor(slots, dtype=torch.int32, device=DEV), kc, vc, layout="head")
    torch.cuda.synchronize()
    ref_k, ref_v = store_ref(host_u16(k), host_u16(v), slots, ref_k, ref_v, layout="head")
    assert np.array_equal(host_u16(kc), ref_k)
    assert np.array_equal(host_u16(vc), ref_v)


# (seed, block size, KV heads, head dim, group, lengths): groups of 1 and 2 on
# the vector kernel (block 8: the ragged chunk on its separate masked path),
# the others on the matrix-core kernel (block 8: two blocks a chunk).
DECODE = [
    (1, 16, 4, 128, 4, [1, 17, 200, 777, 1000, 33]),
    (2, 8, 2, 128, 4, [5, 300, 64, 129]),
    (3, 32, 2, 64, 1, [31, 500, 1, 96]),
    (4, 16, 2, 128, 8, [400, 15, 250]),
    (5, 64, 8, 128, 1, [2048, 2048, 1999, 70]),
    (6, 8, 3, 64, 2, [9, 1000, 255, 8]),
    (7, 8, 4, 64, 6, [16, 7, 333, 1024]),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: f"bs{c[1]}_hkv{c[2]}_d{c[3]}_g{c[4]}")
@pytest.mark.parametrize("num_splits", [0, 7])
def test_head_major_decode_equals_slot_major_and_oracle(case, num_splits):
    seed, bs, hkv, d, g, lens = case
    nb = sum(-(-L // bs) for L in lens) + 8
    kc, vc, tables, lens = problem(seed, nb, bs, hkv, d, lens)
    q = W.normal_fp16((len(lens), hkv * g, d), seed + 50, DEV)
    t = torch.from_numpy(tables).to(DEV)
    ll = torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    say(f"decode layouts bs {bs} hkv {hkv} d {d} g {g} splits {num_splits}")
    kh, vh = head_major(kc), head_major(vc)
    # the plain order's workspace (head-major never takes the head-group order)
    plain = pa.decode_workspace(pa.cache_desc(kh, "head"), len(lens), hkv * g, num_splits, DEV)
    out_s = pa.pa_decode(q, kc, vc, t, ll, scale, max_context_len=max(lens), num_splits=num_splits,
                         workspace=plain)
    out_sd = pa.pa_decode(q, kc, vc, t, ll, scale, max_context_len=max(lens), num_splits=num_splits)
    out_h = pa.pa_decode(q, kh, vh, t, ll, scale, max_context_len=max(lens), num_splits=num_splits,
                         layout="head")
    torch.cuda.synchronize()
    assert torch.equal(out_s.view(torch.int16), out_h.view(torch.int16))
    ref = decode_ref(host_u16(q).view(np.float16), host_u16(kh).view(np.float16),
                     host_u16(vh).view(np.float16), tables, lens, scale, layout="head")
    check_close(out_h, ref, "head-major decode")
    check_close(out_sd, ref, "slot-major decode, default workspace")


@pytest.mark.parametrize("g,bs,d", [(1, 16, 128), (4, 16, 128), (2, 8, 128), (8, 32, 64), (3, 64, 64)])
def test_head_major_prefill_equals_slot_major_and_oracle(g, bs, d):
    hkv = 2
    lens = [300, 77, 129]
    chunks = [100, 77, 33]
    nb = sum(-(-L // bs) for L in lens) + 8
    kc, vc, tables, lens = problem(10 + g + d, nb, bs, hkv, d, lens)
    starts = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = W.normal_fp16((int(starts[-1]), hkv * g, d), 70 + g, DEV)
    t = torch.from_numpy(tables).to(DEV)
    ll = torch.tensor(lens, dtype=torch.int32, device=DEV)
    qs = torch.from_numpy(starts).to(DEV)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    say(f"prefill layouts g {g} bs {bs} d {d}")
    out_s = pa.pa_prefill(q, kc, vc, t, ll, qs, scale, max_query_len=max(chunks))
    kh, vh = head_major(kc), head_major(vc)
    out_h = pa.pa_prefill(q, kh, vh, t, ll, qs, scale, max_query_len=max(chunks), layout="head")
    torch.cuda.synchronize()
    assert torch.equal(out_s.view(torch.int16), out_h.view(torch.int16))
    ref = prefill_ref(host_u16(q).view(np.float16), host_u16(kh).view(np.float16),
                      host_u16(vh).view(np.float16), tables, lens, starts, scale, layout="head")
    check_close(out_h, ref, "head-major prefill")
