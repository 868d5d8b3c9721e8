"""pa_decode_noalloc (partial results in the library's own device array, no
allocation) against pa_decode with a caller workspace: bitwise equal outputs
on two calls in a row, the second with a smaller input, and both within the
bar of the fp64 oracle."""

import numpy as np
import pytest
import torch

import paged_kv_cache_382_amd as pa
import workloads as W
from tests.gpu_problems import DEV, build, check_close, oracle_caches, oracle_out, run_step, say

pytestmark = pytest.mark.gpu

BIG = W.shrink(W.MIX, name="noalloc_big", num_seqs=6, num_blocks=1024, max_blocks_per_seq=256,
               num_q_heads=16, num_kv_heads=4)
BIG_LENS = [1, 17, 200, 1000, 2049, 3333]
SMALL = W.shrink(W.MIX, name="noalloc_small", num_seqs=3, num_blocks=128, max_blocks_per_seq=32,
                 num_q_heads=8, num_kv_heads=2, head_dim=64)
SMALL_LENS = [5, 300, 77]


def problem(wl, lens):
    return build(wl, lambda a: W._plain_plan(a, wl, lens))


def both(p, n_split):
    wl = p["wl"]
    out_ws = run_step(p, num_splits=n_split)          # copies, store, decode with a workspace
    out_na = torch.full_like(out_ws, float("nan"))
    say(f"{wl.name}: pa_decode_noalloc W={n_split}")
    pa.pa_decode_noalloc(p["q"], p["kc"], p["vc"], p["tables"], p["lens"], wl.scale, out_na,
                         max_context_len=p["max_ctx"], num_splits=n_split)
    torch.cuda.synchronize()
    return out_ws, out_na


@pytest.mark.parametrize("n_split", [0, 37, -1])
def test_noalloc_equals_workspace_call_twice_then_smaller(n_split):
    p = problem(BIG, BIG_LENS)
    out_ws, out_na = both(p, n_split)
    assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16))
    kc, vc = oracle_caches(p)
    check_close(out_na, oracle_out(p, kc, vc), f"noalloc big W={n_split}")
    # a second call right after, on a smaller problem: the scratch keeps the
    # first call's contents, which must not leak into the result
    q = problem(SMALL, SMALL_LENS)
    out_ws2, out_na2 = both(q, n_split)
    assert torch.equal(out_na2.view(torch.int16), out_ws2.view(torch.int16))
    kc2, vc2 = oracle_caches(q)
    check_close(out_na2, oracle_out(q, kc2, vc2), f"noalloc small W={n_split}")


def test_noalloc_rejects_a_call_beyond_the_scratch_without_launching():
    p = problem(SMALL, SMALL_LENS)
    out = torch.full_like(p["q"], 7.0)
    with pytest.raises(pa.PaError) as e:
        # 100000 splits need (100000 + pairs) x 4 x 66 x 4 bytes > 8 MiB
        pa.pa_decode_noalloc(p["q"], p["kc"], p["vc"], p["tables"], p["lens"], SMALL.scale, out,
                             num_splits=100000)
    assert e.value.code == "WORKSPACE"
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
