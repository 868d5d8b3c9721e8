"""The binding checks every size the kernels take from its tensors before any
launch (the C ABI receives raw pointers): mismatched shapes raise ValueError
on the host.  CPU tensors suffice, since the checks run before any device
access."""

import pytest
import torch

import paged_kv_cache_382_amd as pa

B, HQ, HKV, D, NB, BS, M = 3, 8, 2, 64, 16, 16, 4


def tensors(**over):
    t = {
        "q": torch.zeros((B, HQ, D), dtype=torch.float16),
        "k_cache": torch.zeros((NB, BS, HKV, D), dtype=torch.float16),
        "v_cache": torch.zeros((NB, BS, HKV, D), dtype=torch.float16),
        "block_tables": torch.zeros((B, M), dtype=torch.int32),
        "context_lens": torch.ones(B, dtype=torch.int32),
    }
    t.update(over)
    return t


def call_decode(out=None, **over):
    t = tensors(**over)
    return pa.pa_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"], t["context_lens"],
                        0.125, out=out)


@pytest.mark.parametrize("over,out", [
    ({"q": torch.zeros((B, HQ, 2 * D), dtype=torch.float16)}, None),       # head dim != cache's
    ({"q": torch.zeros((B, HQ), dtype=torch.float16)}, None),              # not [B, Hq, D]
    ({"q": torch.zeros((B, 7, D), dtype=torch.float16)}, None),            # Hq not a multiple of Hkv
    ({"v_cache": torch.zeros((NB // 2, BS, HKV, D), dtype=torch.float16)}, None),
    ({"block_tables": torch.zeros((B + 1, M), dtype=torch.int32)}, None),
    ({"block_tables": torch.zeros(B * M, dtype=torch.int32)}, None),
    ({"context_lens": torch.ones(B + 1, dtype=torch.int32)}, None),
    ({}, torch.zeros((B, HQ, D // 2), dtype=torch.float16)),                # out shape
    ({}, torch.zeros((B, HQ, D), dtype=torch.float32)),                     # out dtype
])
def test_decode_rejects_mismatched_tensors_before_launch(over, out):
    with pytest.raises(ValueError):
        call_decode(out=out, **over)


def test_decode_with_matching_shapes_reaches_the_device_check():
    # consistent shapes pass the size checks; the CPU tensors then fail the
    # device check, still before any launch
    with pytest.raises(ValueError, match="device tensor"):
        call_decode()


@pytest.mark.parametrize("bad", ["q", "out", "v_cache", "tables"])
def test_prefill_rejects_mismatched_tensors_before_launch(bad):
    T = 5
    q = torch.zeros((T, HQ, D), dtype=torch.float16)
    kc = torch.zeros((NB, BS, HKV, D), dtype=torch.float16)
    vc = kc.clone()
    tables = torch.zeros((B, M), dtype=torch.int32)
    lens = torch.full((B,), 2, dtype=torch.int32)
    qs = torch.tensor([0, 2, 4, 5], dtype=torch.int32)
    out = None
    if bad == "q":
        q = torch.zeros((T, HQ, D + 8), dtype=torch.float16)
    elif bad == "out":
        out = torch.zeros((T + 1, HQ, D), dtype=torch.float16)
    elif bad == "v_cache":
        vc = torch.zeros((NB, BS, HKV, D // 2), dtype=torch.float16)
    else:
        tables = torch.zeros(B * M, dtype=torch.int32)
    with pytest.raises(ValueError):
        pa.pa_prefill(q, kc, vc, tables, lens, qs, 0.125, out=out, max_query_len=2)
