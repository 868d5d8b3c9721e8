"""The benchmark's traffic model against the pages' closed forms."""

import json
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_kv_bytes_per_request_is_about_1gb():
    g = golden("kv_bytes_per_request.json")
    n = bench.kv_bytes_per_request(g["layers"], g["hidden"], g["tokens"], g["bytes_per_element"])
    assert n == 1 << 30                                   # exactly 1 GiB
    assert abs(n - g["approx_bytes"]) / g["approx_bytes"] <= g["approx_rel_tolerance"]


def test_128k_context_table_entries():
    g = golden("blocks_128k.json")
    # one table entry (4 bytes) per block of the context
    lens = [g["context_tokens"]]
    kv = g["context_tokens"] * 1 * 128 * 2 * 2
    n = bench.decode_bytes(lens, 1, 1, 128, g["block_size"])
    assert n - kv - 2 * 128 * 2 - 4 == g["blocks"] * 4


@pytest.mark.parametrize("lens,hq,hkv,bs,expect", [
    ([2048] * 32, 32, 32, 16, 1_074_282_624),            # bs32 ctx2048 MHA
    ([131072] * 4, 32, 8, 16, 2_147_680_272),            # 4 x 128K GQA, block 16
    ([131072] * 4, 32, 8, 8, 2_147_811_344),             # block 8
    ([131072] * 4, 32, 8, 64, 2_147_581_968),            # block 64
])
def test_decode_bytes_worked_values(lens, hq, hkv, bs, expect):
    assert bench.decode_bytes(lens, hq, hkv, 128, bs) == expect


def test_table_overhead_below_one_percent():
    """Mapping-table memory stays under 1% of the KV cache it maps."""
    for hkv, bs in [(8, 8), (8, 16), (32, 16), (8, 64)]:
        per_block_kv = bs * hkv * 128 * 2 * 2
        assert 4 / per_block_kv < 0.01


def test_store_and_copy_bytes():
    assert bench.store_bytes(32, 32, 128) == 4 * 32 * 32 * 128 * 2 + 128
    assert bench.copy_bytes(1, 16, 8, 128) == 4 * 16 * 8 * 128 * 2


@pytest.mark.parametrize("lens,chunks", [([7], [7]), ([10, 3, 5], [4, 3, 0]), ([2048] * 2, [256] * 2)])
def test_prefill_flops_brute_force(lens, chunks):
    """Causal key counts by enumeration: row j of an n-row chunk at the end of
    an L-token context sees L - n + j + 1 keys; 4 flops a key, dim and head."""
    hq, d = 3, 8
    keys = sum(L - n + j + 1 for L, n in zip(lens, chunks) for j in range(n))
    assert bench.prefill_flops(lens, chunks, hq, d) == 4 * keys * hq * d


def test_prefill_flops_benchmarked_workload():
    # 32 chunks of 256 rows ending 2048-token prompts, 32 query heads, D = 128:
    # each chunk sees 256*1792 + 256*257/2 = 491,648 keys
    assert bench.prefill_flops([2048] * 32, [256] * 32, 32, 128) == 4 * 491_648 * 32 * 128 * 32
    assert bench.prefill_flops([2048] * 32, [256] * 32, 32, 128) == 257_765_146_624


def test_prefill_kv_bytes():
    # K and V rows of every context token once: 2048 tokens x 8 heads x 128 x 2 B x 2
    assert bench.prefill_kv_bytes([2048], 8, 128) == 2048 * 8 * 128 * 4


PROFILES = os.path.join(os.path.dirname(bench.__file__), "profiles")


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(PROFILES)
                                        if f.endswith("_counters.json") and not f.endswith("_lds_counters.json")))
def test_committed_counter_runs_reach_the_bench_line(name):
    """Every committed counter summary whose kernel source is unchanged is the
    traffic bench.py reports for its workload."""
    kind, wl = name[:-len("_counters.json")].split("_", 1)
    src = bench.DECODE_SRC if kind == "decode" else bench.PREFILL_SRC
    with open(os.path.join(os.path.dirname(bench.__file__), "profiles", name)) as f:
        rec = json.load(f)
    if rec[f"{kind}_source_sha256_16"] != bench.source_digest(src):
        pytest.skip(f"{kind} kernel changed since {name} was taken")
    wl_name = f"{kind}_{wl}" if kind == "prefill" else wl
    assert bench.counter_traffic(wl_name, kind) == rec["hbm_bytes_per_launch"]


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(PROFILES) if f.endswith("_lds_counters.json")))
def test_committed_lds_counter_runs_reach_the_bench_line(name):
    """The bank-conflict share bench.py reports is the committed pass's figure
    for the split kernel: conflict cycles over LDS-active cycles."""
    wl = name[len("decode_"):-len("_lds_counters.json")]
    with open(os.path.join(PROFILES, name)) as f:
        rec = json.load(f)
    if rec["decode_source_sha256_16"] != bench.source_digest(bench.DECODE_SRC):
        pytest.skip(f"decode kernel changed since {name} was taken")
    k = rec["per_kernel_mean_per_dispatch"][rec["dominant_kernel"]]
    assert rec["dominant_kernel"].startswith(("decode_split_kernel", "decode_mfma_kernel"))
    assert rec["lds_bank_conflict_share"] == pytest.approx(k["SQ_LDS_BANK_CONFLICT"] / k["SQ_LDS_IDX_ACTIVE"], abs=1e-5)
    assert bench.counter_lds_conflicts(wl) == rec["lds_bank_conflict_share"]
