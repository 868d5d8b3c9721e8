"""The measurement probes.  The streaming-read probe reads every 16-byte word
of its buffer: a lane's XOR of the words it read reaches the sink constant
only when the one planted word is read (an odd number of times) by that lane.
The matrix-core probe runs every product it counts: with operand 1 each of
its accumulators ends at exactly 16 per iteration (the sink stays 0), with
operand 2 at four times that (the sink is set)."""

import numpy as np
import pytest
import torch

from paged_kv_cache_382_amd import probe as pa_probe
from tests.gpu_problems import DEV, say

pytestmark = pytest.mark.gpu

MAGIC = np.uint32(0x9E3779B9).view(np.int32)


def probe(nbytes, plant_word=None):
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    if plant_word is not None:
        buf[plant_word] = int(MAGIC)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    say(f"read probe: {nbytes} bytes, planted word {plant_word}")
    pa_probe.pa_read_probe(buf, sink)
    torch.cuda.synchronize()
    return int(sink.item())


def test_zeros_leave_the_sink_untouched():
    assert probe((1 << 20) + 48) == 0


@pytest.mark.parametrize("nbytes,where", [
    ((1 << 20) + 48, "first"),
    ((1 << 20) + 48, "last"),
    (16, "last"),
    ((256 << 20) + 16, "random"),
    ((256 << 20) + 16, "last"),
])
def test_planted_word_is_read(nbytes, where):
    words = nbytes // 4
    w = {"first": 0, "last": words - 1,
         "random": int(np.random.default_rng(7).integers(0, words))}[where]
    assert probe(nbytes, w) == int(MAGIC)


@pytest.mark.parametrize("workgroups,iters", [(1, 1), (3, 17), (512, 256)])
def test_mfma_probe_runs_every_product(workgroups, iters):
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    say(f"mfma probe: {workgroups} workgroups, {iters} iterations, operand 1")
    flops = pa_probe.pa_mfma_probe(sink, workgroups, iters, 1.0)
    torch.cuda.synchronize()
    assert flops == workgroups * iters * 8 * 4 * 32768
    assert int(sink.item()) == 0
    say(f"mfma probe: {workgroups} workgroups, {iters} iterations, operand 2")
    pa_probe.pa_mfma_probe(sink, workgroups, iters, 2.0)
    torch.cuda.synchronize()
    assert int(sink.item()) == 1
