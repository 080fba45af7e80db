"""The HBM streaming probe (attn_hbm_read_probe) reads every 16-byte word of
its buffer exactly once: the XOR of the per-wave results equals the XOR of
all words, for grids that divide the buffer unevenly (tail words)."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_03_amd as pa

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("workgroups", [0, 7, 1000])
def test_probe_reads_every_word_once(workgroups):
    g = torch.Generator(device=DEV)
    g.manual_seed(1200 + workgroups)
    n16 = (1 << 20) * 3 + 5                              # not a multiple of any grid here
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (n16 * 4,), generator=g, dtype=torch.int32, device=DEV)
    wg = workgroups or torch.cuda.get_device_properties(DEV).multi_processor_count
    sink = torch.zeros(wg * 16, dtype=torch.int32, device=DEV)
    pa.attn_hbm_read_probe(buf, sink, workgroups)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().reshape(-1, 4), axis=0)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().reshape(-1, 4), axis=0)
    assert (got == want).all()
