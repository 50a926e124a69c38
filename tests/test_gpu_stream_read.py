"""The streaming-read measurement helper reads every word exactly once: its wrapping
32-bit sum equals the sum computed by torch, for sizes that split evenly over the work
groups and for ragged ones."""
import pytest
import torch

import draft_kv_attention_amd as M

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words,wgs", [(4 * 1000003, 0), (16 << 20, 2048), (4 * 37, 7), (4, 1), (4 * 5000, 700)])
def test_stream_read_sum_matches_torch(n_words, wgs):
    g = torch.Generator(device="cuda")
    g.manual_seed(n_words)
    buf = torch.randint(-(1 << 31), (1 << 31) - 1, (n_words,), dtype=torch.int32, device="cuda", generator=g)
    sums = torch.zeros(M.STREAM_SUMS, dtype=torch.int32, device="cuda")
    M.stream_read(buf, sums, work_groups=wgs)
    expect = int(buf.to(torch.int64).sum().item()) % (1 << 32)
    assert int(sums.to(torch.int64).sum().item()) % (1 << 32) == expect
