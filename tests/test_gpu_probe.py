"""GPU tests of the read-bandwidth probe (w4a16_read_probe): every 32-bit word
of the buffer is read exactly once, for sizes from one 16-byte word (fewer
words than waves) to a layer set's packed weights, so the rate it reports is
the rate of reading exactly those bytes."""
import numpy as np
import pytest

import w4a16_weight_only_gemm_amd as w4

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 1024 + 16, 64 * 1024 * 1024 + 4096 + 48, 173_187_072])
def test_probe_reads_every_word_once(nbytes):
    import torch
    rng = np.random.default_rng(nbytes % 1000)
    words = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    expect = int(words.astype(np.uint64).sum() % 2**32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    sink = torch.zeros(w4.READ_PROBE_SINK_BYTES // 4, dtype=torch.int32, device="cuda")
    w4.w4a16_read_probe(buf, nbytes, sink)
    torch.cuda.synchronize()
    got = int(sink.cpu().numpy().view(np.uint32).astype(np.uint64).sum() % 2**32)
    assert got == expect


def test_probe_is_repeatable():
    import torch
    words = np.arange(1 << 20, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    sums = []
    for _ in range(3):
        sink = torch.zeros(w4.READ_PROBE_SINK_BYTES // 4, dtype=torch.int32, device="cuda")
        w4.w4a16_read_probe(buf, words.nbytes, sink)
        torch.cuda.synchronize()
        sums.append(sink.cpu().numpy().copy())
    assert all(np.array_equal(sums[0], s) for s in sums[1:])
    assert int(sums[0].view(np.uint32).astype(np.uint64).sum() % 2**32) == int(words.astype(np.uint64).sum() % 2**32)
