"""The streaming-read probe behind the measured read ceiling reads every
32-bit word of its buffer exactly once: the XOR of the per-wave folds it
leaves in the sink equals numpy's fold of the same bytes (a word skipped, or read twice,
changes it). Sizes: the ceiling's cold 7B-shape sizes, a ragged count of
16-byte words that leaves a tail past the four-load loop, and tiny buffers."""
import numpy as np
import pytest

from gpu_common import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,groups", [(16, 1), (16 * 4099, 7), (9_437_184, 2048), (25_362_432, 2048),
                                           ((1 << 26) + 48, 4096)])
def test_read_probe_reads_every_word_once(nbytes, groups):
    import torch

    import q4_weight_gemv_amd as q4

    host = np.random.default_rng(nbytes % 997 + groups).integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).cuda()
    sink = torch.zeros(4 * groups, dtype=torch.int32, device="cuda")
    say(f"read probe {nbytes} B, {groups} groups")
    q4.q4_read_probe(buf, sink, groups=groups)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)
