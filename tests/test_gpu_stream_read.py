"""The streaming-read reference kernel reads every 16-byte word of its range exactly
once: the XOR of the per-workgroup folds equals the XOR of all words, for both
layouts and for ranges that do not divide evenly among the workgroups."""
import numpy as np
import pytest
import torch

import block_float_quantized_mxq_amd as mxq
from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 19496960, 139264000 + 16 * 7])
def test_every_word_read_once(layout, nbytes):
    rng = np.random.default_rng(nbytes + layout)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    data = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda:0")
    say("stream read", layout, nbytes)
    mxq.stream_read(data, sink, layout=layout)
    folds = sink.cpu().numpy().view(np.uint32)
    assert np.bitwise_xor.reduce(folds) == np.bitwise_xor.reduce(words)
