"""The read-only streaming kernel the benchmark measures the read ceiling with:
its per-workgroup checksums cover every word of the buffer exactly once."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

sd = pytest.importorskip("kv_cache_activation_amd")
from gpu_helpers import DEV  # noqa: E402


@pytest.mark.parametrize("nbytes", [8192, 8192 * 7, 1 << 22, (1 << 24) + 8192 * 3])
def test_stream_read_checksum_covers_every_word_once(nbytes):
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    out = torch.full((sd.SD_STREAM_BLOCKS,), -1, dtype=torch.int32, device=DEV)
    sd.sd_stream_read(buf, nbytes, out)
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
