"""The read probe (pgkq_stream_read): it must read every byte it is given, so
its XOR fold of the buffer's 32-bit words equals the fold computed on the host,
for sizes from one 16-byte row to several hundred MiB, including sizes that
leave a ragged last slice and a partial last iteration."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 16, 32768 * 4096 + 48, (300 << 20) + 16 * 7])
def test_stream_read_folds_every_word(nbytes):
    import compressed_cache_decode_pgkq_amd as api
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    seed = np.uint32(0x9E3779B9)
    out = torch.tensor([int(seed.view(np.int32))], dtype=torch.int32, device="cuda:0")
    api.pgkq_stream_read(src, out)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host) ^ seed
    assert np.uint32(out.cpu().numpy().view(np.uint32)[0]) == want
