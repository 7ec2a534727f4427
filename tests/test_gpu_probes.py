"""GPU checks of the measurement probes (not part of the attention path).

- vsa_hbm_probe: the copy stream leaves dst equal to src byte for byte
  (sizes that are and are not a multiple of one round of the grid), the write
  stream writes word i as (i, i >> 32, 0, 0), the read stream leaves its
  source unchanged.
- vsa_mfma_probe: the checksums are finite and every workgroup reports a
  positive cycle and tick count.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, (1 << 20) + 48, 16384 * 256 * 64 + 32])
def test_hbm_probe_streams(nbytes):
    import block_sparse_video_cube_amd as vsa

    g = torch.Generator().manual_seed(nbytes % 1000)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).to("cuda:0")
    dst = torch.zeros_like(src)
    vsa.hbm_probe("copy", src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    keep = src.clone()
    vsa.hbm_probe("read", src, None)
    torch.cuda.synchronize()
    assert torch.equal(src, keep)
    vsa.hbm_probe("write", None, dst)
    torch.cuda.synchronize()
    words = dst.cpu().numpy().view(np.uint32).reshape(-1, 4)
    i = np.arange(words.shape[0], dtype=np.uint64)
    assert np.array_equal(words[:, 0], (i & 0xFFFFFFFF).astype(np.uint32))
    assert np.array_equal(words[:, 1], (i >> 32).astype(np.uint32))
    assert not words[:, 2:].any()


def test_mfma_probe_reports():
    import block_sparse_video_cube_amd as vsa

    sink, clk = vsa.mfma_probe(64, 10)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    c = clk.cpu().numpy()
    assert (c[:, 0] > 0).all() and (c[:, 1] > 0).all()
