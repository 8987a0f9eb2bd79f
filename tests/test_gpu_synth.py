"""The GPU twin of the seeded generator writes exactly the host generator's
bf16 tokens (same counter-based draws)."""
import numpy as np
import pytest
import torch

from synth import gen
from synth import gpu as synth_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("which,src,pos0,n", [("k", 0, 0, 1000), ("v", 3, 99_000, 517),
                                              ("k", gen.SHARED_SRC, 64, 300)])
def test_gpu_generator_is_bit_identical(which, src, pos0, n):
    hkv = 3
    ks, vs = gen.outlier_scales(5, hkv)
    scale = ks if which == "k" else vs
    buf = torch.zeros((n, hkv, 128), dtype=torch.int16, device="cuda")
    synth_gpu.fill_kv(buf, n, hkv, hkv * 128, 128, 5, which, src, pos0,
                      torch.from_numpy(scale).cuda(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = buf.cpu().numpy().view(np.uint16)
    for j in range(hkv):
        ref = gen.kv_tokens_bf16(5, which, src, j, pos0, n, scale[j])
        assert np.array_equal(got[:, j], ref)
