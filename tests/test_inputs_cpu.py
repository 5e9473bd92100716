"""The input generators' MXFP4 storage against the oracle's decoding (CPU).

inputs.mx4_tile (which lays out the GPU path's weights) and the oracle's
mx4_untile are written separately; this checks that they are inverse orders,
and that the quantiser's stored values are the drawn weights to within the
format's rounding."""
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from routed_expert_ffn_flint_amd import inputs  # noqa: E402
from oracle import oracle as orc  # noqa: E402


def test_mx4_tile_is_the_oracle_untile_inverse():
    g = torch.Generator().manual_seed(7)
    codes = torch.randint(0, 256, (3, 48, 64), dtype=torch.uint8, generator=g)  # 3 matrices of 48 x 128
    scales = torch.randint(0, 255, (3, 48, 4), dtype=torch.uint8, generator=g)
    ct, st = inputs.mx4_tile(codes, scales)
    assert tuple(ct.shape) == (3, 3, 4, 16, 16) and tuple(st.shape) == (3, 3, 4, 16)
    c, s = orc.mx4_untile(ct.numpy(), st.numpy())
    np.testing.assert_array_equal(c, codes.numpy())
    np.testing.assert_array_equal(s, scales.numpy())


def test_mx4_quantize_rounds_to_nearest_code():
    g = torch.Generator().manual_seed(3)
    w = torch.randn(32, 256, generator=g) * 0.02
    w[0, :32] = 0.0  # an all-zero block
    codes, scales = inputs.mx4_quantize(w)
    deq = orc.mx4_dequant(codes.numpy(), scales.numpy())
    assert np.all(deq[0, :32] == 0.0)
    wb = w.numpy().reshape(32, 8, 32).astype(np.float64)
    db = deq.reshape(32, 8, 32).astype(np.float64)
    unit = np.exp2(scales.numpy().astype(np.float64) - 127)[..., None]  # the block's 2^X
    # every E2M1 magnitude step is at most 2 units, so rounding to nearest is off
    # by at most 1 unit up to the largest code (6 units); a block's largest
    # element lands in [4, 8) units, and beyond 6 units it saturates to 6
    bound = np.maximum(1.0, np.abs(wb) / unit - 6.0) * unit
    assert np.all(np.abs(wb - db) <= bound * (1.0 + 1e-12))
    assert np.all(np.abs(db) <= 6.0 * unit)
    amax = np.abs(wb).max(-1)
    nz = amax > 0
    assert np.all((amax[nz] / unit[..., 0][nz] >= 4.0) & (amax[nz] / unit[..., 0][nz] < 8.0))
