"""GPU parity of the expert FFN GEMMs where one workgroup runs several tiles.

The large-tile GEMM keeps one workgroup per compute unit and walks the
tiles; the first K step of the next tile is loaded while the current tile
finishes, into the LDS stage the current tile's step nk-2 used (or the other
stage when a tile has a single K step).  These cases have more tiles than
compute units, ragged expert row counts (one expert empty), and 1, 2, 3, 44
and 48 K steps per tile (odd counts alternate the stage of each tile's first
step), and check the pre-activation, activation and output of every row
against the CPU oracle's expert FFN.  The forward Linears run row tiles of
up to 320 rows (five 32-row blocks per token-side wave, the fifth block's
accumulators in VGPRs); the last case puts expert row counts on both sides
of each step in the number of row tiles.

Bar: |g - o| <= 2e-2*|o| + 2e-2*rms(o) elementwise (bf16 storage)."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_39_amd import binding as B
from oracle import moe_oracle as O
from tests.gpu_util import close, experts, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _draw(g, shape, std):
    return (torch.randn(*shape, generator=g, device=DEV, dtype=torch.float32) * std).to(torch.bfloat16)


# (rows per expert, d, h, activation, capacity factor or None for no drop);
# h = 0 is a single Linear d -> d.  The capacity only sizes the workspace
# and picks the row tile height (the expert offsets are given).
BANDS = [1, 255, 256, 257, 288, 289, 320, 321, 511, 512, 513, 639, 640, 641, 960, 961, 0]
CASES = [
    ([2500, 0, 3100, 1200], 64, 3072, B.MOE_ACT_GELU, None),    # GEMM1: 1 K step, 336 tiles
    ([2500, 0, 3100, 1200], 192, 2816, B.MOE_ACT_GELU, None),   # GEMM1: 3 K steps, 308 tiles; GEMM2: 44
    ([2500, 0, 3100, 1200], 128, 4096, B.MOE_ACT_RELU, None),   # GEMM1: 2 K steps, 448 tiles
    ([40000, 0, 30000], 64, 0, B.MOE_ACT_NONE, None),           # one Linear, 1 K step, 275 tiles
    # expert row counts on both sides of each step in the number of row
    # tiles (R rows run in ceil(R / tile) row tiles of equal size, rounded up
    # to 32 rows), with 256-row tiles (no drop: the mean of 434 rows gives no
    # fewer tiles at 320) and with 320-row tiles (capacity 564: two tiles of
    # 320 rows against three of 256): one to five 32-row blocks per wave
    (BANDS, 128, 256, B.MOE_ACT_GELU, None),
    (BANDS, 128, 256, B.MOE_ACT_GELU, 1.3),
    (BANDS, 192, 0, B.MOE_ACT_NONE, 1.3),
    (BANDS, 128, 320, B.MOE_ACT_GELU, 1.3),   # 320-row tiles, a part-filled feature tile (N = 320)
    (BANDS, 64, 128, B.MOE_ACT_RELU, 1.3),    # 320-row tiles with 1 and 2 K steps
]


@pytest.mark.parametrize("rows,d,h,act,cf", CASES, ids=lambda v: str(v))
def test_expert_ffn_many_tiles_per_workgroup(rows, d, h, act, cf):
    g = torch.Generator(device=DEV)
    g.manual_seed(4242 + d + h)
    E, n = len(rows), sum(rows)
    hid = h if h else d
    x = _draw(g, (n, d), 1.0)
    w1 = _draw(g, (E, hid, d), 0.02)
    b1 = _draw(g, (E, hid), 0.02)
    w2 = _draw(g, (E, d, h), 0.02) if h else None
    b2 = _draw(g, (E, d), 0.02) if h else None
    off = torch.tensor(np.concatenate([[0], np.cumsum(rows)]), dtype=torch.int32, device=DEV)
    cfg = B.make_config(n, d, E, 1, 1.0 if cf is None else cf, 4, cf is not None, h, act, B.MOE_BF16,
                        save_preact=True)
    assert B.moe_max_rows(cfg) >= n
    ws = torch.empty(B.moe_workspace_size(cfg), dtype=torch.uint8, device=DEV)
    a = torch.full((n, hid), 3.0, dtype=torch.bfloat16, device=DEV) if h else None
    hd = torch.full((n, hid), 3.0, dtype=torch.bfloat16, device=DEV) if h else None
    y = torch.full((n, d), 3.0, dtype=torch.bfloat16, device=DEV)
    B.moe_expert_ffn(cfg, x, off, w1, b1, w2, b2, a, hd, y, ws)
    torch.cuda.synchronize()
    ra, rh, ry = O.expert_ffn(f64(x), np.asarray(off.cpu(), np.int64), experts(w1), experts(b1), experts(w2),
                              experts(b2), act, "bf16")
    if h:
        close(f64(a), ra, 2e-2)
        close(f64(hd), rh, 2e-2)
    close(f64(y), ry, 2e-2)
