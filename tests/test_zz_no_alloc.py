"""GPU: the no-allocation decode (tq_decode_attn_noalloc, the library's static device
scratch) against tq_decode_attn with a caller-provided workspace, through the C ABI.

Two calls in a row on the shared scratch, the second with a smaller input: outputs must
equal the workspace entry point's bit for bit (same kernels, same split count) and stay
within 2e-3 of the fp64 oracle. A request beyond the scratch size is rejected with
TQ_ENOSPC before anything is launched.
"""
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from int4_compressed_domain_amd import tq  # noqa: E402
from int4_compressed_domain_amd import workloads as W  # noqa: E402

from .gpu_util import ATTN_TOL, DEV, Case, attn_err  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()


def _noalloc(c, num_splits=0):
    w = c.w
    out = torch.full((w.batch, w.q_heads, w.head_dim), float("nan"), dtype=torch.float32, device=DEV)
    tq.tq_decode_attn_noalloc(c.layout, c.pool, c.q_dev, c.bt_dev, c.lens_dev, int(c.lens.max()),
                              w.attn_scale, out, num_splits=num_splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_workspace_entry_point():
    big = W.WORKLOADS["llama70b_b1_128k"].scaled(context=6000, batch=3)
    small = W.WORKLOADS["llama8b_b16_8k"].scaled(context=700, batch=2)
    for w, lens, splits in ((big, [6000, 5000, 4097], 0), (small, [700, 33], 0), (small, [700, 33], 3)):
        print("case", w.name, lens, "splits", splits, flush=True)
        c = Case(w, seed=55, lens=lens)
        c.fill()
        ref = c.decode_gpu(num_splits=splits)
        got = _noalloc(c, num_splits=splits)
        assert np.array_equal(got, ref), "differs from tq_decode_attn with a workspace"
        assert attn_err(got, c.decode_oracle()).max() <= ATTN_TOL


def test_noalloc_rejects_requests_beyond_its_scratch():
    # 512 sequences x 64 q heads of one page each: the partials alone exceed the scratch
    B, Hq, Hkv, D = 512, 64, 8, 128
    w = W.Workload("noalloc_big", B, Hq, Hkv, D, 16, "bf16", 1.0 / math.sqrt(D))
    c = Case(w, seed=3, lens=[16] * B, oracle=False)
    assert tq.tq_decode_workspace_size(c.layout, B, 16, 0) > (16 << 20)
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device=DEV)
    with pytest.raises(RuntimeError, match="ENOSPC"):
        tq.tq_decode_attn_noalloc(c.layout, c.pool, c.q_dev, c.bt_dev, c.lens_dev, 16, w.attn_scale, out)
