"""A token's outputs do not depend on how many tokens share its call.

The grouped matmuls pick their tile height from the rows per segment on
average (64, 128 or 256 rows with bf16 tokens; 64, 128 or 192 with fp8
tokens), and the router switches paths at 4096 tokens.  Every row's sums
keep the same order whatever the tile height, so the first n tokens of an
8,000-token batch at the LingBot dims must come out bitwise equal when they
are run alone, for n chosen so that each tile height runs."""
import pytest
import torch

import routed_moe_dit_amd as lbv
import synth
from gpu_util import forward, note, upload
from test_gpu_fp8 import forward_fp8
from test_gpu_w8a8 import forward_w8a8

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lbv.load()
    yield


@pytest.fixture(scope="module")
def lingbot_8000():
    wl = W[3].replace(T=8000)
    inp = synth.make_inputs(wl)
    return wl, upload(wl, inp)


# rows per segment on average at n tokens: 8000 -> 558, 1600 -> 112,
# 800 -> 56, 200 -> 14 (bf16 tokens: 256, 128, 128, 64 rows; fp8 weights:
# 256, 128, 64 for gate/up and 128 for down, 64; fp8 tokens: 192, 192, 128, 64)
@pytest.mark.timeout(300)
@pytest.mark.parametrize("path", ["bf16", "fp8_weights", "w8a8"])
def test_outputs_independent_of_batch_size(path, lingbot_8000):
    wl, d = lingbot_8000
    note("tile height vs batch size, %s" % path)
    run = {"bf16": forward, "fp8_weights": forward_fp8, "w8a8": forward_w8a8}[path]
    out, ids, w = run(wl, d)
    for n in (1600, 800, 200):
        part = dict(d, x=d["x"][:n].contiguous())
        o, i, ww = run(wl.replace(T=n), part)
        assert torch.equal(i, ids[:n]), (path, n)
        assert torch.equal(ww, w[:n]), (path, n)
        assert torch.equal(o, out[:n]), (path, n)
