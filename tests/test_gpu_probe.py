"""GPU checks of the measurement aids (librkv_probe.so, csrc/probe/rkv_probe.h): each computes
what its header states, so the peaks the benchmark reports beside the
published ones come from the stated work."""
import numpy as np
import pytest
import torch

from fp8_ring_kv_amd import probe as rkv
from tests.gpu_common import DEV, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_mfma_probe_accumulates_every_instruction():
    """e4m3 1.0 operands: every 32x32x64 instruction adds 64 to each
    accumulator element; the sink holds four chains' elements per workgroup."""
    wg, iters = 300, 37
    sink = torch.full((wg,), -1.0, dtype=torch.float32, device=DEV)
    rkv.rkv_probe_fp8_mfma(wg, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(sink == 4 * 64 * iters), sink[:4]


def test_stream_probe_rewrites_every_word_once():
    n = (1 << 20) + 48  # not a multiple of the workgroup's 16 KiB step: a ragged tail
    rng = np.random.default_rng(0)
    host = rng.integers(0, 2**32, size=n // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32).copy()).to(DEV)
    s = torch.cuda.current_stream().cuda_stream
    rkv.rkv_probe_stream(buf.data_ptr(), n, s)
    once = buf.cpu().numpy().view(np.uint32).reshape(-1, 4)
    want = host.reshape(-1, 4).copy()
    want[:, 0] = ~want[:, 0]
    assert np.array_equal(once, want)
    rkv.rkv_probe_stream(buf.data_ptr(), n, s)
    assert np.array_equal(buf.cpu().numpy().view(np.uint32), host)
