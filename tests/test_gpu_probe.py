"""The streaming bandwidth probe (cgtp_stream_probe), through the C ABI: a
copy reproduces its source bit for bit, a write leaves the documented
pattern, a read leaves its buffers unchanged, on sizes that are and are not
a multiple of the launch's grid."""
import numpy as np
import pytest

from tests.gpu_util import binding

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_vec", [1, 1000, 256 * 2048 + 37])
def test_stream_probe_kinds(n_vec):
    import torch
    B = binding()
    print(f"stream probe: {n_vec} 16-byte vectors", flush=True)
    g = torch.Generator(device="cpu").manual_seed(n_vec)
    a = torch.randn(4 * n_vec, generator=g).cuda()
    b = torch.full((4 * n_vec,), -5.0, device="cuda")
    B.cgtp_stream_probe("copy", a, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    B.cgtp_stream_probe("write", None, b)
    torch.cuda.synchronize()
    want = np.tile(np.array([1, 2, 3, 0], np.float32), n_vec)
    want[3::4] = (np.arange(n_vec) & 1023).astype(np.float32)
    assert np.array_equal(b.cpu().numpy(), want)
    a0, b0 = a.clone(), b.clone()
    B.cgtp_stream_probe("read", a, b)
    torch.cuda.synchronize()
    assert torch.equal(a, a0) and torch.equal(b, b0)
