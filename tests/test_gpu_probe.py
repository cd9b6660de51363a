"""The HBM probes (the measurement helpers behind the practical ceilings) compute what the
header says, so their timings are of real streams: the per-workgroup XOR of what was read, the
copy, the XOR of two sources and the counter pattern of a write-only stream. Ragged sizes (not a
multiple of one grid step) and several launch shapes."""
import numpy as np
import pytest

from _gpu import ensure_built, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    ensure_built()


def words(buf):
    """XOR of the four 32-bit words of every 16-byte word."""
    w = buf.view(np.uint32).reshape(-1, 4)
    return w[:, 0] ^ w[:, 1] ^ w[:, 2] ^ w[:, 3]


def per_workgroup_xor(x16, workgroups):
    """Workgroup b reads the 16-byte words i with (i mod 256*workgroups) // 256 == b."""
    owner = (np.arange(x16.size) % (256 * workgroups)) // 256
    out = np.zeros(workgroups, dtype=np.uint32)
    np.bitwise_xor.at(out, owner, x16)
    return out


@pytest.mark.parametrize("nbytes,wgs,u", [(16, 1, 1), (4096 * 16 + 48, 3, 2), (1 << 20, 64, 4), (12345 * 16, 7, 1)])
def test_read_probe_xor(nbytes, wgs, u):
    import torch
    from int8_quantized_projections_amd import q8lib
    rng = np.random.default_rng(nbytes + wgs)
    a = rng.integers(0, 256, nbytes, dtype=np.uint8)
    buf = torch.from_numpy(a).to(dev())
    out = torch.full((wgs,), -1, dtype=torch.int32, device=dev())
    q8lib.hbm_read_probe(buf, wgs, u, out)
    got = out.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(got, per_workgroup_xor(words(a), wgs))


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (4096 * 16 + 48, 3), (1 << 20, 64), (12345 * 16, 7)])
def test_stream_probe_patterns(nbytes, wgs):
    import torch
    from int8_quantized_projections_amd import q8lib
    rng = np.random.default_rng(nbytes * 3 + wgs)
    a = rng.integers(0, 256, nbytes, dtype=np.uint8)
    b = rng.integers(0, 256, nbytes, dtype=np.uint8)
    s0, s1 = torch.from_numpy(a).to(dev()), torch.from_numpy(b).to(dev())
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev())
    out = torch.full((wgs,), -1, dtype=torch.int32, device=dev())
    q8lib.hbm_stream_probe(nbytes, wgs, src0=s0, dst=dst)
    np.testing.assert_array_equal(dst.cpu().numpy(), a)
    q8lib.hbm_stream_probe(nbytes, wgs, src0=s0, src1=s1, dst=dst)
    np.testing.assert_array_equal(dst.cpu().numpy(), a ^ b)
    q8lib.hbm_stream_probe(nbytes, wgs, dst=dst)
    n16 = nbytes // 16
    want = np.stack([np.arange(n16, dtype=np.uint32), np.full(n16, 1, np.uint32), np.full(n16, 2, np.uint32),
                     np.full(n16, 3, np.uint32)], axis=1)
    np.testing.assert_array_equal(dst.cpu().numpy().view(np.uint32).reshape(-1, 4), want)
    q8lib.hbm_stream_probe(nbytes, wgs, src0=s0, out=out)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), per_workgroup_xor(words(a), wgs))
    q8lib.hbm_stream_probe(nbytes, wgs, src0=s0, src1=s1, out=out)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), per_workgroup_xor(words(a ^ b), wgs))
