"""GPU check of the streaming-read reference kernel (the read ceiling the
decode roofline is compared with): every 32-bit word of the buffer is read
exactly once, so the XOR of the per-workgroup results equals the XOR of the
buffer computed on the host, for grids that divide the buffer evenly, leave
a ragged tail, or have more threads than 16-byte pieces."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)
import paged_kv_cache_292_amd as P  # noqa: E402  (fails loudly when the library is missing)


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 3 * 2 ** 20 + 16 * 7, 64 * 2 ** 20])
@pytest.mark.parametrize("wg", [1, 7, 1024])
def test_stream_read_reads_every_word_once(nbytes, wg):
    rng = np.random.default_rng(nbytes + wg)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    out = torch.full((wg,), -1, dtype=torch.int32, device="cuda")
    P.stream_read(src, out, wg)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_stream_read_of_an_offset_view():
    """A 16-byte-aligned view into a larger tensor reads only its own bytes."""
    host = np.arange(1 << 16, dtype=np.uint32) * np.uint32(2654435761)
    big = torch.from_numpy(host.view(np.int32)).cuda()
    view = big[4:4 + 4096]  # 16 bytes in, 16 KB long
    out = torch.zeros(64, dtype=torch.int32, device="cuda")
    P.stream_read(view, out, 64)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host[4:4 + 4096])
