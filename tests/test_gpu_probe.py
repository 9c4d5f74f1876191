"""The measurement probes (msa_read_probe, msa_stream_probe) through the C
ABI: they touch only their buffers, and the stream probe writes every word
of its destination."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nb():
    import nvfp4_kv_cache_amd as m
    m.lib()
    return m


def test_read_probe_reads_only(nb):
    print("[probe] read", flush=True)
    buf = torch.randint(0, 256, (1 << 20,), dtype=torch.uint8, device="cuda")
    before = buf.clone()
    sink = torch.zeros(16, dtype=torch.int32, device="cuda")
    nb.msa_read_probe(buf, 1 << 16, sink)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)


@pytest.mark.parametrize("read_bytes,write_bytes,chunk", [
    (1 << 20, 200 * 1024 + 48, 1 << 16), (77872 * 3, 36224 * 3, 77872), (4096, 65536, 4096),
    (1 << 16, 0, 1 << 12)])
def test_stream_probe_writes_its_destination_only(nb, read_bytes, write_bytes, chunk):
    print(f"[probe] stream read={read_bytes} write={write_bytes} chunk={chunk}", flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(read_bytes + write_bytes)
    src = torch.randint(0, 256, (read_bytes,), dtype=torch.uint8, device="cuda", generator=g)
    guard = 4096
    out = torch.full((write_bytes + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    dst = out[guard:guard + write_bytes]
    src_before = src.clone()
    nb.msa_stream_probe(src, dst, chunk)
    torch.cuda.synchronize()
    assert torch.equal(src, src_before)
    host = out.cpu().numpy()
    assert (host[:guard] == 0xA5).all() and (host[guard + write_bytes:] == 0xA5).all()
    if write_bytes == 0:
        return
    # every destination word was written (a written word equals the 0xA5
    # sentinel with probability 2^-128)
    words = dst.cpu().numpy().reshape(-1, 16)
    assert not (words == 0xA5).all(axis=1).any()
