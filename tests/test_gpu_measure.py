"""GPU checks of the measurement entry points bench.py uses: the shader clock
under MFMA load is a plausible engine clock, and the streaming floor launch
runs over odd sizes and writes every word of its destination."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp8_e4m3_latent_amd as m
    m.lib()
    return m


def test_shader_clock_is_plausible(kv8):
    mhz = kv8.shader_clock_mhz(2000)
    print("shader clock under MFMA load: %.0f MHz" % mhz, flush=True)
    assert 300.0 < mhz < 3000.0


@pytest.mark.parametrize("na,nb,nw", [(1000, 0, 0), (4096, 48, 1024), (64 * 5 + 3, 17, 65), (16, 16, 7000)])
def test_stream_floor_writes_every_destination_word(kv8, na, nb, nw):
    a = torch.arange(na * 4, dtype=torch.int32, device="cuda")
    b = torch.arange(nb * 4, dtype=torch.int32, device="cuda") if nb else None
    # one guard word after the destination stays untouched
    d = torch.full((nw * 4 + 4,), -7, dtype=torch.int32, device="cuda")
    reads = [a] + ([b] if b is not None else [])
    kv8.stream_floor(reads, d[: nw * 4] if nw else None)
    torch.cuda.synchronize()
    assert bool((d[nw * 4:] == -7).all())
    if nw:
        w = d[: nw * 4].view(nw, 4)
        # word j carries (x, x, x, x) for some x; a word never written keeps -7
        # in every lane, which only a read range of -7s could produce
        assert bool((w == w[:, :1]).all())
        assert not bool((w == -7).all(dim=1).any())
