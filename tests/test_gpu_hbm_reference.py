"""The HBM reference reads (decode_attn_hbm_reference) through the C ABI: they read the
words, tiles and scale records they are given and nothing else, skip tile entries outside
the pool, and write only their sink. Each case plants one 32-bit word so that exactly the
lanes whose fold of what they read equals the sink key write it. Their rates are measured
by `bench.py --op hbm`, not here."""

import pytest

pytestmark = pytest.mark.gpu

KEY = 0x9e3779b9          # the sink key of the reference kernels
KEY_I32 = KEY - (1 << 32)
TILE = 4096


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available(), "GPU tests need an MI355X"
    return t


@pytest.fixture(scope="module")
def binding(torch):
    from decode_phase_attention_paged_amd import binding as b
    b.load_library()
    return b


def plant(torch, nbytes, offset, fill=0):
    """A device byte buffer of `fill` with the key's four bytes at `offset`."""
    host = torch.full((nbytes,), fill, dtype=torch.uint8)
    host[offset:offset + 4] = torch.tensor(list(KEY.to_bytes(4, "little")), dtype=torch.uint8)
    return host.to("cuda:0")


def hits(torch, sink):
    torch.cuda.synchronize()
    idx = (sink != 0).nonzero().flatten().tolist()
    return idx, [int(sink[i]) for i in idx]


@pytest.mark.parametrize("depth", [1, 2, 4])
@pytest.mark.parametrize("nt", [True, False])
def test_gather_reads_the_listed_tiles_only(torch, binding, depth, nt):
    n_tiles, t, lane, load = 37, 23, 5, 2
    # The key sits in K tile t at the 16-byte word that `lane` reads with its `load`-th
    # load; every other tile of K and all of V hold zeros (tile t of V too), and tiles
    # never listed are 0xFF-filled in a second pool pair to catch stray reads.
    k = plant(torch, n_tiles * TILE, t * TILE + load * 1024 + lane * 16)
    v = torch.zeros_like(k)
    tiles = torch.tensor([-1, n_tiles, t, 1 << 30], dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    binding.hbm_reference(binding.HBM_GATHER, k, sink, b=v, tiles=tiles, depth=depth,
                          nontemporal=nt, grid=1)
    # Four waves over four entries: wave w takes entry w; entry 2 (tile t) is wave 2's.
    assert hits(torch, sink) == ([2 * 64 + lane], [KEY_I32])

    # The same tile with every other tile of both pools non-zero: a lane that read a tile
    # it was not given would fold garbage, not the key.
    k2 = plant(torch, n_tiles * TILE, t * TILE + load * 1024 + lane * 16, fill=0xFF)
    k2[t * TILE:(t + 1) * TILE] = 0
    k2[t * TILE + load * 1024 + lane * 16:t * TILE + load * 1024 + lane * 16 + 4] = \
        torch.tensor(list(KEY.to_bytes(4, "little")), dtype=torch.uint8, device="cuda:0")
    v2 = torch.full_like(k2, 0xFF)
    v2[t * TILE:(t + 1) * TILE] = 0
    sink.zero_()
    one = torch.tensor([t], dtype=torch.int32, device="cuda:0")
    binding.hbm_reference(binding.HBM_GATHER, k2, sink, b=v2, tiles=one, depth=depth,
                          nontemporal=nt, grid=1)
    # One entry over four waves: the last wave takes it.
    assert hits(torch, sink) == ([3 * 64 + lane], [KEY_I32])


@pytest.mark.parametrize("depth", [1, 2, 4])
@pytest.mark.parametrize("nt", [True, False])
def test_scaled_gather_reads_codes_and_scale_records(torch, binding, depth, nt):
    n_tiles, t = 29, 11
    tiles = torch.tensor([t, -5, n_tiles, 2 * n_tiles], dtype=torch.int32, device="cuda:0")
    zeros = lambda n: torch.zeros(n, dtype=torch.uint8, device="cuda:0")
    # The key in V's 2 KiB tile t, at the word lane 40 reads with its second load.
    v = plant(torch, n_tiles * 2048, t * 2048 + 1024 + 40 * 16)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    binding.hbm_reference(binding.HBM_GATHER_SCALED, zeros(n_tiles * 2048), sink, b=v,
                          tiles=tiles, a_scale=zeros(n_tiles * 64), b_scale=zeros(n_tiles * 64),
                          depth=depth, nontemporal=nt, grid=1)
    assert hits(torch, sink) == ([40], [KEY_I32])          # entry 0 is wave 0's
    # The key in dword 7 of K's scale record t: lanes 7, 23, 39 and 55 each read it once.
    ks = plant(torch, n_tiles * 64, t * 64 + 7 * 4)
    sink.zero_()
    binding.hbm_reference(binding.HBM_GATHER_SCALED, zeros(n_tiles * 2048), sink,
                          b=zeros(n_tiles * 2048), tiles=tiles, a_scale=ks,
                          b_scale=zeros(n_tiles * 64), depth=depth, nontemporal=nt, grid=1)
    assert hits(torch, sink) == ([7, 23, 39, 55], [KEY_I32] * 4)


@pytest.mark.parametrize("unroll", [4, 8, 16])
@pytest.mark.parametrize("nt", [True, False])
def test_stream_reads_every_word_once(torch, binding, unroll, nt):
    grid = 3
    step = 256 * unroll
    words = grid * step * 2 + 77            # two steps per workgroup and a ragged tail
    for word in (0, step + 13, words - 1):
        buf = plant(torch, words * 16, word * 16)
        sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda:0")
        binding.hbm_reference(binding.HBM_STREAM, buf, sink, depth=unroll, nontemporal=nt,
                              grid=grid)
        # Word w is read by thread w % 256 of workgroup (w // step) % grid.
        assert hits(torch, sink) == ([((word // step) % grid) * 256 + word % 256], [KEY_I32])
    # A count short of the buffer leaves the rest unread.
    buf = plant(torch, words * 16, (words - 1) * 16)
    sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda:0")
    binding.hbm_reference(binding.HBM_STREAM, buf, sink, depth=unroll, nontemporal=nt,
                          grid=grid, count=words - 1)
    assert hits(torch, sink) == ([], [])
