"""The read-bandwidth calibration kernel (pkv_read_tiles): every lane's sink
word must be the xor of exactly the 32-bit words it was told to read, for
gathered and contiguous tiles, ragged wave counts and ids outside the
buffer.  The expected values are plain numpy xors of the same buffer."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TILE_WORDS = 4096 // 4


def expected_sink(words: np.ndarray, order, n_tiles: int, tpw: int, tile_bytes: int = 4096) -> np.ndarray:
    """words: the buffer as uint32 [tiles * tile_bytes / 4]; lane l of a wave
    reads the 16-byte vectors l, l + 64, ... of each of its tiles."""
    groups = tile_bytes // 1024                          # 16-byte vectors per lane
    tiles = words.reshape(-1, groups, 64, 4)             # [tile][vector group c][lane][word]
    ids = np.arange(n_tiles) if order is None else np.asarray(order, dtype=np.int64)[:n_tiles]
    waves = -(-n_tiles // tpw)
    out = np.zeros((waves, 64), dtype=np.uint32)
    for w in range(waves):
        for t in ids[w * tpw:(w + 1) * tpw]:
            if 0 <= t < tiles.shape[0]:
                out[w] ^= np.bitwise_xor.reduce(tiles[t].transpose(1, 0, 2).reshape(64, 4 * groups), axis=1)
    return out.reshape(-1)


def run(words: np.ndarray, order, n_tiles: int, tpw: int, tile_bytes: int = 4096) -> np.ndarray:
    from paged_kv_cache_08_amd import pkv as P
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    dorder = None if order is None else torch.from_numpy(np.asarray(order, dtype=np.int32)).cuda()
    waves = -(-n_tiles // tpw)
    sink = torch.full((waves * 64,), -1, dtype=torch.int32, device="cuda")
    P.pkv_read_tiles(buf, dorder, n_tiles, tpw, sink, tile_bytes=tile_bytes)
    torch.cuda.synchronize()
    return sink.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("tiles,n,tpw,gather", [
    (64, 64, 16, False),       # whole waves of full depth
    (70, 70, 13, False),       # ragged: a short last wave and a remainder loop in every wave
    (300, 300, 64, True),      # gather over a permutation
    (300, 257, 7, True),       # fewer tiles than the permutation, tiny waves
    (5, 5, 256, True),         # one wave, remainder loop only
])
@pytest.mark.parametrize("tile_bytes", [4096, 2048, 1024])
def test_read_tiles_xor(tiles, n, tpw, gather, tile_bytes):
    rng = np.random.default_rng(tiles * 1000 + n + tpw)
    words = rng.integers(0, 2**32, size=tiles * tile_bytes // 4, dtype=np.uint32)
    order = rng.permutation(tiles).astype(np.int32) if gather else None
    got = run(words, order, n, tpw, tile_bytes)
    np.testing.assert_array_equal(got, expected_sink(words, order, n, tpw, tile_bytes))


def test_read_tiles_ids_outside_buffer_read_nothing():
    rng = np.random.default_rng(7)
    tiles = 40
    words = rng.integers(0, 2**32, size=tiles * TILE_WORDS, dtype=np.uint32)
    order = rng.permutation(tiles).astype(np.int32)
    order[[0, 9, 17, 33]] = [-1, tiles, 1 << 30, -(1 << 30)]
    for tpw in (8, 16, 5):           # invalid ids inside the depth-8 loop and in the remainder loop
        got = run(words, order, tiles, tpw)
        np.testing.assert_array_equal(got, expected_sink(words, order, tiles, tpw))
