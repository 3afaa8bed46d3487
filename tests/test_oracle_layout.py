"""oracle.layout: the stored order of the cache pools, pinned to positions
worked out by hand from the format definition (K chunk c of token t at byte
(c*16 + t)*16; V element (t, d) at ((n//G)*64 + (t//4)*16 + d%16)*16 +
((n%G)*4 + t%4)*eb with n = d//16, G = 4//eb), plus round trips."""
import numpy as np
import pytest

from oracle import layout


def _coded(d, dtype, bs=16):
    """A one-group pool whose element (t, d) holds a unique code t*1000 + d
    (as much of it as the dtype holds)."""
    t = np.arange(bs)[:, None]
    dd = np.arange(d)[None, :]
    code = (t * 1000 + dd) if dtype != np.int8 else ((t * 16 + dd) % 251 - 125)
    return code.astype(dtype).reshape(1, 1, bs, d)


# (dtype, d, kind, token, dim, element index in the stored group) — by hand.
HAND = [
    (np.float16, 128, "k", 3, 9, 153),     # byte ((18>>4)*16 + 3)*16 + (18&15) = 306
    (np.float16, 128, "v", 5, 37, 681),    # n=2 r=5 c=1 i=1 G=2: ((1*64+16+5)*16 + 2) / 2
    (np.float16, 128, "k", 15, 127, 2047),  # last chunk of the last token
    (np.int8, 128, "v", 14, 50, 814),      # n=3 r=2 c=3 i=2 G=4: (48+2)*16 + (3*4+2)
    (np.int8, 64, "k", 9, 40, 2 * 256 + 9 * 16 + 8),   # chunk 2 of token 9, byte 8
    (np.float32, 128, "k", 7, 5, 93),      # byte ((20>>4)*16 + 7)*16 + 4 = 372
    (np.float32, 64, "v", 2, 17, 262),     # n=1 r=1 c=0 i=2 G=1: ((64+1)*16 + 2*4) / 4
]


@pytest.mark.parametrize("dtype,d,kind,t,dim,idx", HAND)
def test_hand_worked_positions(dtype, d, kind, t, dim, idx):
    logical = _coded(d, dtype)
    stored = (layout.k_to_stored if kind == "k" else layout.v_to_stored)(logical)
    assert stored.reshape(-1)[idx] == logical[0, 0, t, dim]


@pytest.mark.parametrize("dtype", [np.float16, np.float32, np.int8, np.uint8, np.uint16])
@pytest.mark.parametrize("d,bs", [(64, 16), (128, 16), (128, 256), (64, 256)])
def test_round_trips_and_permutation(dtype, d, bs):
    rng = np.random.default_rng(3)
    x = rng.integers(0, 120, size=(3, 2, bs, d)).astype(dtype)
    for to, back in ((layout.k_to_stored, layout.k_from_stored),
                     (layout.v_to_stored, layout.v_from_stored)):
        y = to(x)
        assert y.shape == x.shape
        assert np.array_equal(back(y), x)
        # a permutation within each 16-row group of each (block, head) tile
        g = y.reshape(3, 2, bs // 16, -1)
        h = x.reshape(3, 2, bs // 16, -1)
        assert np.array_equal(np.sort(g, axis=-1), np.sort(h, axis=-1))


def test_v_lane_groups_hold_four_tokens_of_one_column():
    """Each 16-byte piece of the stored V (one lane of a load) holds, per column
    it covers, four consecutive tokens of one row-group of 4."""
    d = 128
    logical = _coded(d, np.float16)
    stored = layout.v_to_stored(logical).reshape(-1)
    piece = stored[8 * (16 * 1 + 5): 8 * (16 * 1 + 5) + 8]     # lane 21 of load 0: c=1, r=5
    assert list(piece[:4]) == [logical[0, 0, 4 + i, 5] for i in range(4)]
    assert list(piece[4:]) == [logical[0, 0, 4 + i, 21] for i in range(4)]


# INT4 V: element (t, d) -> (byte, nibble) by hand, d = 128, bs = 16:
# n = d // 16, r = d % 16, c = t // 4, i = t % 4:
#   byte = (c*16 + r)*16 + ((n % 8)//2)*4 + i, high nibble for odd n.
HAND4 = [
    (0, 0, 0, 0),           # token 0, column 0: first byte, low nibble
    (0, 16, 0, 1),          # column 16 (n = 1) shares the byte, high nibble
    (6, 37, (1 * 16 + 5) * 16 + 1 * 4 + 2, 0),   # n=2 r=5 c=1 i=2
    (13, 125, (3 * 16 + 13) * 16 + 3 * 4 + 1, 1),  # n=7 r=13 c=3 i=1
]


@pytest.mark.parametrize("t,dim,byte,hi", HAND4)
def test_int4_v_hand_worked_positions(t, dim, byte, hi):
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 16, size=(1, 1, 16, 128)).astype(np.uint8)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    stored = layout.v4_to_stored(packed).reshape(-1)
    got = (stored[byte] >> 4) if hi else (stored[byte] & 0xF)
    assert got == codes[0, 0, t, dim]


@pytest.mark.parametrize("d,bs", [(128, 16), (128, 256), (256, 16)])
def test_int4_v_round_trip_and_bytes_hold_one_token(d, bs):
    rng = np.random.default_rng(9)
    x = rng.integers(0, 256, size=(2, 3, bs, d // 2)).astype(np.uint8)
    y = layout.v4_to_stored(x)
    assert np.array_equal(layout.v4_from_stored(y), x)
    # every stored byte holds two elements of a single token: stamp each token's
    # nibbles with its own index and read back one value per byte
    tok = np.broadcast_to((np.arange(bs) % 16).astype(np.uint8)[:, None], (bs, d // 2))
    stamped = np.broadcast_to(tok | (tok << 4), x.shape).copy()
    s = layout.v4_to_stored(stamped)
    assert np.all((s & 0xF) == (s >> 4))
