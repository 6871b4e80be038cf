"""Pins of the oracle's page layout (O5) and dequantization (O6)."""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_layout.json")


def _code_fn(expr):
    return {"c % 4": lambda c: c % 4, "c % 8": lambda c: c % 8, "c % 16": lambda c: c % 16,
            "15 - c % 16": lambda c: 15 - c % 16}[expr]


def test_golden_words(orc):
    g = json.load(open(GOLDEN))
    for case in g["cases"]:
        bits = case["bits"]
        block = np.zeros(orc.block_bytes(bits), np.uint8)
        codes = np.array([_code_fn(case["code"])(c) for c in range(128)], np.uint8)
        orc.pack_token(block, case["which"], bits, case["o"], codes, 0, 0)
        words = block[: 64 * 128 * bits // 8].view("<u4")
        expect = np.zeros_like(words)
        for idx, val in case["words"].items():
            expect[int(idx)] = int(val, 16)
        listed = np.zeros(words.shape, bool)
        listed[[int(i) for i in case["words"]]] = True
        assert np.array_equal(words[listed], expect[listed]), case
        # words not listed: zero unless they belong to this token's written set
        written = words != 0
        assert np.all(written <= (listed | written)), case
    m = g["meta"]
    block = np.zeros(orc.block_bytes(2), np.uint8)
    orc.pack_token(block, 0, 2, m["o"], np.zeros(128, np.uint8), int(m["scale_bits"], 16),
                   int(m["zero_bits"], 16))
    meta = block[2048:]
    for idx, val in m["bytes_after_codes"].items():
        assert meta[int(idx)] == int(val, 16)
    for bits, nbytes in g["block_bytes"].items():
        assert orc.block_bytes(int(bits)) == nbytes
        assert nbytes * 8 / (64 * 128) == g["bits_per_element"][bits]


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("which", [0, 1])
def test_round_trip_and_isolation(orc, bits, which):
    rng = np.random.default_rng(bits * 10 + which)
    block = rng.integers(0, 256, orc.block_bytes(bits), dtype=np.uint8)
    before = block.copy()
    ref = {}
    for o in rng.permutation(64)[:40]:
        codes = rng.integers(0, 1 << bits, 128).astype(np.uint8)
        s, z = rng.integers(0, 65536, 2)
        orc.pack_token(block, which, bits, int(o), codes, int(s), int(z))
        ref[int(o)] = (codes, int(s), int(z))
    for o, (codes, s, z) in ref.items():
        c2, s2, z2 = orc.unpack_token(block, which, bits, o)
        assert np.array_equal(c2, codes) and s2 == s and z2 == z
    # tokens never written keep their original codes and metadata
    for o in set(range(64)) - set(ref):
        assert orc.unpack_token(block, which, bits, o)[0].tolist() == \
            orc.unpack_token(before, which, bits, o)[0].tolist()
        assert orc.unpack_token(block, which, bits, o)[1:] == orc.unpack_token(before, which, bits, o)[1:]


def test_dequant_is_fma_of_stored_values(orc):
    rng = np.random.default_rng(5)
    pool = orc.new_pool(3, 2, 4, rng=rng)
    slots = np.array([0, 63, 64, 130, -1], np.int64)
    out = orc.dequant(pool, 1, 4, slots)
    for i, slot in enumerate(slots[:-1]):
        p, o = divmod(int(slot), 64)
        for h in range(2):
            codes, s, z = orc.unpack_token(pool[p, h], 1, 4, o)
            sf = np.array([s], np.uint16).view(np.float16).astype(np.float64)[0]
            zf = np.array([z], np.uint16).view(np.float16).astype(np.float64)[0]
            ref = codes * sf + zf          # exact in fp64; fma rounds once to fp32
            finite = np.isfinite(ref)
            assert np.array_equal(out[i, h][finite], ref[finite].astype(np.float32))
    assert np.all(out[-1] == 0)


def test_append_skips_negative_and_rejects_out_of_range(orc):
    k = np.ones((2, 1, 128), np.float32)
    kp, vp = orc.new_pool(1, 1, 2), orc.new_pool(1, 1, 2)
    orc.append(kp, vp, k, k, np.array([-1, -5], np.int64))
    assert not kp.any() and not vp.any()
    with pytest.raises(ValueError):
        orc.append(kp, vp, k, k, np.array([0, 64], np.int64))


@pytest.mark.parametrize("which", [0, 1])
def test_three_bit_planes_hold_low_bits_as_two_bit_layout(orc, which):
    """The low plane of a 3-bit block is exactly a 2-bit block's code section for codes & 3,
    and the high plane is a bijection of (token, channel) onto its 8192 bits."""
    rng = np.random.default_rng(33 + which)
    b3 = np.zeros(orc.block_bytes(3), np.uint8)
    b2 = np.zeros(orc.block_bytes(2), np.uint8)
    for o in range(64):
        codes = rng.integers(0, 8, 128).astype(np.uint8)
        orc.pack_token(b3, which, 3, o, codes, 0, 0)
        orc.pack_token(b2, which, 2, o, codes & 3, 0, 0)
    assert np.array_equal(b3[:2048], b2[:2048])
    seen = np.zeros(8192, bool)
    for o in range(64):
        for c in range(128):
            blk = np.zeros(orc.block_bytes(3), np.uint8)
            one = np.zeros(128, np.uint8)
            one[c] = 4
            orc.pack_token(blk, which, 3, o, one, 0, 0)
            bits = np.unpackbits(blk[2048:3072], bitorder="little")
            assert bits.sum() == 1 and not blk[:2048].any()
            seen[np.argmax(bits)] = True
    assert seen.all()
