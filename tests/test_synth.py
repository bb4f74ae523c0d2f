"""Host-side checks of the seeded input generators (no GPU)."""
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) >= 3
    for r in rows:
        ctr = np.array([[int(v, 16) for v in r[0:4]]], dtype=np.uint32)
        key = (int(r[4], 16), int(r[5], 16))
        expect = [int(v, 16) for v in r[6:10]]
        assert synth.philox4x32_10(ctr, key)[0].tolist() == expect


def test_words_are_windowed_consistently():
    full = synth.words(3, 77, 40)
    for start in (0, 1, 2, 3, 5, 17):
        np.testing.assert_array_equal(synth.words(3, 77, 40 - start, start=start), full[start:])


def test_distributions_roughly_right():
    u = synth.uniform_f32(1, 2, 200_000, 0.001, 0.02)
    assert u.min() >= 0.001 and u.max() < 0.02
    assert abs(u.mean() - 0.0105) < 1e-4
    z = synth.normal_f32(1, 3, 200_000, 0.05)
    assert abs(z.mean()) < 1e-3 and abs(z.std() - 0.05) < 5e-4
    b = synth.f32_to_bf16_bits(np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                                         1.0 + 2 ** -8 + 2 ** -9], np.float32))
    # ties go to the even mantissa (1+2^-8 -> 1.0, 1+3*2^-8 -> 1+2^-6); above a tie rounds up
    assert b.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81]


def test_expert_block_layout_and_streams():
    H, I, bits = 128, 64, 4
    blk = synth.expert_block(5, 2, 9, H, I, bits)
    lay = synth.expert_layout(H, I, bits)
    assert blk.size == lay["total"]
    o, s = lay["up_codes"]
    np.testing.assert_array_equal(blk[o:o + s],
                                  synth.stream_bytes(5, synth.tensor_id(synth.K_UP_CODES, 9, 2), s))
    codes, sb = synth.matrix(5, 2, 9, 2, H, I, bits)
    o, s = lay["down_codes"]
    np.testing.assert_array_equal(blk[o:o + s], codes.reshape(-1))
    o, s = lay["down_sb"]
    np.testing.assert_array_equal(blk[o:o + s].view(np.uint32), sb.reshape(-1))
