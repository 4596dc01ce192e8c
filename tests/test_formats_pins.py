"""Pins of the storage-format conversions (bf16 and 4-bit blockwise) on both
sides of the inputs: the generator's encoders and the oracle's decoders are
checked against library routines and hand-built cases, not against each other
alone."""
import numpy as np
import scipy.stats
import torch

import oracle as O
import synthetic as S


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        rng.standard_normal(1000).astype(np.float32) * 1e-30,
        rng.standard_normal(1000).astype(np.float32) * 1e30,
        # exact ties: lower 16 bits == 0x8000 with even and odd upper halves
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32) + 0,
    ])
    mine = S.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)


def test_oracle_bf16_decode_matches_torch():
    bits = np.random.default_rng(1).integers(0, 0x7F80, 50000).astype(np.uint16)
    bits[::2] |= 0x8000
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_bits_to_f64(bits), ref)


def test_codebook_is_normal_quantiles():
    cb = S.nf4_codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[-1] == 1.0 and cb[7] == 0.0
    assert (cb > 0).sum() == 8 and (cb < 0).sum() == 7
    d = 1 - 1 / 32
    pos = scipy.stats.norm.ppf(np.linspace(0.5, d, 9)[1:])
    neg = scipy.stats.norm.ppf(np.linspace(0.5, d, 8)[1:])
    np.testing.assert_allclose(cb[8:], pos / pos.max(), rtol=1e-6)
    np.testing.assert_allclose(cb[:7], (-neg / neg.max())[::-1], rtol=1e-6)
    # fp32 values, not narrowed to a shorter format: most entries are not bf16 values
    assert (cb.view(np.uint32) & 0xFFFF).astype(bool).sum() >= 12


def test_nf4_pack_unpack_round_trip_and_nibble_order():
    cb = S.nf4_codebook()
    # weights that sit exactly on codebook values * absmax -> known codes
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 16, size=(3, 128)).astype(np.uint8)
    codes[:, 0] = 15                      # absmax of each block = the +1 entry
    codes[:, 64] = 15
    scale = np.float32(0.5)
    w = cb[codes] * scale
    packed, absmax = S.quantize_nf4(w, cb)
    assert absmax.shape == (3, 2) and np.all(absmax == scale)
    np.testing.assert_array_equal(O.nf4_unpack(packed), codes)
    # element 2i in the low nibble, 2i+1 in the high nibble
    assert packed[0, 0] == (codes[0, 0] | (codes[0, 1] << 4))


def test_nf4_dequant_is_codebook_times_absmax_in_fp32():
    cb = S.nf4_codebook()
    rng = np.random.default_rng(3)
    w = rng.standard_normal((4, 192)).astype(np.float32) * np.float32(0.02)
    packed, absmax = S.quantize_nf4(w, cb)
    deq = O.nf4_dequant(packed, absmax, cb)
    for r in range(4):
        for c in range(192):
            byte = int(packed[r, c // 2])
            code = (byte >> 4) if c % 2 else (byte & 15)
            assert deq[r, c] == np.float32(cb[code] * absmax[r, c // 64])
    # nearest-code quantiser: error at most half the widest codebook gap
    gap = np.diff(cb).max() / 2
    err = np.abs(deq - w) / np.repeat(absmax, 64, axis=1)
    assert err.max() <= gap + 1e-6


def test_workloads_are_seeded_and_shaped():
    a = S.make("tiny")
    b = S.make("tiny")
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w_gate_up, b.w_gate_up)
    assert a.x.shape == (8, 256) and a.w_gate_up.shape == (16, 256, 256) and a.w_down.shape == (16, 256, 128)
    s1 = S.make("tiny", T=4)
    assert s1.x.shape == (4, 256) and not np.array_equal(s1.x, a.x[:4])
    xs = O.bf16_bits_to_f64(a.x)
    assert 0.8 < xs.std() < 1.2
    ws = O.bf16_bits_to_f64(a.w_gate_up)
    assert 0.018 < ws.std() < 0.022
    assert np.allclose(S.skew_bias(4), [-1.1 * np.log(r + 1) for r in range(4)], atol=1e-7)
