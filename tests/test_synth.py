"""Seeded input generators: determinism and the workloads' input structure."""
import numpy as np

from bit_quantized_attention_online_amd import synth


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], dtype=np.float32)
    assert synth.bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x0000]


def test_slices_are_deterministic_and_independent():
    a = synth.normal_bits(2, synth.K_ID, 1, 3, (16, 128))
    b = synth.normal_bits(2, synth.K_ID, 1, 3, (16, 128))
    c = synth.normal_bits(2, synth.K_ID, 1, 4, (16, 128))
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_outlier_structure():
    w = dict(synth.WORKLOADS[2], Nk=64)
    k = synth.prefill_k_slice(2, w, 0, 5)
    plain = synth.normal_bits(2, synth.K_ID, 0, 5, (64, 128))
    ch = synth.outlier_channels(2, 0, 5, 128, 4)
    assert len(set(ch.tolist())) == 4
    other = np.setdiff1d(np.arange(128), ch)
    assert np.array_equal(k[:, other], plain[:, other])
    ratio = synth.bits_to_f32(k[:, ch]) / synth.bits_to_f32(plain[:, ch])
    assert np.allclose(ratio[np.isfinite(ratio)], 20, rtol=1e-2)
    rows = synth.outlier_rows(4, 0, 1, 131072)
    assert len(rows) == 2621 and len(np.unique(rows)) == 2621
