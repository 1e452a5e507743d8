"""Checks of the seeded input generators (CPU only)."""
import numpy as np

import synth


def test_pack_codes_layout_and_determinism():
    raw = np.arange(16, dtype=np.uint8).reshape(1, 16)
    packed = synth.pack_codes(raw)
    assert packed.dtype == np.uint32 and packed.shape == (1, 2)
    assert packed[0, 0] == 0x76543210 and packed[0, 1] == 0xFEDCBA98
    a = synth.single_gemv(seed=0)
    b = synth.single_gemv(seed=0)
    assert np.array_equal(a["w"].codes, b["w"].codes) and np.array_equal(a["x"], b["x"])
    c = synth.single_gemv(seed=1)
    assert not np.array_equal(a["w"].codes, c["w"].codes)


def test_single_gemv_recipe_distribution():
    d = synth.single_gemv(keep_raw=True)
    w = d["w"]
    assert w.codes.shape == (1024, 128) and w.scales.shape == (1024, 16)
    assert w.raw_codes.min() == 0 and w.raw_codes.max() == 15
    counts = np.bincount(w.raw_codes.ravel(), minlength=16) / w.raw_codes.size
    assert np.all(np.abs(counts - 1 / 16) < 0.002)
    assert w.scales.dtype == np.float32 and 0.005 <= w.scales.min() and w.scales.max() <= 0.02
    resid = w.biases.astype(np.float64) + 8 * w.scales.astype(np.float64)
    assert abs(resid.std() - 0.001) < 1e-4 and abs(resid.mean()) < 1e-4
    assert d["x"].dtype == np.float32 and abs(d["x"].std() - 1) < 0.1
    assert w.weight_bytes == 655_360


def test_bf16_recipe_and_weight_bytes():
    d = synth.qkv_multi(hidden=512, outs=(512, 128, 128))
    for w in d["ws"]:
        assert w.scales.dtype == np.uint16 and w.biases.dtype == np.uint16
        s = synth.bf16_bits_to_f32(w.scales)
        b = synth.bf16_bits_to_f32(w.biases)
        assert 0.0049 <= s.min() and s.max() <= 0.0201
        assert np.all(np.abs(b + 8 * s) < 0.01)
    assert d["x"].dtype == np.uint16
    # weight bytes of the full-size q/k/v set: codes + bf16 scales + bf16 biases
    full = sum(n * 4096 // 2 + 2 * 2 * n * 4096 // 64 for n in (4096, 1024, 1024))
    assert full == 14_155_776


def test_moe_recipe_shapes():
    d = synth.moe_layer(n_experts=8, hidden=256, inter=64, n_tokens=3)
    assert d["gate"].codes.shape == (8, 64, 32)
    assert d["down"].codes.shape == (8, 256, 8)
    assert d["x"].shape == (3, 256) and d["residual"].shape == (3, 256)
    assert d["logits"].shape == (3, 8) and d["logits"].dtype == np.float32


def test_prefill_recipe_shapes():
    d = synth.prefill_gemm(T=40, n_out=64, k_in=128)
    assert d["X"].shape == (40, 128) and d["X"].dtype == np.uint16
    assert d["w"].codes.shape == (64, 16)
