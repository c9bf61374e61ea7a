"""The seeded synthetic inputs have the shapes and structure of the pages' workloads."""
import numpy as np
import torch

from w8a8_int8_quantized_qk_amd import workloads as wl


def test_tiny_workload_shapes_and_ranges():
    d = wl.generate("tiny_fp32")
    assert d["x"].dtype == torch.float32 and tuple(d["x"].shape) == (16, 256)
    assert d["w"].dtype == np.int8 and d["w"].shape == (256, 128)
    assert d["w"].min() >= -127 and d["w"].max() <= 127
    assert d["s_ch"].dtype == np.float32 and d["s_ch"].shape == (128,)
    assert d["s_ch"].min() >= 1e-3 and d["s_ch"].max() <= 1e-2


def test_seeded_generation_is_deterministic():
    a = wl.generate("tiny_fp32", seed=0)
    b = wl.generate("tiny_fp32", seed=0)
    c = wl.generate("tiny_fp32", seed=1)
    assert torch.equal(a["x"], b["x"]) and np.array_equal(a["w"], b["w"])
    assert not torch.equal(a["x"], c["x"])


def test_outlier_columns_are_one_percent_of_k_and_fixed_across_rows():
    w = wl.Workload("small_outliers", 64, 4096, 8, "bf16", "bf16", outlier_cols=41)
    x = wl.generate(w)["x"].float().numpy()
    col_rms = np.sqrt((x ** 2).mean(axis=0))
    big = np.where(col_rms > 10)[0]
    assert big.size == 41
    assert np.all(np.abs(x[:, big]).max(axis=0) > 20)


def test_decode_workloads_share_weight_and_first_row():
    # generation draws X first, so only the weight draw after X differs with M;
    # both start from the same seed
    w1 = wl.WORKLOADS["decode_m1"]
    w8 = wl.WORKLOADS["decode_m8"]
    assert (w1.k, w1.n) == (w8.k, w8.n) == (4096, 14336)
    assert w1.m == 1 and w8.m == 8


def test_bits_roundtrip():
    x = wl.cast(np.array([[1.0, -2.5, 3.0e38]], np.float32), "bf16")
    b = wl.bits(x)
    assert b.dtype == np.uint16
    assert torch.equal(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16), x)


def test_edge_rows_cover_the_degenerate_cases():
    for dt in ("f32", "bf16", "f16"):
        r = wl.edge_rows(64, dt).float()
        assert not r[0].any()
        assert (r[1] != 0).sum() == 1
        assert torch.isfinite(r).all()
