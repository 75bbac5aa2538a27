"""Seeded input generators (shared by the tests and the benchmark; no GPU)."""

import numpy as np
import torch

from exact_attention_35_amd import inputs


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(1_000_000).astype(np.float32) * np.float32(3.0),
        rng.standard_normal(10_000).astype(np.float32) * np.float32(1e-38),  # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-45, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8,
                  1.0 + 2.0**-9, 1.0 - 2.0**-9], dtype=np.float32),
    ])
    got = inputs.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    nan = inputs.bf16_round(np.array([np.nan], dtype=np.float32))
    assert np.isnan(nan[0])


def test_ties_round_to_even():
    # 1 + 2^-8 lies halfway between two bf16 values; even mantissa wins (1.0)
    assert inputs.bf16_round(np.array([1.0 + 2.0**-8], np.float32))[0] == 1.0
    assert inputs.bf16_round(np.array([1.0 + 3 * 2.0**-8], np.float32))[0] == 1.0 + 4 * 2.0**-8


def test_seeds_reproduce_and_differ():
    w = inputs.WORKLOADS["gpt2_small_s1k"]
    a = inputs.make_qkv(w, (1, 2, 64, 64))
    b = inputs.make_qkv(w, (1, 2, 64, 64))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], a[1])
    assert a[3] is not None
    assert np.array_equal(inputs.bf16_round(a[0]), a[0])


def test_qk_multiplier():
    w = inputs.WORKLOADS["long_s16k_d128"]
    q, k, v, _ = inputs.make_qkv(w, (1, 1, 4096, 128))
    assert abs(q.std() - 1.7) < 0.02 and abs(k.std() - 1.7) < 0.02 and abs(v.std() - 1.0) < 0.02


def test_block_mask_exact_density():
    w = inputs.WORKLOADS["blocksparse_s64k"]
    nb = w.N // inputs.MASK_BLOCK
    m = inputs.make_block_mask(nb, w.density, w.index, causal=True)
    assert m.shape == (512, 512)
    assert np.all(np.diag(m) == 1)
    assert np.all(np.triu(m, 1) == 0)
    assert int(np.tril(m, -1).sum()) == 8176
    assert int(m.sum()) == 8688
    assert np.array_equal(m, inputs.make_block_mask(nb, w.density, w.index, causal=True))


def test_sample_rows():
    r = inputs.sample_rows(16384, 512, 4)
    assert r.size == 512 and np.all(np.diff(r) > 0)
    for f in (0, 1, 127, 128, 8192, 16383):
        assert f in r
    assert inputs.sample_rows(5, 512, 4).tolist() == [0, 1, 2, 3, 4]


def test_workload_table():
    names = list(inputs.WORKLOADS)
    assert names == ["tiny_f32", "bert_large_s512", "gpt2_small_s1k", "long_s16k_d128", "blocksparse_s64k",
                     "gqa_s16k_h32_kv8_d128"]
    g = inputs.WORKLOADS["gqa_s16k_h32_kv8_d128"]
    assert g.kv_shape == (1, 8, 16384, 128) and g.shape == (1, 32, 16384, 128)
    q, k, v, _ = inputs.make_qkv(g, (1, 4, 256, 128))
    assert q.shape == (1, 4, 256, 128) and k.shape == v.shape == (1, 1, 256, 128)
    q, k, v, do = inputs.random_case(3, 2, 6, 50, 64, backward=True, h_kv=2)
    assert q.shape == do.shape == (2, 6, 50, 64) and k.shape == v.shape == (2, 2, 50, 64)
    assert inputs.WORKLOADS["tiny_f32"].dtype == "f32"
    assert inputs.WORKLOADS["long_s16k_d128"].scale == np.float32(1.0) / np.sqrt(np.float32(128))
