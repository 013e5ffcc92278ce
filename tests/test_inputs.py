"""Seeded input generators: reproducible, exact bf16 rounding, masks as described."""
import numpy as np
import pytest
import torch

from exact_io_aware_46_amd import inputs as inp


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.Generator(np.random.PCG64(1))
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -0.0, 65504.0, 1e-30, 3.0e38], dtype=np.float32),
                        # exact ties: mantissa low half == 0x8000 (round to even both ways)
                        np.array([0x3F808000, 0x3F818000], dtype=np.uint32).view(np.float32)])
    ours = inp.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    np.testing.assert_array_equal(inp.f32_to_bf16_bits(
        np.array([0x3F808000, 0x3F818000], dtype=np.uint32).view(np.float32)), [0x3F80, 0x3F82])


def test_workloads_are_reproducible():
    a = inp.make_inputs(inp.WORKLOADS["bertl_kpad_512"])
    b = inp.make_inputs(inp.WORKLOADS["bertl_kpad_512"])
    for x, y in ((a.q, b.q), (a.do, b.do), (a.kv_len, b.kv_len)):
        np.testing.assert_array_equal(x, y)
    assert a.q.shape == (16, 16, 512, 64) and a.q.dtype == np.uint16
    assert a.kv_len.min() >= 128 and a.kv_len.max() <= 512


def test_block_mask_density_and_diagonal():
    wl = inp.WORKLOADS["blocksparse_8k"]
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    m = inp.draw_block_mask(rng, wl.N, wl.density)
    assert m.shape == (64, 64)
    assert m.sum() == 1024
    assert (np.diag(m) == 1).all()


@pytest.mark.parametrize("n", [1, 127, 128, 129, 300])
def test_block_count(n):
    assert inp.n_blocks(n) == -(-n // 128)


def test_scale_is_float32():
    assert inp.WORKLOADS["long_causal_16k"].scale == float(np.float32(1 / np.sqrt(128)))
    assert inp.WORKLOADS["gpt2s_causal_1k"].scale == 0.125
