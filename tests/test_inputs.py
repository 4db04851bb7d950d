"""The seeded input generator: Philox4x32-10 known answers, distributions, shapes."""
import numpy as np
import pytest
import torch

import kda_inputs as K


def test_philox_known_answers():
    # Known-answer vectors published with the Random123 library (Salmon et al., SC'11).
    assert [int(x) for x in K.philox_block([0, 0, 0, 0], [0, 0])] == [0x6627e8d5, 0xe169c58d, 0xbc57ac4c,
                                                                      0x9b00dbd8]
    assert [int(x) for x in K.philox_block([0xffffffff] * 4, [0xffffffff] * 2)] == [0x408f276d, 0x41c83b0e,
                                                                                    0xa20bc7c6, 0x6d5451fd]
    assert [int(x) for x in K.philox_block([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344],
                                           [0xa4093822, 0x299f31d0])] == [0xd16cfe09, 0x94fdcceb, 0x5001e420,
                                                                          0x24126ea1]


def test_stream_layout_and_offsets():
    a = K.raw_u32(5, 3, 40)
    assert np.array_equal(a[8:12], K.philox_block([2, 0, 0, 0], [5, 3]))
    assert np.array_equal(K.raw_u32(5, 3, 13, first=7), a[7:20])
    z = K.normal(5, 3, 41)
    assert np.array_equal(K.normal(5, 3, 10, first=31), z[31:])
    u = K.uniform(5, 3, 41)
    assert np.array_equal(K.uniform(5, 3, 5, first=3), u[3:8])
    assert (u > 0).all() and (u < 1).all()


def test_normal_moments():
    z = K.normal(11, 1, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1) < 5e-3
    assert abs(((z ** 3).mean())) < 1e-2 and abs((z ** 4).mean() - 3) < 3e-2


def test_unit_rows():
    x = K.unit_rows_f32(2, 1, 1000, 128)
    np.testing.assert_allclose(np.linalg.norm(x.astype(np.float64), axis=1), 1.0, atol=1e-6)


def test_bf16_round_to_nearest_even_matches_torch():
    x = np.concatenate([K.normal_f32(1, 9, 100000, scale=3.0),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -1e-40, np.inf, -np.inf],
                                 np.float32)])
    ours = K.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = K.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_small_workload_recipe():
    inp = K.generate(K.workload("chunk_b1_h1_t256_d64_f32"))
    assert inp.q.shape == (256, 1, 64) and inp.q.dtype == np.float32
    assert inp.s0 is None and list(inp.cu_seqlens) == [0, 256]
    assert (inp.g <= 0).all() and (inp.beta > 0).all() and (inp.beta < 1).all()
    again = K.generate(K.workload("chunk_b1_h1_t256_d64_f32"))
    assert np.array_equal(inp.q, again.q) and np.array_equal(inp.g, again.g)


def test_bounds_fraction():
    spec = K.Spec([512], 4, 128, 128, "bf16", "softplus_bounds", 0.05, seed=1)
    inp = K.generate(spec)
    frac_lo = (inp.g == -5.0).mean()
    frac_hi = (inp.g == 0.0).mean()
    assert abs(frac_lo - 0.025) < 0.004 and abs(frac_hi - 0.025) < 0.004
    assert inp.q.dtype == np.uint16


def test_varlen_lengths():
    spec = K.workload("varlen_n32_h16_d128_bf16")
    assert len(spec.lengths) == 32 and min(spec.lengths) >= 64 and max(spec.lengths) <= 16384
    assert spec.packed and spec.s0_std == 0.02


def test_longmem_gate():
    spec = K.Spec([300], 2, 16, 8, "bf16", "longmem", seed=4)
    inp = K.generate(spec)
    assert (inp.g <= 0).all() and (inp.g >= -0.01).all()
