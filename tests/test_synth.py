"""The seeded input generators: bf16 rounding, determinism, lengths and page tables."""
import hashlib

import numpy as np

from synth import (ATTN_WORKLOADS, DECODE_WORKLOADS, bf16_bits_to_f32, f16_bits_to_f64, f32_to_bf16_bits,
                   f32_to_f16_bits, lengths_to_cu_seqlens, lengths_to_pad_mask, make_attention_inputs,
                   make_decode_inputs, normal_bf16, stream)


def test_bf16_rounding_hand_picked_patterns():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.4028235e38,
                  np.inf, -np.inf, 0.0, -0.0, 1e-40], dtype=np.float32)
    b = f32_to_bf16_bits(f)
    # 1+2^-8 is a tie between 1 and 1+2^-7: ties go to the even mantissa (1.0)
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even is 1+2^-6
    assert list(b[:4]) == [0x3F80, 0x3F80, 0x3F82, 0x3F80]
    assert b[4] == 0xC020
    assert b[5] == 0x7F80            # past the largest bf16 -> +inf
    assert b[6] == 0x7F80 and b[7] == 0xFF80
    assert b[8] == 0x0000 and b[9] == 0x8000
    nan = f32_to_bf16_bits(np.array([np.nan, -np.nan], dtype=np.float32))
    assert (nan & 0x7F80 == 0x7F80).all() and (nan & 0x7F != 0).all()
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    back = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert np.all(np.abs(back - x) <= np.abs(x) * 2 ** -8)


def test_f16_rounding_hand_picked_patterns():
    f = np.array([1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, -2.5, 65504.0, 65520.0, 2.0 ** -24, 2.0 ** -26],
                 dtype=np.float32)
    b = f32_to_f16_bits(f)
    # 1+2^-11 ties between 1 and 1+2^-10 and goes to the even mantissa; 1+3*2^-11 goes up to 1+2^-9
    assert list(b[:3]) == [0x3C00, 0x3C00, 0x3C02]
    assert b[3] == 0xC100
    assert b[4] == 0x7BFF            # largest half
    assert b[5] == 0x7C00            # halfway past it rounds to +inf
    assert b[6] == 0x0001            # smallest subnormal
    assert b[7] == 0x0000            # below half of it: +0
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.all(np.abs(f16_bits_to_f64(f32_to_f16_bits(x)) - x) <= np.abs(x) * 2 ** -11 + 2 ** -25)


def test_generators_are_deterministic_and_streams_independent():
    a = normal_bf16(stream(0, 1, 0), (4, 5))
    b = normal_bf16(stream(0, 1, 0), (4, 5))
    c = normal_bf16(stream(0, 1, 1), (4, 5))
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    w = ATTN_WORKLOADS["tiny_d512"]
    i1, i2 = make_attention_inputs(w, 0), make_attention_inputs(w, 0)
    for key in ("q", "k", "v", "do"):
        assert hashlib.sha256(i1[key].tobytes()).digest() == hashlib.sha256(i2[key].tobytes()).digest()
    assert i1["q"].shape == (1, 128, 2, 512) and i1["k"].shape == (1, 128, 1, 512)


def test_std_of_peaked_draws():
    x = bf16_bits_to_f32(normal_bf16(stream(0, 3, 0), (200000,), std=3.0))
    assert abs(x.std() - 3.0) < 0.05


def test_varlen_metadata():
    w = ATTN_WORKLOADS["varlen_d512"].scaled(S=64, Hq=2, Hkv=1, D=8, len_range=(5, 64))
    inp = make_attention_inputs(w, 0, poison_padding=True)
    L = inp["lengths"]
    assert ((L >= 5) & (L <= 64)).all()
    assert np.array_equal(inp["pad_mask"], lengths_to_pad_mask(L, 64))
    assert np.array_equal(inp["cu_seqlens"], lengths_to_cu_seqlens(L))
    for b, n in enumerate(L):
        assert np.isnan(bf16_bits_to_f32(inp["q"][b, n:])).all()
        assert np.isfinite(bf16_bits_to_f32(inp["q"][b, :n])).all()


def test_page_table_is_a_permutation_over_an_oversized_pool():
    w = DECODE_WORKLOADS["decode_d128"]
    inp = make_decode_inputs(w.scaled(B=8), seed=1)
    ctx, table = inp["ctx_lens"], inp["block_table"]
    pages = -(-ctx // 16)
    used = np.concatenate([table[b, :pages[b]] for b in range(8)])
    assert len(np.unique(used)) == len(used)                     # no page reused
    assert inp["num_pages"] == int(np.ceil(1.5 * pages.sum()))
    assert used.min() >= 0 and used.max() < inp["num_pages"]
    for b in range(8):
        assert (table[b, pages[b]:] == -1).all()
    assert inp["k_cache"].shape == (inp["num_pages"], 16, 8, 128)
