"""Pins of the oracle's 16-bit K/V decoders (``oracle.kv16_ref``) and of the
input encoder in ``workloads`` (CPU only).

The decoders are pinned against values the format definitions fix (bit
patterns worked out by hand from sign / exponent / fraction), against a
library conversion of every one of the 65536 words (NumPy's float16, torch's
bfloat16), and against attention on pages whose values 16 bits store
exactly.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

BF16_KNOWN = [
    (0x3F80, 1.0), (0xC000, -2.0), (0x3E80, 0.25), (0x0000, 0.0), (0x4049, 3.140625),
    (0x0001, 2.0 ** -133),                        # smallest subnormal: 2^-126 * 2^-7
    (0x0080, 2.0 ** -126),                        # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),     # largest finite
    (0x7F80, math.inf), (0xFF80, -math.inf),
]
FP16_KNOWN = [
    (0x3C00, 1.0), (0xC000, -2.0), (0x3555, 0.333251953125), (0x0000, 0.0),
    (0x0001, 2.0 ** -24),                         # smallest subnormal: 2^-14 * 2^-10
    (0x0400, 2.0 ** -14),                         # smallest normal
    (0x7BFF, 65504.0), (0x7C00, math.inf), (0xFC00, -math.inf),
]


@pytest.mark.parametrize("word,value", BF16_KNOWN)
def test_bf16_known_words(word, value):
    assert float(oracle.decode_bf16(np.array([word], np.uint16))[0]) == value


@pytest.mark.parametrize("word,value", FP16_KNOWN)
def test_fp16_known_words(word, value):
    assert float(oracle.decode_fp16(np.array([word], np.uint16))[0]) == value


def test_negative_zero_keeps_its_sign():
    for dec in (oracle.decode_bf16, oracle.decode_fp16):
        z = dec(np.array([0x8000], np.uint16))[0]
        assert z == 0.0 and math.copysign(1.0, float(z)) == -1.0


def test_fp16_all_words_match_numpy():
    words = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_fp16(words)
    want = words.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_bf16_all_words_match_torch():
    words = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bf16(words)
    want = torch.from_numpy(words.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_decode_kv16_dispatch_and_shape():
    w = np.array([[0x3F80, 0x4000], [0x0000, 0xC000]], np.uint16)
    assert oracle.decode_kv16(w, "bf16").shape == (2, 2)
    assert oracle.decode_kv16(w, "bf16")[0, 1] == 2.0
    assert oracle.decode_kv16(w, "fp16")[0, 1] == 2.0
    with pytest.raises(ValueError):
        oracle.decode_kv16(w, "fp8")


@pytest.mark.parametrize("fmt,rel", [("bf16", 2.0 ** -8), ("fp16", 2.0 ** -11)])
def test_encoder_rounds_to_nearest(fmt, rel):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(4096).astype(np.float32)
    y = oracle.decode_kv16(W.encode_kv16(x, fmt), fmt).astype(np.float64)
    # half a unit in the last place of an 8 / 11 significant-bit format
    assert np.all(np.abs(y - x) <= rel * np.abs(x) + 1e-30)


def test_bf16_encoder_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 (even) and 1 + 2^-7: it rounds to 1.0;
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6: it rounds up
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)
    assert list(W.encode_kv16(x, "bf16")) == [0x3F80, 0x3F82]


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_attention_on_exactly_stored_pages(fmt):
    # values that 16 bits hold exactly: attention on the decoded pages is the
    # fp32-input attention on the original values
    w = W.make_random(91, batch=2, qo_max=3, kv_max=40, hkv=2, qhead=2, head_dim=8,
                      page_size=4, pages_per_block=2, topk=3)
    rng = np.random.default_rng(3)
    k = (rng.integers(-8, 9, size=w.k_pages.shape) / 4.0).astype(np.float32)
    v = (rng.integers(-8, 9, size=w.v_pages.shape) / 4.0).astype(np.float32)
    kd = oracle.decode_kv16(W.encode_kv16(k, fmt), fmt)
    vd = oracle.decode_kv16(W.encode_kv16(v, fmt), fmt)
    assert np.array_equal(kd, k) and np.array_equal(vd, v)
    args = (w.selected, w.block_tables, w.cu_seqlens_q, w.used_kv_lens, w.hq, w.hkv,
            w.head_dim, w.block_size, w.page_size, w.softmax_scale, w.causal)
    o1, l1 = oracle.attention_qo_ref(w.q, k, v, *args)
    o2, l2 = oracle.attention_qo_ref(w.q, kd, vd, *args)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
