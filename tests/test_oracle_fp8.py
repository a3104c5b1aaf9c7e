"""Pins of the oracle's FP8 decoding (OCP E4M3 values, OCP MX E8M0 scales).

Values the OCP 8-bit floating point format defines by construction (1.0,
448, the smallest subnormal 2^-9, the smallest normal 2^-6, NaN patterns),
every code against torch's float8_e4m3fn decoding (an independent
implementation), and the block structure of the MX scales.
"""
import numpy as np
import torch

from block_sparse_attention_lf_amd import inputs as I
from oracle import lf_oracle as O


def test_e4m3_printed_values():
    v = O.e4m3_decode(np.array([0x00, 0x80, 0x38, 0x40, 0xB8, 0x7E, 0xFE, 0x01, 0x07, 0x08, 0x30], np.uint8))
    np.testing.assert_array_equal(v, [0.0, -0.0, 1.0, 2.0, -1.0, 448.0, -448.0, 2.0 ** -9, 7 * 2.0 ** -9,
                                      2.0 ** -6, 0.5])
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    pos = ours[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0..126 ascend


def test_e8m0_and_block_structure():
    np.testing.assert_array_equal(O.e8m0_decode(np.array([127, 128, 126, 0], np.uint8)), [1.0, 2.0, 0.5, 2.0 ** -127])
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 0x7E, size=(3, 128), dtype=np.uint8)
    sc = np.full((3, 4), 127, np.uint8)
    base = O.mx_dequantize(codes, sc)
    sc[1, 2] = 129  # x4 on channels 64..95 of token 1 only
    got = O.mx_dequantize(codes, sc)
    ratio = np.where(base != 0, got / np.where(base != 0, base, 1), 1.0)
    want = np.ones_like(ratio)
    want[1, 64:96] = 4.0
    np.testing.assert_array_equal(ratio[base != 0], want[base != 0])


def test_quantiser_round_trip_error_is_within_half_an_e4m3_step():
    """(Checks the input preparation used for the FP8 tests.)"""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 6, 128)).astype(np.float32) * np.exp2(rng.integers(-6, 6, (4, 6, 1)))
    codes, scales = I.mx_quantize(x)
    y = O.mx_dequantize(codes, scales)
    blk = np.abs(x.reshape(4, 6, 4, 32)).max(-1, keepdims=True)
    # no clipping: the block maximum stays within 448 after scaling
    assert np.all(blk[..., 0] / O.e8m0_decode(scales) <= 448.0)
    # E4M3 has 3 mantissa bits: relative error <= 2^-4 of the value above the
    # subnormal range, and below it half the subnormal step 2^-9 times the scale
    err = np.abs(y - x).reshape(4, 6, 4, 32)
    step = O.e8m0_decode(scales)[..., None]
    bound = np.maximum(np.abs(x.reshape(4, 6, 4, 32)) * 2.0 ** -4, step * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))


def _torch_e4m3(rng, shape):
    """Random E4M3 codes and their values, decoded by torch's float8_e4m3fn (not by the oracle)."""
    x = torch.from_numpy(rng.standard_normal(shape) * 3.0).to(torch.float8_e4m3fn)
    return x.view(torch.uint8).numpy().copy(), x.to(torch.float64).numpy()


def test_attention_fp8_is_attention_on_the_values_the_codes_stand_for():
    """attention_fp8(codes, scales) = attention(values) where each value is a torch-decoded E4M3 code times
    2^(scale code - 127) of its own 32-channel block. Scales differ per token and per block, and q's differ
    from k's, so using one tensor's scales for the other, a wrong block width, or decoding V as codes all
    change the result; V is passed as plain values."""
    w = I.TINY_FP32.replace(head_dim=64, seed=3)
    x = I.make_inputs(w)
    rng = np.random.default_rng(7)
    q8, qv = _torch_e4m3(rng, x["q"].shape)
    k8, kv = _torch_e4m3(rng, x["k_cache"].shape)
    qs = rng.integers(124, 131, size=x["q"].shape[:-1] + (2,), dtype=np.uint8)
    ks = rng.integers(121, 128, size=x["k_cache"].shape[:-1] + (2,), dtype=np.uint8)
    q_val = qv * np.repeat(np.exp2(qs.astype(np.float64) - 127.0), 32, axis=-1)
    k_val = kv * np.repeat(np.exp2(ks.astype(np.float64) - 127.0), 32, axis=-1)
    c = O.compress(x["q"], x["k_cache"], x["frame_slot"], w.tokens_per_frame, w.block, w.chunk_frames, w.hist_frames)
    s = O.select(c["q_blk"], c["k_blk"], c["k_frm"], w.hist_frames, w.n_sink, w.blocks_per_frame, w.k_frames,
                 w.k_blocks)
    args = (x["v_cache"], x["frame_slot"], s["sel_blocks"], s["n_sel"], w.tokens_per_frame, w.block, w.chunk_frames,
            w.hist_frames, 0.125)
    want = O.attention(q_val, k_val, *args)
    got = O.attention_fp8(q8, qs, k8, ks, *args)
    np.testing.assert_allclose(got["out"], want["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got["lse"], want["lse"], rtol=0, atol=1e-12)
    # the pin has power: the same codes with every q scale one step up is a different attention
    other = O.attention_fp8(q8, qs + 1, k8, ks, *args)
    assert np.abs(other["out"] - want["out"]).max() > 1e-3
