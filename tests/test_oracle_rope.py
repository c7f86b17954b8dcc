"""Pins of the MLA RoPE + FP8 quantize oracle (mla_rope_quantize_fp8 as the MATE
pages describe it).  CPU only."""
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3fn_decode, e4m3fn_encode, mla_rope_quantize_fp8, rope_fp32

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "rope_quantize.py")
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _torch_cast(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_cast_in_range():
    vals = e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                       # every tie between neighbours
    rng = np.random.default_rng(0)
    rand = rng.uniform(-448, 448, 20000) * np.exp2(-rng.integers(0, 14, 20000))
    x = np.concatenate([vals, -vals, mids, -mids, rand, np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    x = x.astype(np.float32)
    assert np.array_equal(e4m3fn_encode(x), _torch_cast(x))


def test_encode_decode_round_trip_and_saturation():
    assert np.array_equal(e4m3fn_encode(e4m3fn_decode(FINITE)), FINITE)
    big = np.array([448.0, 449.0, 464.0, 1e6, -500.0, -3e38], np.float32)
    assert e4m3fn_encode(big).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert e4m3fn_encode(np.array([-0.0, 0.0])).tolist() == [0x80, 0x00]


def test_encode_nan_and_infinities():
    """A NaN value is cast to a NaN code (as torch's float8_e4m3fn cast does, and as the OCP
    format defines 0x7F / 0xFF); infinities saturate to +-448 like any larger magnitude."""
    x = np.array([np.nan, -np.nan, np.inf, -np.inf], np.float32)
    codes = e4m3fn_encode(x)
    assert np.isnan(e4m3fn_decode(codes[:2])).all()
    assert np.isnan(e4m3fn_decode(_torch_cast(x[:2]))).all()
    assert codes[2:].tolist() == [0x7E, 0xFE]


def test_rope_closed_forms():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    one, zero = np.ones((3, 32), np.float32), np.zeros((3, 32), np.float32)
    for neox in (True, False):
        assert np.array_equal(rope_fp32(x, one, zero, neox), x)
    q = rope_fp32(x, zero, one, True)                       # a quarter turn
    assert np.array_equal(q[:, :32], -x[:, 32:]) and np.array_equal(q[:, 32:], x[:, :32])
    q = rope_fp32(x, zero, one, False)
    assert np.array_equal(q[:, 0::2], -x[:, 1::2]) and np.array_equal(q[:, 1::2], x[:, 0::2])


@pytest.mark.parametrize("neox", [True, False])
def test_rope_is_complex_rotation(neox):
    """Pair (a, b) turned by theta is (a + ib) e^{i theta} (float64 textbook form)."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 64)).astype(np.float32)
    theta = rng.uniform(0, 2 * np.pi, (50, 32))
    got = rope_fp32(x, np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32), neox).astype(np.float64)
    a, b = (x[:, :32], x[:, 32:]) if neox else (x[:, 0::2], x[:, 1::2])
    z = (a + 1j * b) * np.exp(1j * theta.astype(np.float32).astype(np.float64))
    ga, gb = (got[:, :32], got[:, 32:]) if neox else (got[:, 0::2], got[:, 1::2])
    np.testing.assert_allclose(ga, z.real, atol=2e-6)
    np.testing.assert_allclose(gb, z.imag, atol=2e-6)


def test_neox_and_interleaved_layouts_are_a_permutation_apart():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    c, s = rng.uniform(-1, 1, (4, 32)).astype(np.float32), rng.uniform(-1, 1, (4, 32)).astype(np.float32)
    perm = np.r_[np.arange(0, 64, 2), np.arange(1, 64, 2)]  # evens first, then odds
    inter = rope_fp32(x, c, s, False)
    assert np.array_equal(rope_fp32(x[:, perm], c, s, True), inter[:, perm])


def _inputs(seed, nnz=5, H=3, max_seq=40, cache_bf16=False):
    rng = np.random.default_rng(seed)
    bf = lambda shape, sc=1.0: torch.from_numpy(rng.standard_normal(shape).astype(np.float32) * sc).bfloat16().float().numpy()
    theta = np.arange(max_seq)[:, None] * (10000.0 ** (-np.arange(32) / 32.0))[None, :]
    cache = np.concatenate([np.cos(theta), np.sin(theta)], axis=1).astype(np.float32)
    if cache_bf16:
        cache = torch.from_numpy(cache).bfloat16().float().numpy()
    pos = rng.integers(0, max_seq, nnz)
    return bf((nnz, H, 64), 4.0), bf((nnz, 64), 4.0), bf((nnz, H, 512), 4.0), bf((nnz, 512), 4.0), cache, pos


@pytest.mark.parametrize("neox", [True, False])
def test_quantized_outputs_within_half_a_step(neox):
    qr, kr, qn, kn, cache, pos = _inputs(4)
    sq, skv = 20.0, 0.75
    outs = mla_rope_quantize_fp8(qr, kr, qn, kn, cache, pos, neox, sq, skv)
    c, s = cache[pos, :32].astype(np.float64), cache[pos, 32:].astype(np.float64)

    def rot(x, c, s):
        x = x.astype(np.float64)
        a, b = (x[..., :32], x[..., 32:]) if neox else (x[..., 0::2], x[..., 1::2])
        out = np.empty_like(x)
        ra, rb = a * c - b * s, b * c + a * s
        if neox:
            out[..., :32], out[..., 32:] = ra, rb
        else:
            out[..., 0::2], out[..., 1::2] = ra, rb
        return out
    exact = [rot(qr, c[:, None], s[:, None]) * sq, rot(kr, c, s) * skv, qn * sq, kn * skv]
    for codes, ref in zip(outs, exact):
        dec = e4m3fn_decode(codes)
        ref = np.clip(ref, -448, 448)
        step = np.where(np.abs(ref) < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 3))
        assert np.all(np.abs(dec - ref) <= step / 2 + 1e-4 * np.abs(ref))


def test_scale_applies_before_the_cast():
    x = np.full((1, 512), 1.1, np.float32)
    z64, z = np.zeros((1, 64), np.float32), np.zeros((1, 1, 64), np.float32)
    cache = np.tile(np.r_[np.ones(32), np.zeros(32)].astype(np.float32), (1, 1))
    _, _, qn, kn = mla_rope_quantize_fp8(z, z64, x[None], x, cache, [0], True, 3.0, 3.0)
    assert qn[0, 0, 0] == e4m3fn_encode(np.float32(3.3))   # 3.3 -> 3.25 (0x45); cast first would give 3.375
    assert e4m3fn_decode(qn[0, 0, :1])[0] == 3.25 and np.array_equal(qn[0, 0], kn[0])


def test_rejects_out_of_range_positions():
    qr, kr, qn, kn, cache, pos = _inputs(5)
    with pytest.raises(ValueError):
        mla_rope_quantize_fp8(qr, kr, qn, kn, cache, np.r_[pos[:-1], 40], True)


# ---- planted mistakes: each must fail at least one pin
MUTATIONS = {
    "sin_sign": ("a_rot = (a * cos) - (b * sin)", "a_rot = (a * cos) + (b * sin)"),
    "layouts_swapped": ("    if is_neox:\n        a, b = x[..., :32], x[..., 32:]", "    if not is_neox:\n        a, b = x[..., :32], x[..., 32:]"),
    "ties_to_odd": ("(hi % 2 == 0)", "(hi % 2 == 1)"),
    "ties_away": ("(d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))", "(d_hi <= d_lo)"),
    "sign_dropped": ("code = code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)", "code = code"),
    "nan_saturated": ("return np.where(nan, np.uint8(0x7F), code).astype(np.uint8)", "return code"),
    "scale_dropped": ("e4m3fn_encode(np.asarray(q_nope, dtype=np.float32) * sq)", "e4m3fn_encode(np.asarray(q_nope, dtype=np.float32))"),
    "cos_sin_swapped": ("cos, sin = cache[pos, :32], cache[pos, 32:]", "cos, sin = cache[pos, 32:], cache[pos, :32]"),
    "kv_scale_for_q": ("q_rot = rope_fp32(q_rope, cos[:, None, :], sin[:, None, :], is_neox)\n    k_rot", "q_rot = rope_fp32(q_rope, cos[:, None, :], sin[:, None, :], is_neox) * (skv / sq)\n    k_rot"),
}


def _mutant(name):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"rope_mutant_{name}")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


PINS = [test_encode_matches_torch_cast_in_range, test_encode_decode_round_trip_and_saturation, test_rope_closed_forms,
        test_encode_nan_and_infinities,
        lambda: test_rope_is_complex_rotation(True), lambda: test_rope_is_complex_rotation(False),
        test_neox_and_interleaved_layouts_are_a_permutation_apart, lambda: test_quantized_outputs_within_half_a_step(True),
        lambda: test_quantized_outputs_within_half_a_step(False), test_scale_applies_before_the_cast]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod = _mutant(name)
    g = globals()
    for f in ("e4m3fn_encode", "rope_fp32", "mla_rope_quantize_fp8"):
        monkeypatch.setitem(g, f, getattr(mod, f))
    caught = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught {name}"
