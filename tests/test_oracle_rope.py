"""Pins of the RoPE + KV-write oracle against what the mathematics fixes
(closed forms worked by hand, rotation invariants, the relative-position
property), and planted mistakes that those pins must catch.  CPU only."""

import math

import pytest
import torch

import oracle
import oracle.rotary as rope_mod


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64).to(dtype)


def test_worked_example_rotate_half_pairing():
    """D = 4, theta = 100: the pairs are (x0, x2) and (x1, x3), with angles
    pos * 1 and pos * 100^(-1/2) = pos / 10.  Written out by hand for
    x = (1, 2, 3, 4) at position 2; an interleaved pairing, a flipped sign or
    another frequency would give other numbers."""
    x = torch.tensor([[[1.0, 2.0, 3.0, 4.0]]], dtype=torch.float64)
    got = rope_mod.rope(x, [2], theta=100.0)[0, 0]
    a0, a1 = 2.0, 0.2
    want = torch.tensor([1 * math.cos(a0) - 3 * math.sin(a0),
                         2 * math.cos(a1) - 4 * math.sin(a1),
                         3 * math.cos(a0) + 1 * math.sin(a0),
                         4 * math.cos(a1) + 2 * math.sin(a1)], dtype=torch.float64)
    assert torch.allclose(got, want, rtol=0, atol=1e-15)


def test_last_pair_frequency():
    """The last pair (i = D/2 - 1) turns by pos * theta^(-(D-2)/D): for D = 8,
    theta = 10^4 that is pos * 10^-3, so position 1000 turns it by exactly one
    radian, and the unit vector on element 3 (first half of the pair (3, 7))
    goes to cos(1) on element 3 and sin(1) on element 7."""
    x = torch.zeros(1, 1, 8, dtype=torch.float64)
    x[0, 0, 3] = 1.0
    got = rope_mod.rope(x, [1000], theta=1e4)[0, 0]
    want = torch.zeros(8, dtype=torch.float64)
    want[3], want[7] = math.cos(1.0), math.sin(1.0)
    assert torch.allclose(got, want, rtol=0, atol=1e-12)


def test_position_zero_is_identity():
    x = _rand((5, 3, 64), 1)
    assert torch.equal(rope_mod.rope(x, [0] * 5, theta=1e6), x)


def test_pair_norms_preserved():
    x = _rand((7, 4, 128), 2)
    pos = [0, 1, 17, 255, 1024, 7000, 32767]
    y = rope_mod.rope(x, pos, theta=1e6)
    half = 64
    nx = x[..., :half] ** 2 + x[..., half:] ** 2
    ny = y[..., :half] ** 2 + y[..., half:] ** 2
    assert torch.allclose(nx, ny, rtol=1e-12, atol=1e-12)


def test_rotations_compose():
    """Rotating by a then by b equals rotating by a + b (a group action): this
    fixes the sign convention and the per-pair frequencies together."""
    x = _rand((4, 2, 32), 3)
    a, b = [3, 100, 511, 2048], [5, 7, 900, 4000]
    twice = rope_mod.rope(rope_mod.rope(x, a, 1e4), b, 1e4)
    once = rope_mod.rope(x, [i + j for i, j in zip(a, b)], 1e4)
    assert torch.allclose(twice, once, rtol=0, atol=1e-10)


def test_relative_position_property():
    """<rope(q, m), rope(k, n)> depends on m - n only."""
    q = _rand((1, 1, 64), 4)
    k = _rand((1, 1, 64), 5)
    def dot(m, n):
        return float((rope_mod.rope(q, [m], 1e6) * rope_mod.rope(k, [n], 1e6)).sum())
    base = dot(10, 3)
    for shift in (1, 50, 1000, 20000):
        assert abs(dot(10 + shift, 3 + shift) - base) < 1e-9


def test_fused_write_scatters_rotated_k_and_raw_v():
    """q comes back rotated; k lands rotated and v unchanged (same bits) in
    their slots; padded tokens write nothing; every other cache byte (NaN
    payload included) is kept."""
    T, Hq, Hkv, D, B = 5, 4, 2, 16, 4
    qkv = _rand((T, (Hq + 2 * Hkv) * D), 6, torch.bfloat16)
    pos = torch.tensor([0, 3, 9, 4, 40])
    slots = torch.tensor([2, 13, -1, 6, 0])
    kc = torch.full((5, B, Hkv, D), float("nan"), dtype=torch.bfloat16)
    vc = torch.full((5, B, Hkv, D), float("nan"), dtype=torch.bfloat16)
    q_out, kc2, vc2 = rope_mod.fused_rope_kv_write(qkv, pos, slots, kc, vc, Hq, Hkv, theta=1e4)
    rows = qkv.reshape(T, Hq + 2 * Hkv, D)
    assert torch.equal(q_out.view(torch.int16), rope_mod.rope(rows[:, :Hq], pos, 1e4).to(torch.bfloat16).view(torch.int16))
    k_rot = rope_mod.rope(rows[:, Hq:Hq + Hkv], pos, 1e4).to(torch.bfloat16)
    written = set()
    for t in range(T):
        s = int(slots[t])
        if s < 0:
            continue
        written.add((s // B, s % B))
        assert torch.equal(kc2[s // B, s % B].view(torch.int16), k_rot[t].view(torch.int16))
        assert torch.equal(vc2[s // B, s % B].view(torch.int16), rows[t, Hq + Hkv:].view(torch.int16))
    for blk in range(5):
        for off in range(B):
            if (blk, off) not in written:
                assert torch.equal(kc2[blk, off].view(torch.int16), kc[blk, off].view(torch.int16))
                assert torch.equal(vc2[blk, off].view(torch.int16), vc[blk, off].view(torch.int16))
    # position 0 leaves k unrotated: the slot-2 row holds token 0's k bits
    assert torch.equal(kc2[0, 2].view(torch.int16), rows[0, Hq:Hq + Hkv].view(torch.int16))


# ---- planted mistakes: each must make one of the pins above fail ----

def _interleaved(x, positions, theta):
    x = x.to(torch.float64)
    T, H, D = x.shape
    ang = rope_mod.rope_angles(positions, D, theta)
    c = torch.cos(ang).reshape(T, 1, D // 2)
    s = torch.sin(ang).reshape(T, 1, D // 2)
    ev, od = x[..., 0::2], x[..., 1::2]
    out = torch.empty_like(x)
    out[..., 0::2] = ev * c - od * s
    out[..., 1::2] = od * c + ev * s
    return out


def _flipped_sign(x, positions, theta):
    x = x.to(torch.float64)
    T, H, D = x.shape
    half = D // 2
    ang = rope_mod.rope_angles(positions, D, theta)
    c = torch.cos(ang).reshape(T, 1, half)
    s = torch.sin(ang).reshape(T, 1, half)
    lo, hi = x[..., :half], x[..., half:]
    return torch.cat([lo * c + hi * s, hi * c - lo * s], dim=-1)


def _wrong_frequency(positions, head_dim, theta):
    half = head_dim // 2
    pos = torch.as_tensor(positions).to(torch.float64).reshape(-1, 1)
    inv = torch.tensor([theta ** (-1.0 * i / head_dim) for i in range(half)], dtype=torch.float64)
    return pos * inv.reshape(1, -1)


def _position_off_by_one(positions, head_dim, theta):
    half = head_dim // 2
    pos = torch.as_tensor(positions).to(torch.float64).reshape(-1, 1) + 1
    inv = torch.tensor([theta ** (-2.0 * i / head_dim) for i in range(half)], dtype=torch.float64)
    return pos * inv.reshape(1, -1)


MUTANTS = [("rope", _interleaved), ("rope", _flipped_sign), ("rope_angles", _wrong_frequency),
           ("rope_angles", _position_off_by_one)]

PINS = [test_worked_example_rotate_half_pairing, test_last_pair_frequency, test_position_zero_is_identity,
        test_pair_norms_preserved, test_rotations_compose, test_relative_position_property,
        test_fused_write_scatters_rotated_k_and_raw_v]


@pytest.mark.parametrize("attr,mutant", MUTANTS, ids=[m.__name__.lstrip("_") for _, m in MUTANTS])
def test_rope_pins_catch_planted_mistake(monkeypatch, attr, mutant):
    monkeypatch.setattr(rope_mod, attr, mutant)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught the planted mistake in {attr}"


def test_package_exports():
    assert oracle.fused_rope_kv_write is rope_mod.fused_rope_kv_write
