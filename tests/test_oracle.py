"""Pins of the fp64 oracle against things other than itself.

Each test names what it pins and which plausible mistake it would catch:
brute force on tiny inputs (pure-Python loops, rotation written as complex
multiplication), closed forms worked by hand, invariants of the mathematics,
and independent library routines (torch's scaled_dot_product_attention).
"""
import cmath
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import Rope3D

RNG = np.random.default_rng(1234)


@pytest.fixture(autouse=True)
def _seed_per_test(request):
    """Each test draws from its own stream, seeded by its name, so its inputs do not depend on
    which tests ran before it (test order varies with parallel workers)."""
    global RNG
    RNG = np.random.default_rng(zlib.crc32(request.node.name.encode()))


# ----------------------------------------------------------------------------
# independent helpers (pure Python, no numpy vectorisation, no oracle code)

def _angle(n, p, grid, bands, base, t_offset=0):
    """Angle of pair p at token n, from the stated reading, via exp/log."""
    T, Hg, Wg = grid
    t, rem = divmod(n, Hg * Wg)
    y, x = divmod(rem, Wg)
    pos = (t + t_offset, y, x)
    start = 0
    for band, d in enumerate(bands):
        if p < start + d // 2:
            k = p - start
            return pos[band] * math.exp(-(2.0 * k / d) * math.log(base))
        start += d // 2
    raise AssertionError


def _rotate_complex(vec, n, grid, bands, base, t_offset=0):
    out = []
    for p in range(len(vec) // 2):
        z = complex(vec[2 * p], vec[2 * p + 1]) * cmath.exp(1j * _angle(n, p, grid, bands, base, t_offset))
        out += [z.real, z.imag]
    return out


def _bruteforce_linear(q, k, v, g, grid, bands, base, eps, t_offset=0):
    """Explicit N x N weights form: o_i = sum_j (a_i . c_j) v_j / (sum_j phi(q_i).phi(k_j) + eps)."""
    B, N, H, D = q.shape
    out = np.zeros((B, N, H, D))
    for b in range(B):
        for h in range(H):
            fq = [[max(float(x), 0.0) for x in q[b, i, h]] for i in range(N)]
            fk = [[max(float(x), 0.0) for x in k[b, j, h]] for j in range(N)]
            if grid is None:
                a, c = fq, fk
            else:
                a = [_rotate_complex(fq[i], i, grid, bands, base, t_offset) for i in range(N)]
                c = [_rotate_complex(fk[j], j, grid, bands, base, t_offset) for j in range(N)]
            for i in range(N):
                num = [0.0] * D
                den = 0.0
                for j in range(N):
                    w = sum(a[i][d] * c[j][d] for d in range(D))
                    den += sum(fq[i][d] * fk[j][d] for d in range(D))
                    for e in range(D):
                        num[e] += w * float(v[b, j, h, e])
                for e in range(D):
                    o = num[e] / (den + eps)
                    if g is not None:
                        o *= 1.0 / (1.0 + math.exp(-float(g[b, i, h, e])))
                    out[b, i, h, e] = o
    return out


def _randn(*shape):
    return RNG.standard_normal(shape)


# ----------------------------------------------------------------------------
# RoPE

def test_rope_angles_hand_values():
    """Band offsets/widths, frequency exponent and t-major flattening (reading R1-R4)."""
    grid, bands = (5, 6, 8), (16, 24, 24)
    th = oracle.rope3d_angles(Rope3D(grid, bands))
    n = (3 * 6 + 5) * 8 + 7  # token at t=3, y=5, x=7
    assert th.shape == (5 * 6 * 8, 32)
    assert th[n, 0] == pytest.approx(3.0, abs=1e-15)
    assert th[n, 1] == pytest.approx(3.0 * 10.0 ** -0.5, rel=1e-14)  # 10000^(-2/16)
    assert th[n, 7] == pytest.approx(3.0 * 10.0 ** -3.5, rel=1e-14)  # last t pair: 10000^(-14/16)
    assert th[n, 8] == pytest.approx(5.0, abs=1e-15)  # first h pair
    assert th[n, 9] == pytest.approx(5.0 * 10.0 ** (-1.0 / 3.0), rel=1e-14)  # 10000^(-2/24)
    assert th[n, 20] == pytest.approx(7.0, abs=1e-15)  # first w pair
    assert th[n, 31] == pytest.approx(7.0 * 10.0 ** (-22.0 / 6.0), rel=1e-14)  # 10000^(-22/24)
    # t_offset shifts only the t band
    th2 = oracle.rope3d_angles(Rope3D(grid, bands, t_offset=4))
    assert th2[n, 0] == pytest.approx(7.0)
    assert th2[n, 8] == th[n, 8] and th2[n, 20] == th[n, 20]


def test_rope_rotation_matches_complex_multiplication():
    """Pair layout and rotation sign: x' = x * e^{i theta} on (x_2p, x_2p+1)."""
    grid, bands = (2, 3, 4), (16, 24, 24)
    x = _randn(1, 24, 1, 64)
    th = oracle.rope3d_angles(Rope3D(grid, bands))
    got = oracle.rope3d_rotate(x, th)
    for n in range(24):
        ref = _rotate_complex(list(x[0, n, 0]), n, grid, bands, 10000.0)
        np.testing.assert_allclose(got[0, n, 0], ref, rtol=0, atol=1e-13)


def test_rope_hand_worked_d6():
    """D=6, bands 2/2/2: each band has one pair with frequency 1, so the angle is the coordinate."""
    grid = (2, 2, 2)
    x = np.zeros((1, 8, 1, 6))
    x[..., 0::2] = 1.0  # every pair is the unit vector (1, 0)
    out = oracle.rope3d_rotate(x, oracle.rope3d_angles(Rope3D(grid, (2, 2, 2))))
    # token 6 is (t=1, y=1, x=0): pairs rotate by 1, 1, 0 radians
    np.testing.assert_allclose(out[0, 6, 0], [math.cos(1), math.sin(1), math.cos(1), math.sin(1), 1, 0], atol=1e-15)
    # token 5 is (t=1, y=0, x=1)
    np.testing.assert_allclose(out[0, 5, 0], [math.cos(1), math.sin(1), 1, 0, math.cos(1), math.sin(1)], atol=1e-15)


def test_rope_preserves_norm_and_zero_angle_is_identity():
    x = _randn(2, 60, 3, 64)
    th = oracle.rope3d_angles(Rope3D((3, 4, 5)))
    y = oracle.rope3d_rotate(x, th)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(oracle.rope3d_rotate(x, np.zeros_like(th)), x)


def test_rope_t_only_grid_leaves_h_w_bands():
    x = _randn(1, 7, 2, 64)
    y = oracle.rope3d_rotate(x, oracle.rope3d_angles(Rope3D((7, 1, 1))))
    np.testing.assert_array_equal(y[..., 16:], x[..., 16:])
    assert not np.allclose(y[..., :16], x[..., :16])


# ----------------------------------------------------------------------------
# bidirectional linear attention

@pytest.mark.parametrize("gated", [False, True])
def test_linear_matches_bruteforce_tiny_d6(gated):
    """Factorised form == explicit N x N weight form (pure Python), D=6 bands 2/2/2."""
    grid, bands = (2, 2, 3), (2, 2, 2)
    N = 12
    q, k, v = _randn(1, N, 2, 6), _randn(1, N, 2, 6), _randn(1, N, 2, 6)
    g = _randn(1, N, 2, 6) if gated else None
    got = oracle.linear_attention(q, k, v, g, Rope3D(grid, bands), eps=1e-6)
    ref = _bruteforce_linear(q, k, v, g, grid, bands, 10000.0, 1e-6)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_linear_matches_bruteforce_d64():
    """Same at D=64 with the 16/24/24 split, several heads and a batch of 2."""
    grid = (2, 2, 3)
    q, k, v, g = (_randn(2, 12, 2, 64) for _ in range(4))
    got = oracle.linear_attention(q, k, v, g, Rope3D(grid), eps=1e-6)
    ref = _bruteforce_linear(q, k, v, g, grid, (16, 24, 24), 10000.0, 1e-6)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-13)


def test_linear_matches_nxn_matrix_form_full_f32_case():
    """The fp32 single-head case at full size (N=1024, grid 4x16x16) against the N x N
    matrix form, with RoPE built from complex exponentials (independent of the oracle)."""
    grid, N = (4, 16, 16), 1024
    q, k, v = _randn(1, N, 1, 64), _randn(1, N, 1, 64), _randn(1, N, 1, 64)
    got = oracle.linear_attention(q, k, v, None, Rope3D(grid), eps=1e-6)
    ang = np.array([[_angle(n, p, grid, (16, 24, 24), 10000.0) for p in range(32)] for n in range(N)])
    rot = np.exp(1j * ang)
    fq, fk = np.maximum(q[0, :, 0], 0), np.maximum(k[0, :, 0], 0)
    a = (fq[:, 0::2] + 1j * fq[:, 1::2]) * rot
    c = (fk[:, 0::2] + 1j * fk[:, 1::2]) * rot
    # Re(a . conj? ) -- real dot product of the real-pair vectors: Re(a) Re(c) + Im(a) Im(c)
    W = a.real @ c.real.T + a.imag @ c.imag.T  # (N, N) numerator weights
    den = (fq @ fk.T).sum(axis=1)  # denominator without RoPE
    ref = (W @ v[0, :, 0]) / (den[:, None] + 1e-6)
    np.testing.assert_allclose(got[0, :, 0], ref, rtol=1e-10, atol=1e-14)


def test_linear_no_rope_is_plain_relu_linear_attention():
    q, k, v = _randn(1, 9, 1, 64), _randn(1, 9, 1, 64), _randn(1, 9, 1, 64)
    got = oracle.linear_attention(q, k, v, None, None)
    ref = _bruteforce_linear(q, k, v, None, None, None, None, 1e-6)
    np.testing.assert_allclose(got, ref, rtol=1e-11)


def test_linear_relative_position_invariance():
    """Numerator depends only on position differences; denominator has no RoPE, so a
    global frame shift leaves the bidirectional output unchanged (catches RoPE applied
    with opposite signs to Q and K, or RoPE in the denominator)."""
    q, k, v = _randn(1, 60, 2, 64), _randn(1, 60, 2, 64), _randn(1, 60, 2, 64)
    o0 = oracle.linear_attention(q, k, v, None, Rope3D((3, 4, 5)))
    o7 = oracle.linear_attention(q, k, v, None, Rope3D((3, 4, 5), t_offset=7))
    np.testing.assert_allclose(o7, o0, rtol=1e-9, atol=1e-13)


def test_linear_eps_is_added_not_clamped():
    """N=1, q=k=(s,0,..): den = s^2, num = s^2 v, so o = v s^2/(s^2+eps); with s^2 = eps, o = v/2."""
    s = math.sqrt(1e-6)
    q = np.zeros((1, 1, 1, 64)); q[..., 0] = s
    k = q.copy()
    v = np.arange(64, dtype=np.float64).reshape(1, 1, 1, 64)
    got = oracle.linear_attention(q, k, v, None, Rope3D((1, 1, 1)), eps=1e-6)
    np.testing.assert_allclose(got, v / 2, rtol=1e-12)


def test_linear_zero_feature_row_gives_zero():
    q, k, v = _randn(1, 8, 1, 64), _randn(1, 8, 1, 64), _randn(1, 8, 1, 64)
    q[0, 3] = -np.abs(q[0, 3])  # phi(q_3) = 0
    got = oracle.linear_attention(q, k, v, None, Rope3D((2, 2, 2)))
    assert np.all(got[0, 3] == 0.0)


def test_gate_zero_halves_and_saturates():
    q, k, v = _randn(1, 8, 2, 64), _randn(1, 8, 2, 64), _randn(1, 8, 2, 64)
    base = oracle.linear_attention(q, k, v, None, Rope3D((2, 2, 2)))
    half = oracle.linear_attention(q, k, v, np.zeros_like(q), Rope3D((2, 2, 2)))
    np.testing.assert_array_equal(half, base / 2)
    hi = oracle.linear_attention(q, k, v, np.full_like(q, 60.0), Rope3D((2, 2, 2)))
    lo = oracle.linear_attention(q, k, v, np.full_like(q, -60.0), Rope3D((2, 2, 2)))
    np.testing.assert_allclose(hi, base, rtol=1e-15)
    assert np.abs(lo).max() <= 1e-25 * max(1.0, np.abs(base).max())


def test_linear_rows_and_state():
    q, k, v, g = (_randn(1, 24, 2, 64) for _ in range(4))
    full, kv, ks = oracle.linear_attention(q, k, v, g, Rope3D((2, 3, 4)), return_state=True)
    rows = [0, 5, 23]
    np.testing.assert_array_equal(oracle.linear_attention(q, k, v, g, Rope3D((2, 3, 4)), rows=rows), full[:, rows])
    np.testing.assert_allclose(ks, np.maximum(k, 0).sum(axis=1), rtol=1e-14)
    assert kv.shape == (1, 2, 64, 64)


# ----------------------------------------------------------------------------
# block-causal (chunked) linear attention

def test_chunked_single_chunk_equals_bidirectional():
    q, k, v, g = (_randn(2, 30, 2, 64) for _ in range(4))
    r = Rope3D((5, 2, 3))
    out, kv, ks = oracle.linear_attention_chunked(q, k, v, 30, g, r)
    ref, kv_ref, ks_ref = oracle.linear_attention(q, k, v, g, r, return_state=True)
    # the two forms sum in different orders: fp64 rounding, relative to the output's scale
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13 * np.abs(ref).max())
    np.testing.assert_allclose(kv, kv_ref, rtol=1e-12, atol=1e-13 * np.abs(kv_ref).max())
    np.testing.assert_allclose(ks, ks_ref, rtol=1e-12)
    out2, _, _ = oracle.linear_attention_chunked(q, k, v, 1000, g, r)
    np.testing.assert_allclose(out2, ref, rtol=1e-12, atol=1e-13 * np.abs(ref).max())


def test_chunked_is_prefix_bidirectional():
    """Chunk c's output == bidirectional attention of chunk c's queries over tokens 0..end_c
    (the prefix-sum definition), with ragged last chunk."""
    grid = (7, 2, 3)  # 42 tokens, chunks of 2 frames = 12 tokens -> 12, 12, 12, 6
    N, L = 42, 12
    q, k, v, g = (_randn(1, N, 2, 64) for _ in range(4))
    out, _, _ = oracle.linear_attention_chunked(q, k, v, L, g, Rope3D(grid))
    for start in range(0, N, L):
        stop = min(N, start + L)
        frames = stop // 6
        ref = oracle.linear_attention(q[:, :stop], k[:, :stop], v[:, :stop], g[:, :stop],
                                      Rope3D((frames, 2, 3)), rows=np.arange(start, stop))
        np.testing.assert_allclose(out[:, start:stop], ref, rtol=1e-11, atol=1e-14)


def test_chunked_resume_equals_one_call():
    """Two calls carrying (KV, ksum), the second with t_offset, equal one call."""
    grid = (6, 2, 3)
    q, k, v = (_randn(1, 36, 2, 64) for _ in range(3))
    one, kv1, ks1 = oracle.linear_attention_chunked(q, k, v, 12, None, Rope3D(grid))
    a, kva, ksa = oracle.linear_attention_chunked(q[:, :24], k[:, :24], v[:, :24], 12, None, Rope3D((4, 2, 3)))
    b, kvb, ksb = oracle.linear_attention_chunked(q[:, 24:], k[:, 24:], v[:, 24:], 12, None,
                                                  Rope3D((2, 2, 3), t_offset=4), kv_in=kva, ksum_in=ksa)
    np.testing.assert_allclose(np.concatenate([a, b], axis=1), one, rtol=1e-12)
    np.testing.assert_allclose(kvb, kv1, rtol=1e-12)
    np.testing.assert_allclose(ksb, ks1, rtol=1e-12)


def test_chunked_state_out_independent_of_chunk_size():
    q, k, v = (_randn(1, 40, 1, 64) for _ in range(3))
    r = Rope3D((5, 2, 4))
    _, kv_a, ks_a = oracle.linear_attention_chunked(q, k, v, 3, None, r)
    _, kv_b, ks_b = oracle.linear_attention_chunked(q, k, v, 17, None, r)
    np.testing.assert_allclose(kv_a, kv_b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ks_a, ks_b, rtol=1e-13)


def test_chunk_of_one_is_token_causal_equation():
    """L=1, no RoPE: o_i = phi(q_i)(sum_{j<=i} S_j) / (phi(q_i) sum_{j<=i} phi(k_j) + eps),
    the causal equation with the own term included (pure-Python loops)."""
    N, D = 7, 64
    q, k, v = _randn(1, N, 1, D), _randn(1, N, 1, D), _randn(1, N, 1, D)
    got, _, _ = oracle.linear_attention_chunked(q, k, v, 1, None, None)
    for i in range(N):
        fq = [max(x, 0.0) for x in q[0, i, 0]]
        S = [[0.0] * D for _ in range(D)]
        z = [0.0] * D
        for j in range(i + 1):
            fk = [max(x, 0.0) for x in k[0, j, 0]]
            for d in range(D):
                z[d] += fk[d]
                for e in range(D):
                    S[d][e] += fk[d] * v[0, j, 0, e]
        den = sum(fq[d] * z[d] for d in range(D)) + 1e-6
        ref = [sum(fq[d] * S[d][e] for d in range(D)) / den for e in range(D)]
        np.testing.assert_allclose(got[0, i, 0], ref, rtol=1e-11)


def _bruteforce_causal(q, k, v, g, grid, bands, base, eps, kv_in, ksum_in):
    """o_i = (a_i KV_in + sum_{j<=i} (a_i . c_j) v_j) / (phi(q_i) ksum_in + sum_{j<=i} phi(q_i).phi(k_j) + eps)."""
    B, N, H, D = q.shape
    out = np.zeros((B, N, H, D))
    for b in range(B):
        for h in range(H):
            fq = [[max(float(x), 0.0) for x in q[b, i, h]] for i in range(N)]
            fk = [[max(float(x), 0.0) for x in k[b, j, h]] for j in range(N)]
            a = [_rotate_complex(fq[i], i, grid, bands, base) for i in range(N)]
            c = [_rotate_complex(fk[j], j, grid, bands, base) for j in range(N)]
            for i in range(N):
                num = [sum(a[i][d] * kv_in[b, h, d, e] for d in range(D)) for e in range(D)]
                den = sum(fq[i][d] * ksum_in[b, h, d] for d in range(D))
                for j in range(i + 1):
                    w = sum(a[i][d] * c[j][d] for d in range(D))
                    den += sum(fq[i][d] * fk[j][d] for d in range(D))
                    for e in range(D):
                        num[e] += w * float(v[b, j, h, e])
                for e in range(D):
                    o = num[e] / (den + eps)
                    if g is not None:
                        o *= 1.0 / (1.0 + math.exp(-float(g[b, i, h, e])))
                    out[b, i, h, e] = o
    return out


def test_causal_matches_bruteforce_with_rope_gate_and_state():
    """Token-causal output against pure-Python loops (complex-exponential RoPE,
    carried state added to numerator and denominator); catches a wrong mask
    (j < i instead of j <= i), RoPE on the denominator or a dropped state."""
    grid, bands, D = (3, 1, 3), (2, 2, 4), 8
    B, N, H = 1, 9, 2
    q, k, v, g = (_randn(B, N, H, D) for _ in range(4))
    kv_in = _randn(B, H, D, D)
    ks_in = np.abs(_randn(B, H, D)) * 3
    got, _, _ = oracle.linear_attention_causal(q, k, v, g, Rope3D(grid, bands), kv_in=kv_in, ksum_in=ks_in)
    ref = _bruteforce_causal(q, k, v, g, grid, bands, 10000.0, 1e-6, kv_in, ks_in)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_causal_invariants():
    """The last token sees the whole sequence (equals the bidirectional output);
    the final state is the bidirectional state; outputs do not depend on the
    order rows are asked in; a chunk of one token gives the same outputs."""
    grid = (2, 3, 5)
    B, N, H, D = 2, 30, 2, 64
    q, k, v, g = (_randn(B, N, H, D) for _ in range(4))
    rope = Rope3D(grid)
    out, kv, ks = oracle.linear_attention_causal(q, k, v, g, rope)
    bi, kv_b, ks_b = oracle.linear_attention(q, k, v, g, rope, return_state=True)
    # summed in a different order than the bidirectional form: fp64 rounding at the outputs' scale
    np.testing.assert_allclose(out[:, -1], bi[:, -1], rtol=1e-12, atol=1e-13 * np.abs(bi).max())
    np.testing.assert_allclose(kv, kv_b, rtol=1e-12, atol=1e-13 * np.abs(kv_b).max())
    np.testing.assert_allclose(ks, ks_b, rtol=1e-12)
    rows = [17, 3, 29, 0, 3]
    sel, _, _ = oracle.linear_attention_causal(q, k, v, g, rope, rows=rows)
    np.testing.assert_allclose(sel, out[:, rows], rtol=1e-12)
    kv_in, ks_in = _randn(B, H, D, D), np.abs(_randn(B, H, D))
    c1, kv1, ks1 = oracle.linear_attention_chunked(q, k, v, 1, g, rope, kv_in=kv_in, ksum_in=ks_in)
    c2, kv2, ks2 = oracle.linear_attention_causal(q, k, v, g, rope, kv_in=kv_in, ksum_in=ks_in)
    np.testing.assert_allclose(c2, c1, rtol=1e-11)
    np.testing.assert_allclose(kv2, kv1, rtol=1e-12)
    np.testing.assert_allclose(ks2, ks1, rtol=1e-12)


def _torch_forward(q, k, v, g, grid, bands, base, eps):
    """The bidirectional forward written directly in torch ops (fp64), rotation via cos/sin of
    angles computed here; differentiated by autograd to pin the hand-written backward."""
    B, N, H, D = q.shape
    fq, fk = torch.relu(q), torch.relu(k)
    if grid is None:
        a, c = fq, fk
    else:
        ang = torch.tensor([[_angle(n, p, grid, bands, base) for p in range(D // 2)] for n in range(N)],
                           dtype=torch.float64)
        cos, sin = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]

        def rot(x):
            ev, od = x[..., 0::2], x[..., 1::2]
            return torch.stack([ev * cos - od * sin, ev * sin + od * cos], dim=-1).reshape(x.shape)

        a, c = rot(fq), rot(fk)
    kv = torch.einsum("bnhd,bnhe->bhde", c, v)
    num = torch.einsum("bnhd,bhde->bnhe", a, kv)
    den = torch.einsum("bnhd,bhd->bnh", fq, fk.sum(dim=1))[..., None] + eps
    out = num / den
    return out if g is None else torch.sigmoid(g) * out


@pytest.mark.parametrize("gated,roped", [(True, True), (False, True), (True, False)])
def test_backward_matches_autograd(gated, roped):
    """Hand-derived gradients against torch autograd of an independently written forward;
    catches a dropped term (gate factor, denominator, key sum), a wrong sign or a missing
    inverse rotation."""
    grid, bands = (2, 2, 3), (16, 24, 24)
    B, N, H, D = 2, 12, 2, 64
    q, k, v, g, do = (_randn(B, N, H, D) for _ in range(5))
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, g)]
    out = _torch_forward(ts[0], ts[1], ts[2], ts[3] if gated else None, grid if roped else None, bands, 10000.0, 1e-6)
    out.backward(torch.tensor(do))
    dq, dk, dv, dg = oracle.linear_attention_backward(q, k, v, do, g if gated else None,
                                                      Rope3D(grid, bands) if roped else None)
    for got, ref in ((dq, ts[0].grad), (dk, ts[1].grad), (dv, ts[2].grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-9, atol=1e-12)
    if gated:
        np.testing.assert_allclose(dg, ts[3].grad.numpy(), rtol=1e-9, atol=1e-12)
    else:
        assert dg is None


def test_backward_matches_finite_differences():
    """Central differences of the forward oracle (a scalar loss sum(dO * o)) on a tiny case."""
    grid, bands, D = (2, 1, 3), (2, 2, 4), 8
    B, N, H = 1, 6, 1
    q, k, v, g, do = (_randn(B, N, H, D) for _ in range(5))
    rope = Rope3D(grid, bands)
    dq, dk, dv, dg = oracle.linear_attention_backward(q, k, v, do, g, rope)

    def loss(q_, k_, v_, g_):
        return float(np.sum(do * oracle.linear_attention(q_, k_, v_, g_, rope)))

    h = 1e-6
    for which, grad in enumerate((dq, dk, dv, dg)):
        for idx in np.ndindex(q.shape):
            xs = [q.copy(), k.copy(), v.copy(), g.copy()]
            if which < 2 and abs(xs[which][idx]) < 1e-3:
                continue  # ReLU kink
            xs[which][idx] += h
            up = loss(*xs)
            xs[which][idx] -= 2 * h
            dn = loss(*xs)
            assert abs((up - dn) / (2 * h) - grad[idx]) <= 1e-5 * (1.0 + abs(grad[idx])), (which, idx)


def _torch_chunked_forward(q, k, v, g, kv_in, ks_in, L, grid, bands, base, eps):
    """Block-causal forward in its quadratic masked form (token j reaches token i when
    chunk(j) <= chunk(i)), plus the carried state; returns (out, kv_out, ksum_out)."""
    B, N, H, D = q.shape
    fq, fk = torch.relu(q), torch.relu(k)
    if grid is None:
        a, c = fq, fk
    else:
        ang = torch.tensor([[_angle(n, p, grid, bands, base) for p in range(D // 2)] for n in range(N)],
                           dtype=torch.float64)
        cos, sin = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]

        def rot(x):
            ev, od = x[..., 0::2], x[..., 1::2]
            return torch.stack([ev * cos - od * sin, ev * sin + od * cos], dim=-1).reshape(x.shape)

        a, c = rot(fq), rot(fk)
    blk = torch.arange(N) // L
    mask = (blk[None, :] <= blk[:, None]).to(torch.float64)  # [i, j]
    w_num = torch.einsum("bihd,bjhd->bhij", a, c) * mask
    w_den = torch.einsum("bihd,bjhd->bhij", fq, fk) * mask
    num = torch.einsum("bhij,bjhe->bihe", w_num, v) + torch.einsum("bihd,bhde->bihe", a, kv_in)
    den = w_den.sum(-1).permute(0, 2, 1) + torch.einsum("bihd,bhd->bih", fq, ks_in)
    out = num / (den[..., None] + eps)
    out = out if g is None else torch.sigmoid(g) * out
    kv_out = kv_in + torch.einsum("bnhd,bnhe->bhde", c, v)
    ks_out = ks_in + fk.sum(dim=1)
    return out, kv_out, ks_out


@pytest.mark.parametrize("L,gated,roped", [(5, True, True), (4, False, True), (12, True, False), (1, True, True)])
def test_chunked_backward_matches_autograd(L, gated, roped):
    """Chunked gradients, including those of the carried and returned cache, against autograd
    of the masked quadratic form; catches a prefix taken the wrong way (suffix vs prefix), a
    chunk's own term dropped or the cache gradients left out."""
    grid, bands = (3, 2, 2), (16, 24, 24)
    B, N, H, D = 2, 12, 2, 64
    q, k, v, g, do = (_randn(B, N, H, D) for _ in range(5))
    kv_in, dkv_out = _randn(B, H, D, D), _randn(B, H, D, D)
    ks_in, dks_out = np.abs(_randn(B, H, D)) * 4, _randn(B, H, D)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, g, kv_in, ks_in)]
    out, kv_out, ks_out = _torch_chunked_forward(ts[0], ts[1], ts[2], ts[3] if gated else None, ts[4], ts[5], L,
                                                 grid if roped else None, bands, 10000.0, 1e-6)
    loss = (out * torch.tensor(do)).sum() + (kv_out * torch.tensor(dkv_out)).sum() + \
        (ks_out * torch.tensor(dks_out)).sum()
    loss.backward()
    got = oracle.linear_attention_chunked_backward(q, k, v, do, L, g if gated else None,
                                                   Rope3D(grid, bands) if roped else None, kv_in=kv_in,
                                                   ksum_in=ks_in, dkv_out=dkv_out, dksum_out=dks_out)
    for i, (x, t) in enumerate(zip(got, ts)):
        if i == 3 and not gated:
            assert x is None
            continue
        np.testing.assert_allclose(x, t.grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=str(i))


def test_chunked_backward_matches_finite_differences():
    """Central differences of the chunked forward oracle, cache terms included, on a tiny
    ragged case (7 tokens in chunks of 3)."""
    grid, bands, D = (7, 1, 1), (4, 2, 2), 8
    B, N, H, L = 1, 7, 1, 3
    q, k, v, g, do = (_randn(B, N, H, D) for _ in range(5))
    kv_in, dkv_out = _randn(B, H, D, D), _randn(B, H, D, D)
    ks_in, dks_out = np.abs(_randn(B, H, D)) * 2, _randn(B, H, D)
    rope = Rope3D(grid, bands)
    grads = oracle.linear_attention_chunked_backward(q, k, v, do, L, g, rope, kv_in=kv_in, ksum_in=ks_in,
                                                     dkv_out=dkv_out, dksum_out=dks_out)

    def loss(q_, k_, v_, g_, kv_, ks_):
        o, kvo, kso = oracle.linear_attention_chunked(q_, k_, v_, L, g_, rope, kv_in=kv_, ksum_in=ks_)
        return float(np.sum(do * o) + np.sum(dkv_out * kvo) + np.sum(dks_out * kso))

    h = 1e-6
    base = [q, k, v, g, kv_in, ks_in]
    for which, grad in enumerate(grads):
        for idx in np.ndindex(base[which].shape):
            xs = [x.copy() for x in base]
            if which < 2 and abs(xs[which][idx]) < 1e-3:
                continue  # ReLU kink
            xs[which][idx] += h
            up = loss(*xs)
            xs[which][idx] -= 2 * h
            dn = loss(*xs)
            assert abs((up - dn) / (2 * h) - grad[idx]) <= 1e-5 * (1.0 + abs(grad[idx])), (which, idx)


def test_chunked_backward_one_chunk_is_bidirectional():
    """One chunk and no cache: the chunked gradients reduce to the bidirectional ones."""
    grid, bands = (2, 3, 2), (16, 24, 24)
    q, k, v, g, do = (_randn(2, 12, 2, 64) for _ in range(5))
    rope = Rope3D(grid, bands)
    a = oracle.linear_attention_chunked_backward(q, k, v, do, 12, g, rope)
    b = oracle.linear_attention_backward(q, k, v, do, g, rope)
    for x, y in zip(a[:4], b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


def test_chunked_kv_in_is_added():
    q, k, v = (_randn(1, 6, 1, 64) for _ in range(3))
    kv_in = _randn(1, 1, 64, 64)
    ks_in = np.abs(_randn(1, 1, 64))
    out, kv, ks = oracle.linear_attention_chunked(q, k, v, 6, None, None, kv_in=kv_in, ksum_in=ks_in)
    fq, fk = np.maximum(q[0, :, 0], 0), np.maximum(k[0, :, 0], 0)
    S = kv_in[0, 0] + fk.T @ v[0, :, 0]
    z = ks_in[0, 0] + fk.sum(0)
    np.testing.assert_allclose(out[0, :, 0], (fq @ S) / ((fq @ z)[:, None] + 1e-6), rtol=1e-12)
    np.testing.assert_allclose(kv[0, 0], S, rtol=1e-12)


# ----------------------------------------------------------------------------
# softmax anchor

def test_anchor_matches_python_loops():
    B, N, H, D = 1, 5, 2, 4
    q, k, v, g = (_randn(B, N, H, D) for _ in range(4))
    got = oracle.softmax_anchor(q, k, v, g, scale=0.5)
    for h in range(H):
        for i in range(N):
            ls = [0.5 * sum(q[0, i, h, d] * k[0, j, h, d] for d in range(D)) for j in range(N)]
            m = max(ls)
            e = [math.exp(x - m) for x in ls]
            s = sum(e)
            for c in range(D):
                o = sum(e[j] / s * v[0, j, h, c] for j in range(N))
                o /= 1 + math.exp(-g[0, i, h, c])
                assert got[0, i, h, c] == pytest.approx(o, rel=1e-12, abs=1e-15)


def test_anchor_matches_torch_sdpa_f64():
    """Independent library routine: torch.nn.functional.scaled_dot_product_attention (CPU, fp64)."""
    B, N, H, D = 2, 300, 3, 64
    q, k, v = (_randn(B, N, H, D) for _ in range(3))
    got = oracle.softmax_anchor(q, k, v, None, scale=0.125, row_block=64)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3)))
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=0.125)
    np.testing.assert_allclose(got, ref.numpy().transpose(0, 2, 1, 3), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("gated", [True, False])
def test_anchor_backward_matches_autograd(gated):
    """Hand-derived anchor gradients against torch autograd of an independently written forward
    (softmax over the key axis, sigmoid gate), fp64 on the CPU; row blocks smaller than N so the
    key-side sums run over several blocks."""
    B, N, H, D = 2, 40, 2, 16
    q, k, v, g, do = (_randn(B, N, H, D) for _ in range(5))
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, g)]
    att = torch.softmax(torch.einsum("bihd,bjhd->bhij", ts[0], ts[1]) * 0.3, dim=-1)
    out = torch.einsum("bhij,bjhd->bihd", att, ts[2])
    if gated:
        out = torch.sigmoid(ts[3]) * out
    out.backward(torch.tensor(do))
    got = oracle.softmax_anchor_backward(q, k, v, do, g if gated else None, scale=0.3, row_block=16)
    for x, t in zip(got[:3], ts[:3]):
        np.testing.assert_allclose(x, t.grad.numpy(), rtol=1e-9, atol=1e-12)
    if gated:
        np.testing.assert_allclose(got[3], ts[3].grad.numpy(), rtol=1e-9, atol=1e-12)
    else:
        assert got[3] is None


def test_anchor_backward_matches_finite_differences():
    """Central differences of the forward anchor oracle (loss sum(dO * o)) on a tiny case."""
    B, N, H, D = 1, 5, 1, 4
    q, k, v, g, do = (_randn(B, N, H, D) for _ in range(5))
    grads = oracle.softmax_anchor_backward(q, k, v, do, g, scale=0.7, row_block=2)

    def loss(q_, k_, v_, g_):
        return float(np.sum(do * oracle.softmax_anchor(q_, k_, v_, g_, scale=0.7)))

    h = 1e-6
    for which, grad in enumerate(grads):
        for idx in np.ndindex(q.shape):
            xs = [q.copy(), k.copy(), v.copy(), g.copy()]
            xs[which][idx] += h
            up = loss(*xs)
            xs[which][idx] -= 2 * h
            dn = loss(*xs)
            assert abs((up - dn) / (2 * h) - grad[idx]) <= 1e-6 * (1.0 + abs(grad[idx])), (which, idx)


def test_sparse_anchor_matches_python_loops():
    """Tiny block-sparse case against loops over the allowed keys (query blocks of 4, key blocks of 3)."""
    B, N, H, D = 1, 10, 2, 4
    q, k, v, g = (_randn(B, N, H, D) for _ in range(4))
    # [b][h][query block][entry]; 9, -1 and 7 name nothing (4 key blocks)
    blocks = np.array([[[[2, 0, 9], [1, -1, 7], [3, 0, 0]], [[0, 1, 2], [1, 0, 0], [2, 3, 1]]]])
    counts = np.array([[[3, 3, 1], [0, 1, 3]]])
    got = oracle.softmax_anchor_block_sparse(q, k, v, blocks, counts, g, scale=0.5, q_block=4, k_block=3)
    for h in range(H):
        for i in range(N):
            r = i // 4
            named = {m for m in blocks[0, h, r, :counts[0, h, r]] if 0 <= m < 4}
            keys = [j for j in range(N) if j // 3 in named]
            if not keys:
                assert np.all(got[0, i, h] == 0)
                continue
            ls = [0.5 * sum(q[0, i, h, d] * k[0, j, h, d] for d in range(D)) for j in keys]
            m = max(ls)
            e = [math.exp(x - m) for x in ls]
            for c in range(D):
                o = sum(ej / sum(e) * v[0, j, h, c] for ej, j in zip(e, keys))
                o /= 1 + math.exp(-g[0, i, h, c])
                assert got[0, i, h, c] == pytest.approx(o, rel=1e-12, abs=1e-15)


def test_sparse_anchor_all_blocks_is_dense():
    """Every key block named (any order, plus entries that name nothing) gives the dense anchor."""
    B, N, H, D = 2, 300, 2, 64
    q, k, v, g = (_randn(B, N, H, D) for _ in range(4))
    n_qb, n_kb = 3, 5
    blocks = np.full((B, H, n_qb, n_kb + 2), -1, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for r in range(n_qb):
                blocks[b, h, r, :n_kb + 1] = np.append(RNG.permutation(n_kb), n_kb + 3)
    counts = np.full((B, H, n_qb), n_kb + 2)
    got = oracle.softmax_anchor_block_sparse(q, k, v, blocks, counts, g, scale=0.125)
    np.testing.assert_allclose(got, oracle.softmax_anchor(q, k, v, g, scale=0.125), rtol=1e-10, atol=1e-13)


def test_sparse_anchor_one_block_and_empty():
    """One named block equals the dense anchor over that block's keys; no named block gives zero."""
    B, N, H, D = 1, 200, 1, 64
    q, k, v = (_randn(B, N, H, D) for _ in range(3))
    blocks = np.array([[[[3], [0]]]])  # query block 0 -> keys 192..199 (ragged), block 1 -> keys 0..63
    counts = np.array([[[1, 0]]])
    got = oracle.softmax_anchor_block_sparse(q, k, v, blocks, counts, scale=0.125)
    ref = oracle.softmax_anchor(q, k[:, 192:], v[:, 192:], scale=0.125, rows=np.arange(128))
    np.testing.assert_allclose(got[:, :128], ref, rtol=1e-12, atol=1e-14)
    assert np.all(got[:, 128:] == 0)


def test_anchor_lse_pins():
    """softmax_anchor_lse: zero keys give log N exactly, one key gives scale q.k, and in general it
    equals scipy's logsumexp of the logits; exp(l - lse) rows sum to one and, applied to V,
    reproduce softmax_anchor."""
    from scipy.special import logsumexp

    rng = np.random.default_rng(5)
    B, N, H, D = 2, 37, 3, 16
    q = rng.standard_normal((B, N, H, D)) * 3
    k = rng.standard_normal((B, N, H, D))
    v = rng.standard_normal((B, N, H, D))
    lse = oracle.softmax_anchor_lse(q, np.zeros_like(k), scale=0.25)
    assert np.allclose(lse, np.log(N), rtol=0, atol=1e-14)
    lse1 = oracle.softmax_anchor_lse(q[:, :1], k[:, :1], scale=0.25)
    assert np.allclose(lse1[:, :, 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, 0], k[:, 0]), rtol=0, atol=1e-12)
    lse = oracle.softmax_anchor_lse(q, k, scale=0.25, rows=[0, 5, 36])
    for b in range(B):
        for h in range(H):
            logits = 0.25 * q[b, [0, 5, 36], h] @ k[b, :, h].T
            assert np.allclose(lse[b, h], logsumexp(logits, axis=1), rtol=1e-13, atol=0)
            p = np.exp(logits - lse[b, h][:, None])
            assert np.allclose(p.sum(axis=1), 1.0, atol=1e-13)
            ref = oracle.softmax_anchor(q, k, v, None, 0.25, rows=[0, 5, 36])[b, :, h]
            assert np.allclose(p @ v[b, :, h], ref, atol=1e-12)


def test_anchor_special_cases():
    B, N, H, D = 1, 16, 1, 64
    q, v = _randn(B, N, H, D), _randn(B, N, H, D)
    k_same = np.repeat(_randn(B, 1, H, D), N, axis=1)  # identical keys -> uniform weights
    np.testing.assert_allclose(oracle.softmax_anchor(q, k_same, v)[0, :, 0], np.repeat(v[0, :, 0].mean(0, keepdims=True), N, 0),
                               rtol=1e-12, atol=1e-14)
    k = np.zeros((B, N, H, D)); k[0, 9, 0, 0] = 1.0
    q1 = np.zeros((B, N, H, D)); q1[..., 0] = 1e4  # logit 1250 for key 9, 0 otherwise
    np.testing.assert_allclose(oracle.softmax_anchor(q1, k, v)[0, :, 0], np.repeat(v[0, 9:10, 0], N, 0), rtol=1e-12)
    np.testing.assert_array_equal(oracle.softmax_anchor(q, k, v, np.zeros_like(q)), oracle.softmax_anchor(q, k, v) / 2)
    rows = [3, 11]
    np.testing.assert_array_equal(oracle.softmax_anchor(q, k, v, rows=rows), oracle.softmax_anchor(q, k, v)[:, rows])


# ----------------------------------------------------------------------------
# AttnRes router

def test_route_matches_python_loops():
    B, T, C, S = 2, 3, 8, 3
    vs = [_randn(B, T, C) for _ in range(S)]
    w, phi = _randn(C), _randn(B, C)
    h, alpha = oracle.attnres_route(vs, w, phi, eps=1e-6)
    for b in range(B):
        for t in range(T):
            u = [w[c] + phi[b, c] for c in range(C)]
            ls = []
            for i in range(S):
                ms = sum(vs[i][b, t, c] ** 2 for c in range(C)) / C
                ls.append(sum(u[c] * vs[i][b, t, c] / math.sqrt(ms + 1e-6) for c in range(C)))
            m = max(ls)
            e = [math.exp(x - m) for x in ls]
            a = [x / sum(e) for x in e]
            np.testing.assert_allclose(alpha[b, t], a, rtol=1e-12)
            # h sums signed terms, so its rounding error scales with the terms, not with h
            scale = max(abs(vs[i][b, t, c]) for i in range(S) for c in range(C))
            np.testing.assert_allclose(h[b, t], [sum(a[i] * vs[i][b, t, c] for i in range(S)) for c in range(C)],
                                       rtol=1e-12, atol=1e-14 * scale)


def test_route_hand_worked_two_sources():
    """C=2, u=(1,0): v1=(3,4) -> RMSNorm=(3,4)/sqrt(12.5+eps), v2=(-2,0) -> (-2,0)/sqrt(2+eps)."""
    v1 = np.array([[[3.0, 4.0]]])
    v2 = np.array([[[-2.0, 0.0]]])
    h, alpha = oracle.attnres_route([v1, v2], np.array([1.0, 0.0]), None, eps=1e-6)
    l1 = 3.0 / math.sqrt(12.5 + 1e-6)
    l2 = -2.0 / math.sqrt(2.0 + 1e-6)
    a1 = 1.0 / (1.0 + math.exp(l2 - l1))
    assert alpha[0, 0, 0] == pytest.approx(a1, rel=1e-14)
    np.testing.assert_allclose(h[0, 0], a1 * v1[0, 0] + (1 - a1) * v2[0, 0], rtol=1e-14)


def test_route_invariants():
    B, T, C = 1, 5, 16
    vs = [_randn(B, T, C) for _ in range(4)]
    w, phi = _randn(C), _randn(B, C)
    # a single source is returned unchanged
    h1, a1 = oracle.attnres_route(vs[:1], w, phi)
    np.testing.assert_array_equal(a1, 1.0)
    np.testing.assert_allclose(h1, vs[0], rtol=1e-15)
    # zero query -> uniform weights, h = mean of sources
    h0, a0 = oracle.attnres_route(vs, np.zeros(C), None)
    np.testing.assert_allclose(h0, sum(vs) / 4, rtol=1e-13)
    # weights sum to one; permuting sources permutes alpha and keeps h
    h, a = oracle.attnres_route(vs, w, phi)
    np.testing.assert_allclose(a.sum(-1), 1.0, rtol=1e-14)
    hp, ap = oracle.attnres_route(vs[::-1], w, phi)
    np.testing.assert_allclose(ap, a[..., ::-1], rtol=1e-13)
    np.testing.assert_allclose(hp, h, rtol=1e-12)
    # with eps=0, scaling a source by c>0 leaves alpha unchanged (RMSNorm is scale-free)
    _, a_s = oracle.attnres_route([vs[0] * 7.5] + vs[1:], w, phi, eps=0.0)
    _, a_r = oracle.attnres_route(vs, w, phi, eps=0.0)
    np.testing.assert_allclose(a_s, a_r, rtol=1e-12)
    # phi_t=None equals phi_t = 0
    np.testing.assert_array_equal(oracle.attnres_route(vs, w, None)[0], oracle.attnres_route(vs, w, np.zeros((B, C)))[0])
