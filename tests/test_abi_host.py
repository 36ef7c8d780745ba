"""Host-side tests of the C ABI: symbols, argument validation, workspace sizes,
RoPE tables. Nothing here launches a kernel or touches a device: every call
either is pure host code or is rejected by validation before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from softmax_attention_relu_amd import hla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation rejects first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hla.LIB_PATH):
        from softmax_attention_relu_amd.build import build

        build()
    return hla.lib()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hla_\w+)\s*\(", src)))


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert len(names) == 23
    assert sorted(hla.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n


def test_noalloc_validation(L):
    assert hla.hla_linear_attn_noalloc_max_workspace() == 64 << 20
    rope = _rope()
    call = L.hla_linear_attn_noalloc
    assert call(0, 1, 8, 1, 64, None, FAKE, FAKE, None, None, 1e-6, FAKE, None) == hla.HLA_ERR_INVALID_ARG
    assert call(0, 1, 8, 1, 32, FAKE, FAKE, FAKE, None, None, 1e-6, FAKE, None) == hla.HLA_ERR_UNSUPPORTED
    assert call(0, 1, 9, 1, 64, FAKE, FAKE, FAKE, None, ctypes.byref(rope), 1e-6, FAKE, None) == \
        hla.HLA_ERR_INVALID_ARG
    # partial sums above the static array: rejected before any device call
    assert hla.hla_linear_attn_workspace(64, 4096, 64, 64) > 64 << 20
    assert call(0, 64, 4096, 64, 64, FAKE, FAKE, FAKE, None, None, 1e-6, FAKE, None) == hla.HLA_ERR_WORKSPACE


def test_status_strings(L):
    for code in range(5):
        assert hla.hla_status_string(code).startswith("HLA_")
    assert "UNKNOWN" in hla.hla_status_string(99)


def test_rope_table_matches_oracle_angles(L):
    grid, bands = (5, 6, 8), (16, 24, 24)
    th = oracle.rope3d_angles(oracle.Rope3D(grid, bands, t_offset=3))
    tt = hla.hla_rope_table_host(5, 3, 16)
    th_t = th[np.arange(5) * 48, :8]  # tokens (t, 0, 0)
    np.testing.assert_allclose(tt[..., 0], np.cos(th_t), atol=1e-7)
    np.testing.assert_allclose(tt[..., 1], np.sin(th_t), atol=1e-7)
    tw = hla.hla_rope_table_host(8, 0, 24)
    np.testing.assert_allclose(tw[..., 0], np.cos(th[:8, 20:]), atol=1e-7)
    np.testing.assert_allclose(tw[..., 1], np.sin(th[:8, 20:]), atol=1e-7)
    # 720p/60s frame range: angles up to 240 rad still rounded from double
    big = hla.hla_rope_table_host(241, 0, 16)
    a = np.arange(241)[:, None] * 10000.0 ** (-2.0 * np.arange(8) / 16)
    np.testing.assert_allclose(big[..., 1], np.sin(a), atol=1e-7)


def test_rope_table_rejects_bad_args(L):
    out = (ctypes.c_float * 16)()
    assert L.hla_rope_table_host(0, 0, 16, 1e4, out) == hla.HLA_ERR_INVALID_ARG
    assert L.hla_rope_table_host(1, 0, 15, 1e4, out) == hla.HLA_ERR_INVALID_ARG
    assert L.hla_rope_table_host(1, 0, 16, 0.0, out) == hla.HLA_ERR_INVALID_ARG
    assert L.hla_rope_table_host(1, 0, 16, 1e4, None) == hla.HLA_ERR_INVALID_ARG


def test_workspace_sizes(L):
    w3 = hla.hla_linear_attn_workspace(1, 75600, 32, 64)
    assert 0 < w3 < 64 << 20  # fp32 partials stay a few percent of the 1.5 GB of tensors
    assert hla.hla_linear_attn_workspace(1, 75600, 32, 32) == 0
    assert hla.hla_linear_attn_workspace(0, 10, 1, 64) == 0
    w5 = hla.hla_linear_attn_chunked_workspace(1, 867600, 32, 64, 36000)
    assert 0 < w5 < 128 << 20
    assert hla.hla_linear_attn_chunked_workspace(1, 100, 1, 64, 0) == 0
    # one chunk covering everything needs the same as the bidirectional call
    assert hla.hla_linear_attn_chunked_workspace(2, 999, 3, 64, 999) == hla.hla_linear_attn_workspace(2, 999, 3, 64)
    wa = hla.hla_softmax_anchor_workspace(1, 75600, 32, 64)
    vt = 32 * 64 * 75648 * 2  # V^T padded to 64 tokens
    blk = -(-32 * (75648 // 64) * 4 // 256) * 256  # one K norm (then one |v| maximum) per 64-key block
    assert wa == -(-vt // 256) * 256 + 2 * blk + vt  # then K in fp16, padded like V^T


def _rope(grid=(2, 2, 2), bands=(16, 24, 24)):
    s = hla.hla_rope3d()
    s.grid_t, s.grid_h, s.grid_w = grid
    s.d_t, s.d_h, s.d_w = bands
    s.cs_t = s.cs_h = s.cs_w = 0x10000
    return s


def _linear(L, dt=0, B=1, N=8, H=1, D=64, q=FAKE, k=FAKE, v=FAKE, o=FAKE, rope=None, eps=1e-6, ws=FAKE,
            ws_bytes=1 << 40):
    return L.hla_linear_attn(dt, B, N, H, D, q, k, v, None, ctypes.byref(rope) if rope else None, eps, o, ws,
                             ws_bytes, None)


def test_linear_validation(L):
    E = hla
    assert _linear(L, q=None) == E.HLA_ERR_INVALID_ARG
    assert _linear(L, o=None) == E.HLA_ERR_INVALID_ARG
    assert _linear(L, N=0) == E.HLA_ERR_INVALID_ARG
    assert _linear(L, B=-1) == E.HLA_ERR_INVALID_ARG
    # (batch, head) pairs index a launch grid dimension: at most 65 535 of them
    assert _linear(L, B=256, H=256) == E.HLA_ERR_INVALID_ARG
    assert _linear(L, B=65536) == E.HLA_ERR_INVALID_ARG
    assert _linear(L, B=5, H=13107, ws=None) == E.HLA_ERR_WORKSPACE  # 65 535 pairs pass the shape check
    assert _linear(L, D=128) == E.HLA_ERR_UNSUPPORTED
    assert _linear(L, dt=7) == E.HLA_ERR_UNSUPPORTED
    assert _linear(L, eps=-1.0) == E.HLA_ERR_INVALID_ARG
    assert _linear(L, eps=float("nan")) == E.HLA_ERR_INVALID_ARG
    assert _linear(L, rope=_rope((2, 2, 3))) == E.HLA_ERR_INVALID_ARG  # grid != N
    assert _linear(L, rope=_rope((2, 2, 2), (15, 25, 24))) == E.HLA_ERR_INVALID_ARG  # odd band
    assert _linear(L, rope=_rope((2, 2, 2), (16, 24, 26))) == E.HLA_ERR_INVALID_ARG  # sum != D
    bad = _rope()
    bad.cs_h = None
    assert _linear(L, rope=bad) == E.HLA_ERR_INVALID_ARG
    assert _linear(L, ws=None) == E.HLA_ERR_WORKSPACE
    need = hla.hla_linear_attn_workspace(1, 8, 1, 64)
    assert _linear(L, rope=_rope(), ws_bytes=need - 1) == E.HLA_ERR_WORKSPACE


def test_chunked_validation(L):
    E = hla

    def call(chunk=4, kv_in=None, ks_in=None, kv_out=None, ks_out=None, ws_bytes=1 << 40, ws=FAKE):
        return L.hla_linear_attn_chunked(0, 1, 8, 1, 64, chunk, FAKE, FAKE, FAKE, None, None, 1e-6, kv_in, ks_in,
                                         kv_out, ks_out, FAKE, ws, ws_bytes, None)

    assert call(chunk=0) == E.HLA_ERR_INVALID_ARG
    assert call(chunk=-3) == E.HLA_ERR_INVALID_ARG
    # one-token chunks of 2^30 tokens and 32 heads: 2^33 work-groups per batch element
    assert L.hla_linear_attn_chunked(0, 1, 1 << 30, 32, 64, 1, FAKE, FAKE, FAKE, None, None, 1e-6, None, None,
                                     None, None, FAKE, FAKE, 1 << 62, None) == E.HLA_ERR_INVALID_ARG
    assert call(kv_in=FAKE) == E.HLA_ERR_INVALID_ARG  # ksum_in missing
    assert call(ks_out=FAKE) == E.HLA_ERR_INVALID_ARG  # kv_out missing
    assert call(ws_bytes=16) == E.HLA_ERR_WORKSPACE


def test_causal_validation(L):
    E = hla

    def call(dt=0, rope=None, kv_in=None, ks_in=None, kv_out=None, ks_out=None, ws_bytes=1 << 40, q=FAKE):
        return L.hla_linear_attn_causal(dt, 1, 8, 1, 64, q, FAKE, FAKE, None, ctypes.byref(rope) if rope else None,
                                        1e-6, kv_in, ks_in, kv_out, ks_out, FAKE, FAKE, ws_bytes, None)

    assert call(q=None) == E.HLA_ERR_INVALID_ARG
    assert call(kv_in=FAKE) == E.HLA_ERR_INVALID_ARG  # ksum_in missing
    assert call(ks_out=FAKE) == E.HLA_ERR_INVALID_ARG  # kv_out missing
    assert call(dt=1) == E.HLA_ERR_UNSUPPORTED  # bf16 only
    assert call(rope=_rope((2, 2, 2), (18, 22, 24))) == E.HLA_ERR_UNSUPPORTED  # band widths not multiples of 8
    assert call(ws_bytes=16) == E.HLA_ERR_WORKSPACE
    assert hla.hla_linear_attn_causal_workspace(1, 75600, 32, 64) > 0
    assert hla.hla_linear_attn_causal_workspace(1, 75600, 32, 48) == 0


def test_backward_validation(L):
    E = hla

    def call(dt=0, rope=None, g=None, dg=None, dO=FAKE, dk=FAKE, ws_bytes=1 << 40, L_=8, kv_in=None, ks_in=None,
             dkv_out=None, dks_out=None, dkv_in=None, dks_in=None, chunked=True):
        if not chunked:
            return L.hla_linear_attn_backward(dt, 1, 8, 1, 64, FAKE, FAKE, FAKE, g,
                                              ctypes.byref(rope) if rope else None, 1e-6, dO, FAKE, dk, FAKE, dg,
                                              FAKE, ws_bytes, None)
        return L.hla_linear_attn_chunked_backward(dt, 1, 8, 1, 64, L_, FAKE, FAKE, FAKE, g,
                                                  ctypes.byref(rope) if rope else None, 1e-6, kv_in, ks_in, dO,
                                                  dkv_out, dks_out, FAKE, dk, FAKE, dg, dkv_in, dks_in, FAKE,
                                                  ws_bytes, None)

    for chunked in (False, True):
        assert call(dO=None, chunked=chunked) == E.HLA_ERR_INVALID_ARG
        assert call(dk=None, chunked=chunked) == E.HLA_ERR_INVALID_ARG
        assert call(g=FAKE, chunked=chunked) == E.HLA_ERR_INVALID_ARG  # gate without dg
        assert call(dg=FAKE, chunked=chunked) == E.HLA_ERR_INVALID_ARG  # dg without gate
        assert call(dt=1, chunked=chunked) == E.HLA_ERR_UNSUPPORTED  # bf16 only
        assert call(rope=_rope((2, 2, 3), (16, 24, 24)), chunked=chunked) == E.HLA_ERR_INVALID_ARG  # grid != N
        assert call(ws_bytes=16, chunked=chunked) == E.HLA_ERR_WORKSPACE
    assert call(L_=0) == E.HLA_ERR_INVALID_ARG
    assert call(kv_in=FAKE) == E.HLA_ERR_INVALID_ARG
    assert call(dks_out=FAKE) == E.HLA_ERR_INVALID_ARG
    assert call(dkv_in=FAKE) == E.HLA_ERR_INVALID_ARG
    # workspace: forward state regions plus bf16 dnum and fp32 dden
    n = hla.hla_linear_attn_backward_workspace(1, 75600, 32, 64)
    assert n >= hla.hla_linear_attn_workspace(1, 75600, 32, 64) + 75600 * 32 * (64 * 2 + 4)
    assert hla.hla_linear_attn_backward_workspace(1, 75600, 32, 48) == 0
    assert hla.hla_linear_attn_chunked_backward_workspace(1, 100, 2, 64, 0) == 0
    assert hla.hla_linear_attn_chunked_backward_workspace(1, 100, 2, 64, 30) > 0


def test_anchor_validation(L):
    E = hla

    def call(dt=0, N=8, D=64, scale=0.125, q=FAKE, ws=FAKE, ws_bytes=1 << 40):
        return L.hla_softmax_anchor(dt, 1, N, 1, D, q, FAKE, FAKE, None, scale, FAKE, ws, ws_bytes, None)

    assert call(q=None) == E.HLA_ERR_INVALID_ARG
    assert call(N=0) == E.HLA_ERR_INVALID_ARG
    assert call(scale=float("inf")) == E.HLA_ERR_INVALID_ARG
    assert call(scale=0.0) == E.HLA_ERR_INVALID_ARG
    assert call(scale=-1.0) == E.HLA_ERR_INVALID_ARG
    assert call(dt=1) == E.HLA_ERR_UNSUPPORTED
    assert call(D=32) == E.HLA_ERR_UNSUPPORTED
    assert call(ws=None) == E.HLA_ERR_WORKSPACE
    assert call(ws_bytes=64 * 64 * 2 - 1) == E.HLA_ERR_WORKSPACE
    assert L.hla_softmax_anchor(0, 2, 8, 32768, 64, FAKE, FAKE, FAKE, None, 0.125, FAKE, FAKE, 1 << 40,
                                None) == E.HLA_ERR_INVALID_ARG  # 65 536 (batch, head) pairs


def test_anchor_backward_validation(L):
    E = hla

    def call(dt=0, N=8, D=64, scale=0.125, g=None, dg=None, dO=FAKE, dq=FAKE, ws_bytes=1 << 40):
        return L.hla_softmax_anchor_backward(dt, 1, N, 1, D, FAKE, FAKE, FAKE, g, scale, dO, dq, FAKE, FAKE, dg,
                                             FAKE, ws_bytes, None)

    assert call(dO=None) == E.HLA_ERR_INVALID_ARG
    assert call(dq=None) == E.HLA_ERR_INVALID_ARG
    assert call(g=FAKE) == E.HLA_ERR_INVALID_ARG
    assert call(dg=FAKE) == E.HLA_ERR_INVALID_ARG
    assert call(scale=-1.0) == E.HLA_ERR_INVALID_ARG
    assert call(N=0) == E.HLA_ERR_INVALID_ARG
    assert call(dt=1) == E.HLA_ERR_UNSUPPORTED
    assert call(D=32) == E.HLA_ERR_UNSUPPORTED
    assert call(ws_bytes=1024) == E.HLA_ERR_WORKSPACE
    # four transposed [64][Npad] copies, dY and two fp32 row vectors
    n = hla.hla_softmax_anchor_backward_workspace(1, 75600, 32, 64)
    assert n >= 4 * 32 * 64 * 75648 * 2 + 75600 * 32 * 64 * 2 + 2 * 75600 * 32 * 4
    assert hla.hla_softmax_anchor_backward_workspace(1, 75600, 32, 48) == 0


def test_anchor_saved_forward_validation(L):
    """The forward that writes row normalisers and the backward from a saved forward reject a missing
    lse or o, then check the rest as their base calls do (no GPU work is reached)."""
    E = hla

    def fwd(lse=FAKE, q=FAKE, dt=0, D=64, ws_bytes=1 << 40):
        return L.hla_softmax_anchor_lse(dt, 1, 8, 1, D, q, FAKE, FAKE, None, 0.125, FAKE, lse, FAKE, ws_bytes, None)

    assert fwd(lse=None) == E.HLA_ERR_INVALID_ARG
    assert fwd(q=None) == E.HLA_ERR_INVALID_ARG
    assert fwd(dt=1) == E.HLA_ERR_UNSUPPORTED
    assert fwd(D=32) == E.HLA_ERR_UNSUPPORTED
    assert fwd(ws_bytes=16) == E.HLA_ERR_WORKSPACE

    def bwd(o=FAKE, lse=FAKE, g=None, dg=None, dO=FAKE, N=8, ws_bytes=1 << 40):
        return L.hla_softmax_anchor_backward_saved(0, 1, N, 1, 64, FAKE, FAKE, FAKE, g, 0.125, o, lse, dO, FAKE, FAKE,
                                                   FAKE, dg, FAKE, ws_bytes, None)

    assert bwd(o=None) == E.HLA_ERR_INVALID_ARG
    assert bwd(lse=None) == E.HLA_ERR_INVALID_ARG
    assert bwd(dO=None) == E.HLA_ERR_INVALID_ARG
    assert bwd(g=FAKE) == E.HLA_ERR_INVALID_ARG
    assert bwd(N=0) == E.HLA_ERR_INVALID_ARG
    assert bwd(ws_bytes=1024) == E.HLA_ERR_WORKSPACE


def test_linear_backward_saved_validation(L):
    """hla_linear_attn_backward_saved rejects a missing kv or ksum before anything else is reached."""
    E = hla

    def call(kv=FAKE, ksum=FAKE, dO=FAKE, ws_bytes=1 << 40):
        return L.hla_linear_attn_backward_saved(0, 1, 8, 1, 64, FAKE, FAKE, FAKE, None, None, 1e-6, kv, ksum, dO,
                                                FAKE, FAKE, FAKE, None, FAKE, ws_bytes, None)

    assert call(kv=None) == E.HLA_ERR_INVALID_ARG
    assert call(ksum=None) == E.HLA_ERR_INVALID_ARG
    assert call(dO=None) == E.HLA_ERR_INVALID_ARG
    assert call(ws_bytes=64) == E.HLA_ERR_WORKSPACE


def test_sparse_anchor_validation(L):
    E = hla

    def call(dt=0, N=8, D=64, scale=0.125, blocks=FAKE, counts=FAKE, max_blocks=4, ws_bytes=1 << 40):
        return L.hla_softmax_anchor_block_sparse(dt, 1, N, 1, D, FAKE, FAKE, FAKE, None, scale, blocks, counts,
                                                 max_blocks, FAKE, FAKE, ws_bytes, None)

    assert call(blocks=None) == E.HLA_ERR_INVALID_ARG
    assert call(counts=None) == E.HLA_ERR_INVALID_ARG
    assert call(max_blocks=0) == E.HLA_ERR_INVALID_ARG
    assert call(scale=0.0) == E.HLA_ERR_INVALID_ARG
    assert call(N=0) == E.HLA_ERR_INVALID_ARG
    assert call(dt=1) == E.HLA_ERR_UNSUPPORTED
    assert call(D=32) == E.HLA_ERR_UNSUPPORTED
    assert call(ws_bytes=64 * 64 * 2 - 1) == E.HLA_ERR_WORKSPACE
    assert call(N=1677312 + 64 * 32) == E.HLA_ERR_UNSUPPORTED  # key-block bitmaps above 16 KB of LDS
    src = open(os.path.join(ROOT, "include", "hla.h")).read()
    assert "#define HLA_SPARSE_Q_BLOCK 128" in src and hla.SPARSE_Q_BLOCK == 128
    assert "#define HLA_SPARSE_K_BLOCK 64" in src and hla.SPARSE_K_BLOCK == 64


def test_route_validation(L):
    E = hla

    def call(S=4, C=2048, srcs=None, w=FAKE, h=FAKE, dt=0, B=1, T=4, eps=1e-6):
        arr = (ctypes.c_void_p * 16)(*([0x10000] * 16)) if srcs is None else srcs
        return L.hla_attnres_route(dt, B, T, C, S, arr, w, None, eps, h, None, None)

    assert call(S=0) == E.HLA_ERR_INVALID_ARG
    assert call(S=17) == E.HLA_ERR_INVALID_ARG
    assert call(C=12) == E.HLA_ERR_INVALID_ARG
    assert call(C=0) == E.HLA_ERR_INVALID_ARG
    assert call(T=0) == E.HLA_ERR_INVALID_ARG
    assert call(w=None) == E.HLA_ERR_INVALID_ARG
    assert call(h=None) == E.HLA_ERR_INVALID_ARG
    assert call(eps=-1.0) == E.HLA_ERR_INVALID_ARG
    holes = (ctypes.c_void_p * 4)(0x10000, None, 0x10000, 0x10000)
    assert call(srcs=holes) == E.HLA_ERR_INVALID_ARG
    assert L.hla_attnres_route(0, 1, 4, 2048, 4, None, FAKE, None, 1e-6, FAKE, None, None) == E.HLA_ERR_INVALID_ARG
    assert call(C=4104) == E.HLA_ERR_UNSUPPORTED
    assert call(dt=5) == E.HLA_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(hla, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(hla, "_lib", None)
    with pytest.raises(ImportError):
        hla.lib()


# ----------------------------------------------------------------------------
# the Python binding checks every tensor before anything reaches the library

class _NoLibrary:
    def __getattr__(self, name):
        raise AssertionError(f"the library was called ({name}) before the argument checks failed")


@pytest.fixture
def no_library(monkeypatch):
    monkeypatch.setattr(hla, "_lib", _NoLibrary())


def _bnhd(*shape, dtype=None):
    torch = pytest.importorskip("torch")
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("case", [
    "k_short", "k_dtype", "g_shape", "o_dtype", "kv_in_shape", "ksum_out_dtype", "anchor_v_shape", "lse_shape",
    "saved_kv_shape", "grad_do_shape", "route_w_dtype", "route_alpha_shape", "route_source_shape", "rope_grid",
])
def test_binding_rejects_mismatched_tensors(no_library, case):
    torch = pytest.importorskip("torch")
    B, N, H, D = 1, 12, 2, 64
    q = _bnhd(B, N, H, D)
    x = _bnhd(B, N, H, D)
    f32 = torch.float32
    with pytest.raises(ValueError) as e:
        if case == "k_short":
            hla.hla_linear_attn(q, _bnhd(B, N - 1, H, D), x)
        elif case == "k_dtype":
            hla.hla_linear_attn(q, _bnhd(B, N, H, D, dtype=f32), x)
        elif case == "g_shape":
            hla.hla_linear_attn(q, x, x, g=_bnhd(B, N, H + 1, D))
        elif case == "o_dtype":
            hla.hla_linear_attn(q, x, x, o=_bnhd(B, N, H, D, dtype=f32))
        elif case == "kv_in_shape":
            hla.hla_linear_attn_chunked(q, x, x, 4, kv_in=torch.zeros(B, H, D), ksum_in=torch.zeros(B, H, D))
        elif case == "ksum_out_dtype":
            hla.hla_linear_attn_chunked(q, x, x, 4, kv_out=torch.zeros(B, H, D, D),
                                        ksum_out=torch.zeros(B, H, D, dtype=torch.float64))
        elif case == "anchor_v_shape":
            hla.hla_softmax_anchor(q, x, _bnhd(B, N + 1, H, D))
        elif case == "lse_shape":
            hla.hla_softmax_anchor_lse(q, x, x, lse=torch.zeros(B, N, H))
        elif case == "saved_kv_shape":
            hla.hla_linear_attn_backward_saved(q, x, x, torch.zeros(B, H, D), torch.zeros(B, H, D), x)
        elif case == "grad_do_shape":
            hla.hla_softmax_anchor_backward(q, x, x, _bnhd(B, N, H, 32))
        elif case == "route_w_dtype":
            srcs = [torch.zeros(B, N, 256, dtype=torch.bfloat16) for _ in range(3)]
            hla.hla_attnres_route(srcs, torch.zeros(256, dtype=torch.bfloat16))
        elif case == "route_alpha_shape":
            srcs = [torch.zeros(B, N, 256, dtype=torch.bfloat16) for _ in range(3)]
            hla.hla_attnres_route(srcs, torch.zeros(256), alpha=torch.zeros(B, N, 4))
        elif case == "route_source_shape":
            srcs = [torch.zeros(B, N, 256, dtype=torch.bfloat16) for _ in range(2)] + \
                   [torch.zeros(B, N - 1, 256, dtype=torch.bfloat16)]
            hla.hla_attnres_route(srcs, torch.zeros(256))
        elif case == "rope_grid":
            tabs = [np.zeros((2, d // 2, 2), np.float32) for d in (16, 24, 24)]
            r = hla.Rope3D((2, 2, 2), device="cpu", tables=tabs)
            hla.hla_linear_attn(q, x, x, rope=r)
    msg = str(e.value)
    assert "device" not in msg, msg  # the shape or dtype check fires first


def test_binding_requires_device_tensors(no_library):
    q = _bnhd(1, 8, 2, 64)
    with pytest.raises(ValueError, match="device tensors"):
        hla.hla_linear_attn(q, q.clone(), q.clone())
