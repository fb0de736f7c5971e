"""C-ABI checks that need no GPU: the library loads, exports every function
include/so2attn.h declares, its host-side edge frame / Wigner-D code agrees
with the oracle, and argument errors come back as status codes before
anything is launched (device pointers are never touched on these paths)."""

import ctypes
import os
import re

import numpy as np
import pytest

import so_equivariant_graph_amd as sea
from oracle import real_sh, so2_weight_count, wigner_d_blocks

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "so2attn.h")
FAKE = ctypes.c_void_p(1 << 30)  # never dereferenced: every call below fails validation first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_0-9]+)\s*\(", text)
    skip = {"if", "sizeof", "defined"}
    return sorted({n for n in names if n not in skip and (n.startswith("so2_") or n == "build_neighbors")})


def test_library_exports_every_declared_function():
    lib = sea.load_library()
    declared = _declared_functions()
    assert "build_neighbors" in declared and "so2_attention_fwd" in declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(sea.EXPORTED_SYMBOLS)


@pytest.mark.parametrize("L", [0, 1, 2, 4, 6])
@pytest.mark.parametrize("C", [1, 16, 128])
def test_weight_count_matches_oracle(L, C):
    assert sea.weight_count(L, C) == so2_weight_count(L, C)


def test_status_strings():
    lib = sea.load_library()
    for code in range(7):
        assert lib.so2_status_string(code).decode().startswith("SO2_")


@pytest.mark.parametrize(
    "rhat",
    [(0.3, -0.2, 0.9), (0.0, 0.0, 1.0), (0.0, 0.0, -1.0), (1e-6, 0.0, -1.0), (-1.0, 0.0, 0.0), (0.0, 1.0, 0.0)],
)
def test_host_edge_frame_and_wigner_match_oracle(rhat):
    L = 6
    R, D = sea.edge_frame_host(L, rhat)
    r = np.asarray(rhat, dtype=np.float64)
    r /= np.linalg.norm(r)
    np.testing.assert_allclose(R @ R.T, np.eye(3), atol=2e-7)
    np.testing.assert_allclose(R @ r, [0, 0, 1], atol=2e-7)
    assert abs(np.linalg.det(R) - 1) < 1e-6
    ref = wigner_d_blocks(L, R)
    for l in range(L + 1):
        np.testing.assert_allclose(D[l], ref[l], atol=2e-6)
    # Lemma 4.1 of the E2Former-V2 summary: in the aligned frame only m = 0 survives
    Y = real_sh(L, r[None])[0]
    for l in range(L + 1):
        v = D[l] @ Y[l * l : (l + 1) ** 2]
        v[l] -= np.sqrt((2 * l + 1) / (4 * np.pi))
        assert np.abs(v).max() < 3e-6


def test_host_edge_frame_random_directions():
    rng = np.random.default_rng(0)
    for _ in range(20):
        r = rng.standard_normal(3)
        R, D = sea.edge_frame_host(4, r)
        ref = wigner_d_blocks(4, R)
        for l in range(5):
            np.testing.assert_allclose(D[l], ref[l], atol=2e-6)


def test_edge_frame_rejects_bad_input():
    lib = sea.load_library()
    z = np.zeros(3, dtype=np.float32)
    out = np.zeros(500, dtype=np.float32)
    assert lib.so2_edge_frame_host(4, z.ctypes.data, out.ctypes.data, out.ctypes.data) == sea.SO2_ERR_INVALID_ARGUMENT
    r = np.ones(3, dtype=np.float32)
    assert lib.so2_edge_frame_host(7, r.ctypes.data, out.ctypes.data, out.ctypes.data) == sea.SO2_ERR_INVALID_ARGUMENT
    assert lib.so2_edge_frame_host(2, None, out.ctypes.data, out.ctypes.data) == sea.SO2_ERR_INVALID_ARGUMENT


def _desc(**kw):
    base = dict(n_atoms=10, n_targets=10, l_max=2, channels=16, heads=2, n_rbf=8,
                envelope_p=5, cutoff=5.0, flags=0, dtype=sea.SO2_FP32)
    base.update(kw)
    return sea.make_desc(**base)


def _fwd(desc, box=None, ws_bytes=None, null=(), stages=None, ptr=None):
    lib = sea.load_library()
    names = ["pos", "box", "row_ptr", "col", "x", "w_q", "w_k", "w_rad", "w_so2", "y", "ws"]
    keep, box_p = sea._host_box(box)
    ptr = ptr or {}
    args = []
    for name in names:
        if name == "box":
            args.append(box_p)
        elif name in null:
            args.append(ctypes.c_void_p(0))
        else:
            args.append(ptr.get(name, FAKE))
    wsb = 0 if ws_bytes is None else ws_bytes
    if stages is None:
        return lib.so2_attention_fwd(ctypes.byref(desc), *args, wsb, ctypes.c_void_p(0))
    return lib.so2_attention_fwd_stages(stages, ctypes.byref(desc), *args, wsb, ctypes.c_void_p(0))


@pytest.mark.parametrize(
    "kw,status",
    [
        (dict(channels=15), sea.SO2_ERR_INVALID_ARGUMENT),  # C % H != 0
        (dict(l_max=7), sea.SO2_ERR_UNSUPPORTED),
        (dict(l_max=-1), sea.SO2_ERR_INVALID_ARGUMENT),
        (dict(n_rbf=1), sea.SO2_ERR_INVALID_ARGUMENT),
        (dict(cutoff=0.0), sea.SO2_ERR_INVALID_ARGUMENT),
        (dict(cutoff=float("nan")), sea.SO2_ERR_INVALID_ARGUMENT),
        (dict(n_targets=11), sea.SO2_ERR_INVALID_ARGUMENT),
        (dict(n_atoms=0, n_targets=0), sea.SO2_ERR_INVALID_ARGUMENT),
        (dict(flags=8), sea.SO2_ERR_INVALID_ARGUMENT),
        (dict(dtype=7), sea.SO2_ERR_INVALID_ARGUMENT),
        (dict(envelope_p=0), sea.SO2_ERR_INVALID_ARGUMENT),
        (dict(channels=512, heads=8), sea.SO2_ERR_UNSUPPORTED),
    ],
)
def test_attention_desc_errors(kw, status):
    d = _desc(**kw)
    assert _fwd(d, ws_bytes=1 << 40) == status
    assert sea.attention_workspace_bytes(d) == 0


def test_attention_pointer_box_and_workspace_errors():
    d = _desc()
    need = sea.attention_workspace_bytes(d)
    assert need > 0
    assert _fwd(d, ws_bytes=need, null=("x",)) == sea.SO2_ERR_INVALID_ARGUMENT
    assert _fwd(d, ws_bytes=need, null=("y",)) == sea.SO2_ERR_INVALID_ARGUMENT
    assert _fwd(d, ws_bytes=need, box=[10.0, 10.0, 10.0]) == sea.SO2_ERR_BOX  # 10 <= 2 * 5
    assert _fwd(d, ws_bytes=need - 1) == sea.SO2_ERR_WORKSPACE
    lib = sea.load_library()
    misaligned = ctypes.c_void_p((1 << 30) + 4)
    args = [FAKE, ctypes.c_void_p(0)] + [FAKE] * 8 + [misaligned]
    assert lib.so2_attention_fwd(ctypes.byref(d), *args, need, ctypes.c_void_p(0)) == sea.SO2_ERR_WORKSPACE


def test_attention_stage_errors():
    d = _desc()
    need = sea.attention_workspace_bytes(d)
    assert _fwd(d, ws_bytes=need, stages=0) == sea.SO2_ERR_INVALID_ARGUMENT
    assert _fwd(d, ws_bytes=need, stages=4) == sea.SO2_ERR_INVALID_ARGUMENT
    # y is not needed by the prologue alone, but by every call with the fused stage
    assert _fwd(d, ws_bytes=need, stages=sea.STAGE_FUSED, null=("y",)) == sea.SO2_ERR_INVALID_ARGUMENT
    assert _fwd(d, ws_bytes=need, stages=sea.STAGE_PREPARE, null=("x",)) == sea.SO2_ERR_INVALID_ARGUMENT
    assert _fwd(d, ws_bytes=need - 1, stages=sea.STAGE_PREPARE, null=("y",)) == sea.SO2_ERR_WORKSPACE


def test_mfma_inputs_must_be_16_byte_aligned():
    d = _desc(l_max=4, channels=128, heads=8, n_rbf=16, dtype=sea.SO2_BF16)
    need = sea.attention_workspace_bytes(d)
    assert need > 0
    odd = ctypes.c_void_p((1 << 30) + 8)
    for name in ("x", "w_rad", "w_so2"):
        assert _fwd(d, ws_bytes=need, ptr={name: odd}) == sea.SO2_ERR_INVALID_ARGUMENT, name


def test_mfma_shape_past_its_atom_limit_is_unsupported():
    # 32-bit offsets into the repacked x: (2^32 - 2^16) / (2 (L+1)(L+2) C) atoms
    for L in (4, 6):
        limit = (2**32 - 2**16 - 1) // (2 * (L + 1) * (L + 2) * 128)
        ok = _desc(n_atoms=limit, n_targets=16, l_max=L, channels=128, heads=8, n_rbf=16, dtype=sea.SO2_BF16)
        assert sea.attention_kernel_kind(ok) == sea.KERNEL_MFMA
        big = _desc(n_atoms=limit + 1, n_targets=16, l_max=L, channels=128, heads=8, n_rbf=16, dtype=sea.SO2_BF16)
        assert sea.attention_kernel_kind(big) == sea.KERNEL_NONE
        assert sea.attention_workspace_bytes(big) == 0
        assert _fwd(big, ws_bytes=1 << 40) == sea.SO2_ERR_UNSUPPORTED
    assert 559_000 < (2**32 - 2**16 - 1) // (2 * 5 * 6 * 128) < 560_000


def test_kernel_kind_selection():
    assert sea.attention_kernel_kind(_desc()) == sea.KERNEL_BATCH
    assert sea.attention_kernel_kind(_desc(l_max=7)) == sea.KERNEL_NONE
    for L in range(1, 7):
        d = _desc(l_max=L, channels=128, heads=8, n_rbf=16, dtype=sea.SO2_BF16)
        assert sea.attention_kernel_kind(d) == sea.KERNEL_MFMA
    assert sea.attention_kernel_kind(_desc(l_max=0, channels=128, heads=8, dtype=sea.SO2_BF16)) == sea.KERNEL_BATCH
    assert sea.attention_kernel_kind(_desc(l_max=6, channels=128, heads=8, dtype=sea.SO2_FP32)) == sea.KERNEL_BATCH


def test_norm_errors_before_launch():
    lib = sea.load_library()
    call = lambda x, g, y, n, L, C, eps, dt: lib.so2_merged_rms_norm(x, g, y, n, L, C, ctypes.c_float(eps), dt, None)
    assert call(None, FAKE, FAKE, 4, 2, 8, 1e-5, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, None, FAKE, 4, 2, 8, 1e-5, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, FAKE, None, 4, 2, 8, 1e-5, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, FAKE, FAKE, -1, 2, 8, 1e-5, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, FAKE, FAKE, 4, -1, 8, 1e-5, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, FAKE, FAKE, 4, 2, 0, 1e-5, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, FAKE, FAKE, 4, 2, 8, -1.0, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, FAKE, FAKE, 4, 2, 8, float("nan"), sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, FAKE, FAKE, 4, 2, 8, 1e-5, 7) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, FAKE, FAKE, 4, 7, 8, 1e-5, sea.SO2_BF16) == sea.SO2_ERR_UNSUPPORTED
    assert call(None, None, None, 0, 2, 8, 1e-5, sea.SO2_FP32) == sea.SO2_OK  # nothing to do


def test_swiglu_errors_before_launch():
    lib = sea.load_library()

    def call(n, L, C, dt, ptrs=(FAKE,) * 6, ws=None, ws_bytes=0):
        return lib.so2_swiglu_s2(*ptrs, n, L, C, dt, ws, ws_bytes, None)

    for stages in (0, 8, 9):
        assert lib.so2_swiglu_s2_stages(stages, *(FAKE,) * 6, 4, 2, 8, sea.SO2_FP32, FAKE, 1 << 30, None) == \
            sea.SO2_ERR_INVALID_ARGUMENT

    for i in range(6):  # x, w_a, w_b, w_g, w_o, y
        ptrs = [FAKE] * 6
        ptrs[i] = None
        assert call(4, 2, 8, sea.SO2_BF16, ptrs) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(-1, 2, 8, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(4, -1, 8, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(4, 2, 0, sea.SO2_BF16) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(4, 2, 8, 7) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(4, 7, 8, sea.SO2_BF16) == sea.SO2_ERR_UNSUPPORTED
    assert call(4, 2, 8, sea.SO2_FP32) == sea.SO2_ERR_WORKSPACE  # no workspace
    need = lib.so2_swiglu_s2_workspace_bytes(4, 2, 8, sea.SO2_FP32)
    assert need >= 3 * 4 * 9 * 8 * 4 + 4 * 8 * 4  # u, v, s and the gate in fp32
    assert call(4, 2, 8, sea.SO2_FP32, ws=FAKE, ws_bytes=need - 1) == sea.SO2_ERR_WORKSPACE
    assert lib.so2_swiglu_s2_workspace_bytes(4, 7, 8, sea.SO2_FP32) == 0
    assert lib.so2_swiglu_s2_workspace_bytes(-1, 2, 8, sea.SO2_FP32) == 0
    assert call(0, 2, 8, sea.SO2_FP32, (None,) * 6) == sea.SO2_OK  # nothing to do


def test_neighbor_errors_before_launch():
    lib = sea.load_library()
    n_e = ctypes.c_int64(0)
    ws = sea.neighbors_workspace_bytes(100)
    assert ws > 0
    call = lambda pos, n, box, rc, rp, col, cap, wsp, wsb: lib.build_neighbors(
        pos, n, None, box, ctypes.c_float(rc), rp, col, cap, ctypes.byref(n_e), wsp, wsb, None
    )
    keep, box_small = sea._host_box([9.0, 20.0, 20.0])
    assert call(None, 100, None, 4.5, FAKE, FAKE, 10, FAKE, ws) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, 0, None, 4.5, FAKE, FAKE, 10, FAKE, ws) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, 100, None, -1.0, FAKE, FAKE, 10, FAKE, ws) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(FAKE, 100, box_small, 4.5, FAKE, FAKE, 10, FAKE, ws) == sea.SO2_ERR_BOX
    assert call(FAKE, 100, None, 4.5, FAKE, FAKE, 10, FAKE, ws - 1) == sea.SO2_ERR_WORKSPACE
    assert call(FAKE, 100, None, 4.5, FAKE, None, 10, FAKE, ws) == sea.SO2_ERR_INVALID_ARGUMENT


def test_host_rotation_generators_match_the_oracle():
    # J_a^l = d/dt D^l(exp(t [e_a]x)) at 0, against central differences of the
    # oracle's quadrature Wigner-D
    from scipy.spatial.transform import Rotation

    L = 6
    J = sea.wigner_generators_host(L)
    h = 1e-5
    for a in range(3):
        e = np.zeros(3)
        e[a] = 1.0
        Dp = wigner_d_blocks(L, Rotation.from_rotvec(h * e).as_matrix())
        Dm = wigner_d_blocks(L, Rotation.from_rotvec(-h * e).as_matrix())
        for l in range(L + 1):
            fd = (Dp[l] - Dm[l]) / (2 * h)
            np.testing.assert_allclose(J[a][l], fd, atol=2e-5)
            np.testing.assert_allclose(J[a][l], -J[a][l].T, atol=1e-5)
    assert sea.load_library().so2_wigner_generators_host(7, None) == sea.SO2_ERR_INVALID_ARGUMENT


def test_backward_errors_before_launch():
    lib = sea.load_library()
    d = _desc()
    need = lib.so2_attention_bwd_workspace_bytes(ctypes.byref(d))
    assert need > 0
    keep, box_p = sea._host_box(None)

    def call(desc, ws_bytes, null=(), box=None):
        keep2, bp = sea._host_box(box)
        names = ["pos", "row_ptr", "col", "x", "w_q", "w_k", "w_rad", "w_so2", "dy", "dx", "dpos", "dw_q", "dw_k",
                 "dw_rad", "dw_so2", "ws"]
        args = [ctypes.c_void_p(0) if n in null else FAKE for n in names]
        return lib.so2_attention_bwd(ctypes.byref(desc), args[0], bp, *args[1:15], args[15], ws_bytes, None)

    assert call(d, need, null=("dy",)) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(d, need, null=("dpos",)) == sea.SO2_ERR_INVALID_ARGUMENT
    assert call(d, need - 1) == sea.SO2_ERR_WORKSPACE
    assert call(d, need, box=[9.0, 9.0, 9.0]) == sea.SO2_ERR_BOX
    assert call(_desc(l_max=7), need) == sea.SO2_ERR_UNSUPPORTED
    big = _desc(l_max=6, channels=512, heads=8)
    assert lib.so2_attention_bwd_workspace_bytes(ctypes.byref(big)) == 0
    assert call(big, 1 << 40) == sea.SO2_ERR_UNSUPPORTED


def test_variant_counts_and_errors():
    lib = sea.load_library()
    for L, C, m, F in ((4, 128, -1, 1), (4, 128, 2, 1), (3, 12, 1, 3), (6, 8, 0, 2)):
        assert lib.so2_weight_count_variant(L, C, m, F) == so2_weight_count(L, C, None if m < 0 else m, F)
    assert lib.so2_weight_count_variant(4, 128, 5, 1) == -1
    assert lib.so2_weight_count_variant(4, 128, 2, 3) == -1  # 3 does not divide 128
    d = _desc()
    bad = [sea.AttnVariant(3, 1), sea.AttnVariant(-2, 1), sea.AttnVariant(-1, 0), sea.AttnVariant(-1, 3)]
    for v in bad:
        assert lib.so2_attention_variant_workspace_bytes(ctypes.byref(d), ctypes.byref(v)) == 0
        args = [FAKE, ctypes.c_void_p(0)] + [FAKE] * 10 + [ctypes.c_void_p(1 << 30)]
        assert lib.so2_attention_fwd_variant(ctypes.byref(d), ctypes.byref(v), *args, 1 << 40, None) == \
            sea.SO2_ERR_INVALID_ARGUMENT
    v = sea.AttnVariant(-1, 2)
    args = [FAKE, ctypes.c_void_p(0)] + [FAKE] * 8 + [ctypes.c_void_p(0)] + [FAKE, ctypes.c_void_p(1 << 30)]
    assert lib.so2_attention_fwd_variant(ctypes.byref(d), ctypes.byref(v), *args, 1 << 40, None) == \
        sea.SO2_ERR_INVALID_ARGUMENT  # w_focus missing
    mf = _desc(l_max=4, channels=128, heads=8, n_rbf=16, dtype=sea.SO2_BF16)
    assert lib.so2_attention_variant_kernel_kind(ctypes.byref(mf), ctypes.byref(sea.AttnVariant(-1, 1))) == \
        sea.KERNEL_MFMA
    # truncated orders run on the MFMA kernel; so do 2, 4 or 8 focus streams
    # with every order at L <= 4 when they hold whole heads; other focus
    # streams on the edge-batch path
    kind = lambda d, m, f: lib.so2_attention_variant_kernel_kind(ctypes.byref(d), ctypes.byref(sea.AttnVariant(m, f)))
    for m in (0, 2, 3):
        assert kind(mf, m, 1) == sea.KERNEL_MFMA
    for f in (2, 4, 8):
        assert kind(mf, -1, f) == sea.KERNEL_MFMA
    assert kind(mf, 2, 2) == sea.KERNEL_BATCH  # focus streams with truncated orders
    assert kind(mf, -1, 16) == sea.KERNEL_BATCH  # 8 channels per stream
    m4 = _desc(l_max=4, channels=128, heads=4, n_rbf=16, dtype=sea.SO2_BF16)
    assert kind(m4, -1, 8) == sea.KERNEL_BATCH  # streams that split a head
    m6 = _desc(l_max=6, channels=128, heads=8, n_rbf=16, dtype=sea.SO2_BF16)
    assert kind(m6, -1, 4) == sea.KERNEL_BATCH  # 32-edge chunks
