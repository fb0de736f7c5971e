"""MI355X (gfx950) on-the-fly SO(2) equivariant graph attention forward.

Thin Python binding over the C ABI in include/so2attn.h (libso2attn.so,
built in-tree by ``so_equivariant_graph_amd.build``).  This module only
marshals arguments: it allocates outputs and workspace with PyTorch, passes
raw device pointers and the current stream, and raises on a non-OK status.
Every step of the computation runs in the HIP library; there is no other
implementation behind these calls, and loading fails loudly when the
library is missing.

    row_ptr, col = build_neighbors(pos, cutoff, box=None, mol_id=None)
    y = so2_attention_fwd(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2,
                          l_max=4, heads=8, cutoff=6.0)
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libso2attn.so")

SO2_OK = 0
SO2_ERR_INVALID_ARGUMENT = 1
SO2_ERR_UNSUPPORTED = 2
SO2_ERR_CAPACITY = 3
SO2_ERR_BOX = 4
SO2_ERR_DEVICE = 5
SO2_ERR_WORKSPACE = 6

SO2_FP32 = 0
SO2_BF16 = 1

FLAG_RBF_ENVELOPE = 1
FLAG_NO_RADIAL = 2

KERNEL_NONE, KERNEL_VALU, KERNEL_MFMA, KERNEL_BATCH = 0, 1, 2, 3

STAGE_PREPARE = 1  # so2_attention_fwd_stages: q/k, statistics, repack, schedule
STAGE_FUSED = 2  # the fused attention kernel
STAGE_SW_MAPS, STAGE_SW_GRID, STAGE_SW_OUT = 1, 2, 4  # so2_swiglu_s2_stages

EXPORTED_SYMBOLS = (
    "so2_status_string",
    "so2_last_device_error",
    "so2_neighbors_workspace_bytes",
    "build_neighbors",
    "so2_weight_count",
    "so2_attention_workspace_bytes",
    "so2_attention_kernel_kind",
    "so2_attention_fwd",
    "so2_attention_fwd_stages",
    "so2_attention_fwd_noalloc",
    "so2_weight_count_variant",
    "so2_attention_variant_workspace_bytes",
    "so2_attention_variant_kernel_kind",
    "so2_attention_fwd_variant",
    "so2_attention_bwd_workspace_bytes",
    "so2_attention_bwd",
    "so2_edge_frame_host",
    "so2_wigner_generators_host",
    "so2_merged_rms_norm",
    "so2_swiglu_s2_workspace_bytes",
    "so2_swiglu_s2",
    "so2_swiglu_s2_stages",
)


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("n_atoms", ctypes.c_int32),
        ("n_targets", ctypes.c_int32),
        ("l_max", ctypes.c_int32),
        ("channels", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("n_rbf", ctypes.c_int32),
        ("envelope_p", ctypes.c_int32),
        ("cutoff", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
    ]


class AttnVariant(ctypes.Structure):
    _fields_ = [("m_max", ctypes.c_int32), ("n_focus", ctypes.c_int32)]


class SO2Error(RuntimeError):
    def __init__(self, status, where, detail=""):
        self.status = status
        msg = f"{where}: {status_string(status)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


_lib_handle = None


def load_library(path: str = LIB_PATH):
    """Load libso2attn.so; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is not None:
        return _lib_handle
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m so_equivariant_graph_amd.build` "
            "(the SO(2) attention path has no other implementation)"
        )
    try:  # bind to the HIP runtime torch already uses, so there is only one
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.so2_status_string.argtypes = [ctypes.c_int]
    lib.so2_status_string.restype = ctypes.c_char_p
    lib.so2_last_device_error.argtypes = []
    lib.so2_last_device_error.restype = ctypes.c_char_p
    lib.so2_neighbors_workspace_bytes.argtypes = [i32]
    lib.so2_neighbors_workspace_bytes.restype = sz
    lib.build_neighbors.argtypes = [vp, i32, vp, vp, f32, vp, vp, i64, ctypes.POINTER(i64), vp, sz, vp]
    lib.build_neighbors.restype = ctypes.c_int
    lib.so2_weight_count.argtypes = [i32, i32]
    lib.so2_weight_count.restype = i64
    lib.so2_attention_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc)]
    lib.so2_attention_workspace_bytes.restype = sz
    lib.so2_attention_kernel_kind.argtypes = [ctypes.POINTER(AttnDesc)]
    lib.so2_attention_kernel_kind.restype = i32
    lib.so2_attention_fwd.argtypes = [ctypes.POINTER(AttnDesc)] + [vp] * 11 + [sz, vp]
    lib.so2_attention_fwd.restype = ctypes.c_int
    lib.so2_attention_fwd_stages.argtypes = [ctypes.c_uint32, ctypes.POINTER(AttnDesc)] + [vp] * 11 + [sz, vp]
    lib.so2_attention_fwd_stages.restype = ctypes.c_int
    lib.so2_attention_fwd_noalloc.argtypes = [ctypes.POINTER(AttnDesc)] + [vp] * 11
    lib.so2_attention_fwd_noalloc.restype = ctypes.c_int
    lib.so2_weight_count_variant.argtypes = [i32, i32, i32, i32]
    lib.so2_weight_count_variant.restype = i64
    lib.so2_attention_variant_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnVariant)]
    lib.so2_attention_variant_workspace_bytes.restype = sz
    lib.so2_attention_variant_kernel_kind.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnVariant)]
    lib.so2_attention_variant_kernel_kind.restype = i32
    lib.so2_attention_fwd_variant.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(AttnVariant)] + [vp] * 13 + [
        sz, vp]
    lib.so2_attention_fwd_variant.restype = ctypes.c_int
    lib.so2_attention_bwd_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc)]
    lib.so2_attention_bwd_workspace_bytes.restype = sz
    lib.so2_attention_bwd.argtypes = [ctypes.POINTER(AttnDesc)] + [vp] * 17 + [sz, vp]
    lib.so2_attention_bwd.restype = ctypes.c_int
    lib.so2_edge_frame_host.argtypes = [i32, vp, vp, vp]
    lib.so2_edge_frame_host.restype = ctypes.c_int
    lib.so2_wigner_generators_host.argtypes = [i32, vp]
    lib.so2_wigner_generators_host.restype = ctypes.c_int
    lib.so2_merged_rms_norm.argtypes = [vp, vp, vp, i32, i32, i32, f32, i32, vp]
    lib.so2_merged_rms_norm.restype = ctypes.c_int
    lib.so2_swiglu_s2_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.so2_swiglu_s2_workspace_bytes.restype = ctypes.c_size_t
    lib.so2_swiglu_s2.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.so2_swiglu_s2.restype = ctypes.c_int
    lib.so2_swiglu_s2_stages.argtypes = [ctypes.c_uint32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp,
                                         ctypes.c_size_t, vp]
    lib.so2_swiglu_s2_stages.restype = ctypes.c_int
    _lib_handle = lib
    return lib


def status_string(status: int) -> str:
    return load_library().so2_status_string(int(status)).decode()


def _check(status, where):
    if status != SO2_OK:
        detail = ""
        if status == SO2_ERR_DEVICE:
            detail = load_library().so2_last_device_error().decode()
        raise SO2Error(status, where, detail)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream_handle(device):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _host_box(box):
    if box is None:
        return None, ctypes.c_void_p(0)
    arr = (ctypes.c_float * 3)(*[float(v) for v in np.asarray(box, dtype=np.float32).reshape(3)])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def weight_count(l_max: int, channels: int) -> int:
    return int(load_library().so2_weight_count(l_max, channels))


def neighbors_workspace_bytes(n_atoms: int) -> int:
    return int(load_library().so2_neighbors_workspace_bytes(n_atoms))


def make_desc(*, n_atoms, n_targets, l_max, channels, heads, n_rbf, envelope_p, cutoff, flags,
              dtype) -> AttnDesc:
    return AttnDesc(
        int(n_atoms), int(n_targets), int(l_max), int(channels), int(heads), int(n_rbf),
        int(envelope_p), float(np.float32(cutoff)), int(flags), int(dtype),
    )


def attention_workspace_bytes(desc: AttnDesc) -> int:
    return int(load_library().so2_attention_workspace_bytes(ctypes.byref(desc)))


def attention_kernel_kind(desc: AttnDesc) -> int:
    return int(load_library().so2_attention_kernel_kind(ctypes.byref(desc)))


def build_neighbors(pos, cutoff, box=None, mol_id=None, capacity=None, workspace=None):
    """Radius graph on the device.  pos: [N,3] float32 CUDA tensor.
    Returns (row_ptr int32 [N+1], col int32 [E]) on pos.device."""
    import torch

    lib = load_library()
    if pos.dtype != torch.float32 or pos.dim() != 2 or pos.shape[1] != 3 or not pos.is_cuda:
        raise ValueError("pos must be a [N,3] float32 CUDA tensor")
    pos = pos.contiguous()
    n = pos.shape[0]
    dev = pos.device
    if mol_id is not None:
        mol_id = mol_id.to(device=dev, dtype=torch.int32).contiguous()
    ws_bytes = lib.so2_neighbors_workspace_bytes(n)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(n + 1, dtype=torch.int32, device=dev)
    cap = int(capacity) if capacity is not None else 96 * n
    keep, box_p = _host_box(box)
    stream = _stream_handle(dev)
    for _ in range(2):
        col = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        n_edges = ctypes.c_int64(0)
        st = lib.build_neighbors(
            _ptr(pos), n, _ptr(mol_id), box_p, ctypes.c_float(float(cutoff)), _ptr(row_ptr),
            _ptr(col), cap, ctypes.byref(n_edges), _ptr(workspace), ws_bytes, stream,
        )
        if st == SO2_ERR_CAPACITY:
            cap = int(n_edges.value)
            continue
        _check(st, "build_neighbors")
        return row_ptr, col[: n_edges.value]
    raise SO2Error(SO2_ERR_CAPACITY, "build_neighbors")


_DTYPES = {}


def _dtype_code(t):
    import torch

    if t.dtype == torch.float32:
        return SO2_FP32
    if t.dtype == torch.bfloat16:
        return SO2_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def so2_attention_fwd(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, *, l_max, heads, cutoff,
                      envelope_p=5, box=None, flags=0, n_targets=None, out=None, workspace=None,
                      stages=STAGE_PREPARE | STAGE_FUSED):
    """Fused SO(2) attention forward.  x: [N,(L+1)^2,C] (float32 or bfloat16);
    the weights share x's dtype.  Returns y [n_targets,(L+1)^2,C] float32.
    `stages` selects the steps (so2_attention_fwd_stages): a FUSED call
    reuses the workspace a PREPARE call with the same arguments filled."""
    import torch

    lib = load_library()
    dt = _dtype_code(x)
    for name, t in (("w_q", w_q), ("w_k", w_k), ("w_rad", w_rad), ("w_so2", w_so2)):
        if t.dtype != x.dtype:
            raise ValueError(f"{name} must have x's dtype {x.dtype}")
    n, nc, C = x.shape
    if nc != (l_max + 1) ** 2:
        raise ValueError("x has the wrong number of irreps components")
    if w_so2.numel() != lib.so2_weight_count(l_max, C):
        raise ValueError("w_so2 has the wrong number of entries")
    if w_rad.dim() != 2 or w_rad.shape[1] != C:
        raise ValueError("w_rad must be [K, C]")
    nt = n if n_targets is None else int(n_targets)
    tensors = [t.contiguous() for t in (pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2)]
    pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2 = tensors
    desc = make_desc(
        n_atoms=n, n_targets=nt, l_max=l_max, channels=C, heads=heads, n_rbf=w_rad.shape[0],
        envelope_p=envelope_p, cutoff=cutoff, flags=flags, dtype=dt,
    )
    ws_bytes = lib.so2_attention_workspace_bytes(ctypes.byref(desc))
    if ws_bytes == 0:
        st = lib.so2_attention_fwd(ctypes.byref(desc), *([ctypes.c_void_p(0)] * 11), 0, ctypes.c_void_p(0))
        _check(st if st != SO2_OK else SO2_ERR_INVALID_ARGUMENT, "so2_attention_fwd")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    y = out if out is not None else torch.empty((nt, nc, C), dtype=torch.float32, device=x.device)
    keep, box_p = _host_box(box)
    col_arg = col if col.numel() > 0 else row_ptr  # any valid device pointer when E = 0
    st = lib.so2_attention_fwd_stages(
        int(stages), ctypes.byref(desc), _ptr(pos), box_p, _ptr(row_ptr), _ptr(col_arg), _ptr(x),
        _ptr(w_q), _ptr(w_k), _ptr(w_rad), _ptr(w_so2), _ptr(y), _ptr(workspace), ws_bytes,
        _stream_handle(x.device),
    )
    _check(st, "so2_attention_fwd")
    return y


def so2_attention_fwd_variant(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, *, l_max, heads, cutoff, envelope_p=5,
                              box=None, flags=0, n_targets=None, m_max=-1, n_focus=1, w_logit=None, w_focus=None,
                              out=None, workspace=None):
    """so2_attention_fwd with the variants of so2_attention_fwd_variant:
    truncated orders (m_max), F focus streams with w_focus [C], and a radial
    logit bias w_logit [K, H] (each in x's dtype)."""
    import torch

    lib = load_library()
    dt = _dtype_code(x)
    n, nc, C = x.shape
    nt = n if n_targets is None else int(n_targets)
    for name, t in (("w_logit", w_logit), ("w_focus", w_focus)):
        if t is not None and t.dtype != x.dtype:
            raise ValueError(f"{name} must have x's dtype {x.dtype}")
    want = lib.so2_weight_count_variant(l_max, C, m_max, n_focus)
    if w_so2.numel() != want:
        raise ValueError(f"w_so2 has {w_so2.numel()} entries, the variant needs {want}")
    tensors = [None if t is None else t.contiguous()
               for t in (pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, w_logit, w_focus)]
    pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, w_logit, w_focus = tensors
    desc = make_desc(n_atoms=n, n_targets=nt, l_max=l_max, channels=C, heads=heads, n_rbf=w_rad.shape[0],
                     envelope_p=envelope_p, cutoff=cutoff, flags=flags, dtype=dt)
    var = AttnVariant(int(m_max), int(n_focus))
    ws_bytes = lib.so2_attention_variant_workspace_bytes(ctypes.byref(desc), ctypes.byref(var))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    y = out if out is not None else torch.empty((nt, nc, C), dtype=torch.float32, device=x.device)
    keep, box_p = _host_box(box)
    col_arg = col if col.numel() > 0 else row_ptr
    st = lib.so2_attention_fwd_variant(
        ctypes.byref(desc), ctypes.byref(var), _ptr(pos), box_p, _ptr(row_ptr), _ptr(col_arg), _ptr(x), _ptr(w_q),
        _ptr(w_k), _ptr(w_rad), _ptr(w_so2), _ptr(w_logit), _ptr(w_focus), _ptr(y), _ptr(workspace), ws_bytes,
        _stream_handle(x.device),
    )
    _check(st, "so2_attention_fwd_variant")
    return y


def so2_attention_bwd(pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, dy, *, l_max, heads, cutoff, envelope_p=5,
                      box=None, flags=0, n_targets=None, weights=True, workspace=None):
    """Gradients of a loss with upstream gradient dy through so2_attention_fwd
    (same arguments).  Returns a dict of float32 tensors: dx, dpos and, with
    weights=True, dw_q, dw_k, dw_rad, dw_so2."""
    import torch

    lib = load_library()
    dt = _dtype_code(x)
    n, nc, C = x.shape
    nt = n if n_targets is None else int(n_targets)
    if tuple(dy.shape) != (nt, nc, C) or dy.dtype != torch.float32:
        raise ValueError("dy must be float32 [n_targets, (L+1)^2, C]")
    tensors = [t.contiguous() for t in (pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, dy)]
    pos, row_ptr, col, x, w_q, w_k, w_rad, w_so2, dy = tensors
    desc = make_desc(n_atoms=n, n_targets=nt, l_max=l_max, channels=C, heads=heads, n_rbf=w_rad.shape[0],
                     envelope_p=envelope_p, cutoff=cutoff, flags=flags, dtype=dt)
    ws_bytes = lib.so2_attention_bwd_workspace_bytes(ctypes.byref(desc))
    if ws_bytes == 0:
        _check(SO2_ERR_UNSUPPORTED if l_max <= 6 else SO2_ERR_INVALID_ARGUMENT, "so2_attention_bwd")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    f32 = dict(dtype=torch.float32, device=x.device)
    out = {"dx": torch.empty((n, nc, C), **f32), "dpos": torch.empty((n, 3), **f32)}
    if weights:
        out.update(dw_q=torch.empty((C, C), **f32), dw_k=torch.empty((C, C), **f32),
                   dw_rad=torch.empty(tuple(w_rad.shape), **f32), dw_so2=torch.empty(w_so2.numel(), **f32))
    keep, box_p = _host_box(box)
    col_arg = col if col.numel() > 0 else row_ptr
    st = lib.so2_attention_bwd(
        ctypes.byref(desc), _ptr(pos), box_p, _ptr(row_ptr), _ptr(col_arg), _ptr(x), _ptr(w_q), _ptr(w_k),
        _ptr(w_rad), _ptr(w_so2), _ptr(dy), _ptr(out["dx"]), _ptr(out["dpos"]), _ptr(out.get("dw_q")),
        _ptr(out.get("dw_k")), _ptr(out.get("dw_rad")), _ptr(out.get("dw_so2")), _ptr(workspace), ws_bytes,
        _stream_handle(x.device),
    )
    _check(st, "so2_attention_bwd")
    return out


def merged_rms_norm(x, gamma, *, eps=1e-5, out=None):
    """Merged RMS layer norm: one RMS statistic per node over every degree,
    gain gamma [L+1, C] (float32) per degree and channel.  x: [N,(L+1)^2,C]
    float32 or bfloat16; returns y of x's shape and dtype (out may be x)."""
    import torch

    lib = load_library()
    dt = _dtype_code(x)
    n, nc, C = x.shape
    L = int(round(nc ** 0.5)) - 1
    if (L + 1) ** 2 != nc:
        raise ValueError("x has the wrong number of irreps components")
    if gamma.dtype != torch.float32 or tuple(gamma.shape) != (L + 1, C):
        raise ValueError("gamma must be float32 [L+1, C]")
    x, gamma = x.contiguous(), gamma.contiguous()
    y = out if out is not None else torch.empty_like(x)
    st = lib.so2_merged_rms_norm(_ptr(x), _ptr(gamma), _ptr(y), n, L, C, ctypes.c_float(eps), dt,
                                 _stream_handle(x.device))
    _check(st, "so2_merged_rms_norm")
    return y


def edge_frame_host(l_max: int, rhat):
    """CPU evaluation of the kernels' edge frame and Wigner-D code (fp32).
    Returns (R [3,3], [D^0..D^L])."""
    lib = load_library()
    r = np.ascontiguousarray(np.asarray(rhat, dtype=np.float32).reshape(3))
    R = np.zeros(9, dtype=np.float32)
    total = sum((2 * l + 1) ** 2 for l in range(l_max + 1))
    D = np.zeros(total, dtype=np.float32)
    st = lib.so2_edge_frame_host(l_max, r.ctypes.data, R.ctypes.data, D.ctypes.data)
    _check(st, "so2_edge_frame_host")
    blocks, off = [], 0
    for l in range(l_max + 1):
        n = 2 * l + 1
        blocks.append(D[off : off + n * n].reshape(n, n).astype(np.float64))
        off += n * n
    return R.reshape(3, 3).astype(np.float64), blocks


def wigner_generators_host(l_max: int):
    """The backward's rotation generators (CPU, same code): [3][l] blocks."""
    lib = load_library()
    total = sum((2 * l + 1) ** 2 for l in range(l_max + 1))
    J = np.zeros(3 * total, dtype=np.float32)
    _check(lib.so2_wigner_generators_host(l_max, J.ctypes.data), "so2_wigner_generators_host")
    out = []
    for a in range(3):
        blocks, off = [], a * total
        for l in range(l_max + 1):
            n = 2 * l + 1
            blocks.append(J[off : off + n * n].reshape(n, n).astype(np.float64))
            off += n * n
        out.append(blocks)
    return out


__all__ = [
    "build_neighbors",
    "so2_attention_fwd",
    "edge_frame_host",
    "weight_count",
    "neighbors_workspace_bytes",
    "attention_workspace_bytes",
    "attention_kernel_kind",
    "make_desc",
    "load_library",
    "SO2Error",
    "AttnDesc",
]


def swiglu_s2(x, w_a, w_b, w_g, w_o, *, out=None, workspace=None,
              stages=STAGE_SW_MAPS | STAGE_SW_GRID | STAGE_SW_OUT):
    """SwiGLU-S2 activation of node features.  x: [N,(L+1)^2,C] float32 or
    bfloat16; w_a, w_b, w_o: [L+1,C,C] ([l][in][out]) and w_g: [C,C] in x's
    dtype.  Returns y [N,(L+1)^2,C] float32.  `stages` selects the steps
    (so2_swiglu_s2_stages), which pass their results through `workspace`."""
    import torch

    lib = load_library()
    dt = _dtype_code(x)
    n, nc, C = x.shape
    L = int(round(nc ** 0.5)) - 1
    if (L + 1) ** 2 != nc:
        raise ValueError("x must be [N,(L+1)^2,C]")
    for name, t, shape in (("w_a", w_a, (L + 1, C, C)), ("w_b", w_b, (L + 1, C, C)), ("w_o", w_o, (L + 1, C, C)),
                           ("w_g", w_g, (C, C))):
        if t.dtype != x.dtype:
            raise ValueError(f"{name} must have x's dtype {x.dtype}")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {list(shape)}")
    x, w_a, w_b, w_g, w_o = (t.contiguous() for t in (x, w_a, w_b, w_g, w_o))
    ws_bytes = lib.so2_swiglu_s2_workspace_bytes(n, L, C, dt)
    if ws_bytes == 0 and n > 0:
        _check(SO2_ERR_UNSUPPORTED if L > 6 else SO2_ERR_INVALID_ARGUMENT, "so2_swiglu_s2")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    y = out if out is not None else torch.empty((n, nc, C), dtype=torch.float32, device=x.device)
    st = lib.so2_swiglu_s2_stages(int(stages), _ptr(x), _ptr(w_a), _ptr(w_b), _ptr(w_g), _ptr(w_o), _ptr(y), n,
                                  L, C, dt, _ptr(workspace), ws_bytes, _stream_handle(x.device))
    _check(st, "so2_swiglu_s2")
    return y
