"""libmhla: the MHLA forward pass on AMD Instinct MI355X (gfx950).

Thin ctypes binding over the C ABI declared in ``include/mhla.h``: the
functions below carry the C names and only marshal arguments (tensor data
pointers, shape structs, the current HIP stream).  Every step of the forward
pass runs in the HIP kernels of ``libmhla.so``; there is no Python or CPU
fallback -- if the library is missing, every call raises.

MHLA (arXiv 2601.07832; paperlayer.ai summary, section 4) splits the tokens of
a 2D/3D grid into M non-overlapping blocks, summarises each block as
S_j = phi(K_j)^T V_j and z_j = sum phi(k), mixes the summaries with a learnable
M x M matrix W, and gives every query o = phi(q) St_i / (phi(q) . zt_i + eps).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmhla.so")

MHLA_OK = 0
MHLA_ERR_INVALID_ARG = 1
MHLA_ERR_UNSUPPORTED = 2
MHLA_ERR_MISALIGNED = 3
MHLA_ERR_ALLOC = 4
MHLA_ERR_HIP = 5

MHLA_F32 = 0
MHLA_BF16 = 1

MHLA_PATH_3KERNEL = 0
MHLA_PATH_FUSED = 1
MHLA_PATH_CAUSAL = 2

MHLA_VARIANT_MIX_RESIDENT = 1 << 8
MHLA_VARIANT_MIX_TILED = 1 << 9
MHLA_VARIANT_NO_PAIR_HEADS = 1 << 10
MHLA_VARIANT_MIX_SPLIT = 1 << 11
MHLA_VARIANT_APPLY_REGS = 1 << 12

MHLA_PHI_ELU1 = 0
MHLA_PHI_RELU_EPS = 1


class mhla_grid(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("extent", ctypes.c_int32 * 3),
                ("eps", ctypes.c_float)]


class mhla_block(ctypes.Structure):
    _fields_ = [("extent", ctypes.c_int32 * 3)]


class mhla_layer_params(ctypes.Structure):
    _fields_ = [("ln_w", ctypes.c_void_p), ("ln_b", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p),
                ("b_qkv", ctypes.c_void_p), ("qn_w", ctypes.c_void_p), ("kn_w", ctypes.c_void_p),
                ("lepe_w", ctypes.c_void_p), ("lepe_b", ctypes.c_void_p), ("w_out", ctypes.c_void_p),
                ("b_out", ctypes.c_void_p), ("phi", ctypes.c_int32), ("phi_eps", ctypes.c_float),
                ("ln_eps", ctypes.c_float), ("rms_eps", ctypes.c_float)]


class MhlaError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {mhla_status_string(status)}" if what else mhla_status_string(status))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmhla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m token_level_head_block_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        G, Bk = ctypes.POINTER(mhla_grid), ctypes.POINTER(mhla_block)
        vp = ctypes.c_void_p
        L.mhla_status_string.argtypes = [ctypes.c_int]
        L.mhla_status_string.restype = ctypes.c_char_p
        L.mhla_check_problem.argtypes = [G, Bk, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        L.mhla_check_problem.restype = ctypes.c_int
        L.mhla_launch_plan.argtypes = [G, Bk, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_char_p)]
        L.mhla_launch_plan.restype = ctypes.c_int
        L.mhla_backward_workspace_bytes.argtypes = [G, Bk]
        L.mhla_backward_workspace_bytes.restype = ctypes.c_size_t
        L.mhla_backward.argtypes = [vp, vp, vp, vp, vp, G, Bk, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
        L.mhla_backward.restype = ctypes.c_int
        L.mhla_backward_ex.argtypes = [vp, vp, vp, vp, vp, G, Bk, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                       ctypes.c_int32, vp, vp]
        L.mhla_backward_ex.restype = ctypes.c_int
        L.mhla_causal_backward_workspace_bytes.argtypes = [G, Bk]
        L.mhla_causal_backward_workspace_bytes.restype = ctypes.c_size_t
        L.mhla_causal_backward.argtypes = [vp, vp, vp, vp, vp, G, Bk, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp]
        L.mhla_causal_backward.restype = ctypes.c_int
        L.mhla_causal_state_bytes.argtypes = [G, Bk, ctypes.c_int32]
        L.mhla_causal_state_bytes.restype = ctypes.c_size_t
        L.mhla_causal_stream_workspace_bytes.argtypes = [G, Bk]
        L.mhla_causal_stream_workspace_bytes.restype = ctypes.c_size_t
        L.mhla_causal_stream.argtypes = [vp, vp, vp, vp, ctypes.c_int32, G, Bk, ctypes.c_int32, vp, ctypes.c_int32,
                                         vp, vp, ctypes.c_size_t, vp]
        L.mhla_causal_stream.restype = ctypes.c_int
        L.mhla_workspace_bytes.argtypes = [G, Bk]
        L.mhla_workspace_bytes.restype = ctypes.c_size_t
        L.mhla_forward.argtypes = [vp, vp, vp, vp, G, Bk, vp, vp]
        L.mhla_forward.restype = ctypes.c_int
        L.mhla_forward_ws.argtypes = [vp, vp, vp, vp, G, Bk, vp, vp, ctypes.c_size_t, vp]
        L.mhla_forward_ws.restype = ctypes.c_int
        L.mhla_forward_ex.argtypes = [vp, vp, vp, vp, G, Bk, vp, vp, ctypes.c_size_t, ctypes.c_int32,
                                      vp, vp]
        L.mhla_forward_ex.restype = ctypes.c_int
        L.mhla_forward_noalloc.argtypes = [vp, vp, vp, vp, G, Bk, vp, vp]
        L.mhla_forward_noalloc.restype = ctypes.c_int
        L.mhla_layer_workspace_bytes.argtypes = [G, Bk]
        L.mhla_layer_workspace_bytes.restype = ctypes.c_size_t
        L.mhla_layer_forward.argtypes = [vp, vp, G, Bk, ctypes.POINTER(mhla_layer_params), vp, vp,
                                         ctypes.c_size_t, vp, vp]
        L.mhla_layer_forward.restype = ctypes.c_int
        _lib = L
    return _lib


# ---------------------------------------------------------------- structs

def make_grid(batch: int, heads: int, head_dim: int, dtype: int, extents, eps: float = 1e-6) -> mhla_grid:
    g = mhla_grid()
    g.batch, g.heads, g.head_dim, g.dtype = batch, heads, head_dim, dtype
    g.ndim = len(extents)
    for a in range(3):
        g.extent[a] = int(extents[a]) if a < len(extents) else 0
    g.eps = eps
    return g


def make_block(extents) -> mhla_block:
    b = mhla_block()
    for a in range(3):
        b.extent[a] = int(extents[a]) if a < len(extents) else 0
    return b


# ---------------------------------------------------------------- C entry points

def mhla_status_string(status: int) -> str:
    return lib().mhla_status_string(int(status)).decode()


def mhla_check_problem(grid: mhla_grid, block: mhla_block):
    """(status, M, T)."""
    m, t = ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib().mhla_check_problem(ctypes.byref(grid), ctypes.byref(block), ctypes.byref(m), ctypes.byref(t))
    return st, m.value, t.value


def mhla_launch_plan(grid: mhla_grid, block: mhla_block, path: int = 0):
    """(status, [kernel names in launch order])."""
    n = ctypes.c_int32(0)
    names = (ctypes.c_char_p * 3)()
    st = lib().mhla_launch_plan(ctypes.byref(grid), ctypes.byref(block), int(path), ctypes.byref(n), names)
    return st, [names[i].decode() for i in range(n.value)]


def mhla_workspace_bytes(grid: mhla_grid, block: mhla_block) -> int:
    return int(lib().mhla_workspace_bytes(ctypes.byref(grid), ctypes.byref(block)))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check_tensors(q, k, v, W, out, grid: mhla_grid, block: mhla_block):
    """Host-side shape/dtype checks of torch tensors against the grid, so the
    kernels never index past a buffer whose size the C ABI cannot see."""
    import torch
    st, M, _ = mhla_check_problem(grid, block)
    if st != MHLA_OK:
        return
    N = 1
    for a in range(grid.ndim):
        N *= grid.extent[a]
    want = (grid.batch, N, grid.heads, grid.head_dim)
    tdt = torch.bfloat16 if grid.dtype == MHLA_BF16 else torch.float32
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not isinstance(t, torch.Tensor):
            continue
        if tuple(t.shape) != want or t.dtype != tdt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {tdt} tensor of shape {want}, "
                             f"got {t.dtype} {tuple(t.shape)}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a GPU")
    if isinstance(W, torch.Tensor):
        if tuple(W.shape) != (M, M) or W.dtype != torch.float32 or not W.is_contiguous() or not W.is_cuda:
            raise ValueError(f"W must be a contiguous float32 GPU tensor of shape {(M, M)}")


def mhla_forward(q, k, v, W, grid: mhla_grid, block: mhla_block, out, stream=None) -> int:
    _check_tensors(q, k, v, W, out, grid, block)
    return lib().mhla_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(W), ctypes.byref(grid),
                              ctypes.byref(block), _ptr(out), _stream(stream))


def mhla_forward_ws(q, k, v, W, grid: mhla_grid, block: mhla_block, out, ws, ws_bytes: int,
                    stream=None) -> int:
    _check_tensors(q, k, v, W, out, grid, block)
    return lib().mhla_forward_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(W), ctypes.byref(grid),
                                 ctypes.byref(block), _ptr(out), _ptr(ws), int(ws_bytes),
                                 _stream(stream))


MHLA_NOALLOC_SCRATCH_BYTES = 32 << 20


def mhla_forward_noalloc(q, k, v, W, grid: mhla_grid, block: mhla_block, out, stream=None) -> int:
    """mhla_forward with the library's fixed per-GPU scratch as workspace (allocates nothing)."""
    _check_tensors(q, k, v, W, out, grid, block)
    return lib().mhla_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(W), ctypes.byref(grid),
                                      ctypes.byref(block), _ptr(out), _stream(stream))


def mhla_forward_ex(q, k, v, W, grid: mhla_grid, block: mhla_block, out, ws, ws_bytes: int,
                    path: int = MHLA_PATH_3KERNEL, stage_events=None, stream=None) -> int:
    """stage_events: None or 4 events, each a torch.cuda.Event (already
    recorded once, so that its HIP handle exists) or a raw hipEvent_t handle
    (int)."""
    _check_tensors(q, k, v, W, out, grid, block)
    ev = None
    if stage_events is not None:
        if len(stage_events) != 4:
            raise ValueError("stage_events needs 4 events")
        arr = (ctypes.c_void_p * 4)(*[e if isinstance(e, int) else e.cuda_event for e in stage_events])
        if any(a is None or a == 0 for a in arr):
            raise ValueError("stage events have no HIP handle yet; record each once first")
        ev = ctypes.cast(arr, ctypes.c_void_p)
    return lib().mhla_forward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(W), ctypes.byref(grid),
                                 ctypes.byref(block), _ptr(out), _ptr(ws), int(ws_bytes), int(path),
                                 ev, _stream(stream))


def mhla_backward_workspace_bytes(grid: mhla_grid, block: mhla_block) -> int:
    return int(lib().mhla_backward_workspace_bytes(ctypes.byref(grid), ctypes.byref(block)))


def _events(stage_events, n):
    if stage_events is None:
        return None
    if len(stage_events) != n:
        raise ValueError(f"stage_events needs {n} events")
    arr = (ctypes.c_void_p * n)(*[e if isinstance(e, int) else e.cuda_event for e in stage_events])
    if any(a is None or a == 0 for a in arr):
        raise ValueError("stage events have no HIP handle yet; record each once first")
    return ctypes.cast(arr, ctypes.c_void_p)


def mhla_backward(q, k, v, W, dout, grid: mhla_grid, block: mhla_block, dq, dk, dv, dW, ws=None,
                  ws_bytes: int = 0, stage_events=None, stream=None) -> int:
    """Gradients dq, dk, dv (bf16 tensors like q) and dW (fp32 [M, M]) for the
    upstream gradient dout.  stage_events: None or 5 events (torch.cuda.Event
    already recorded once, or raw hipEvent_t handles)."""
    _check_tensors(q, k, v, W, dout, grid, block)
    _check_tensors(dq, dk, dv, dW, None, grid, block)
    return lib().mhla_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(dout), ctypes.byref(grid),
                               ctypes.byref(block), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dW), _ptr(ws),
                               int(ws_bytes), _events(stage_events, 5), _stream(stream))


def mhla_backward_ex(q, k, v, W, dout, grid: mhla_grid, block: mhla_block, dq, dk, dv, dW, ws=None,
                     ws_bytes: int = 0, variant: int = 0, stage_events=None, stream=None) -> int:
    """As mhla_backward, with MHLA_VARIANT_* flags (MHLA_VARIANT_NO_PAIR_HEADS)."""
    _check_tensors(q, k, v, W, dout, grid, block)
    _check_tensors(dq, dk, dv, dW, None, grid, block)
    return lib().mhla_backward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(dout), ctypes.byref(grid),
                                  ctypes.byref(block), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dW), _ptr(ws),
                                  int(ws_bytes), int(variant), _events(stage_events, 5), _stream(stream))


def mhla_causal_backward_workspace_bytes(grid: mhla_grid, block: mhla_block) -> int:
    return int(lib().mhla_causal_backward_workspace_bytes(ctypes.byref(grid), ctypes.byref(block)))


def mhla_causal_backward(q, k, v, W, dout, grid: mhla_grid, block: mhla_block, dq, dk, dv, dW, ws=None,
                         ws_bytes: int = 0, stage_events=None, stream=None) -> int:
    """Gradients through the causal chunkwise form; arguments as mhla_backward."""
    _check_tensors(q, k, v, W, dout, grid, block)
    _check_tensors(dq, dk, dv, dW, None, grid, block)
    return lib().mhla_causal_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(W), _ptr(dout), ctypes.byref(grid),
                                      ctypes.byref(block), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dW), _ptr(ws),
                                      int(ws_bytes), _events(stage_events, 5), _stream(stream))


def mhla_causal_state_bytes(grid: mhla_grid, block: mhla_block, max_chunks: int) -> int:
    return int(lib().mhla_causal_state_bytes(ctypes.byref(grid), ctypes.byref(block), int(max_chunks)))


def mhla_causal_stream_workspace_bytes(grid: mhla_grid, block: mhla_block) -> int:
    return int(lib().mhla_causal_stream_workspace_bytes(ctypes.byref(grid), ctypes.byref(block)))


def mhla_causal_stream(q, k, v, W, grid: mhla_grid, block: mhla_block, n_past: int, state, max_chunks: int, out,
                       ws=None, ws_bytes: int = 0, stream=None) -> int:
    """One call of a causal stream: q, k, v, out [B, N_new, H, d] (the new
    chunks), W fp32 [w_dim, w_dim] (w_dim from W's shape), state fp32 with
    mhla_causal_state_bytes(grid, block, max_chunks) bytes."""
    for t in (q, k, v, out):
        if t is None or not t.is_contiguous():
            raise ValueError("q, k, v and out must be contiguous device tensors")
    if W.dim() != 2 or W.shape[0] != W.shape[1] or not W.is_contiguous():
        raise ValueError("W must be a contiguous square fp32 matrix")
    if not state.is_contiguous() or state.numel() * state.element_size() < mhla_causal_state_bytes(grid, block,
                                                                                                  max_chunks):
        raise ValueError("state is smaller than mhla_causal_state_bytes")
    return lib().mhla_causal_stream(_ptr(q), _ptr(k), _ptr(v), _ptr(W), int(W.shape[0]), ctypes.byref(grid),
                                    ctypes.byref(block), int(n_past), _ptr(state), int(max_chunks), _ptr(out),
                                    _ptr(ws), int(ws_bytes), _stream(stream))


# ---------------------------------------------------------------- convenience

def forward(q, k, v, W, grid_extents, block_extents, eps: float = 1e-6, out=None, ws=None,
            path: int = MHLA_PATH_3KERNEL, stream=None):
    """Allocate `out` if needed, call mhla_forward_ex, raise MhlaError on failure."""
    import torch
    dt = MHLA_BF16 if q.dtype == torch.bfloat16 else MHLA_F32
    B, N, H, d = q.shape
    g = make_grid(B, H, d, dt, grid_extents, eps)
    b = make_block(block_extents)
    if out is None:
        out = torch.empty_like(q)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = mhla_forward_ex(q, k, v, W, g, b, out, ws, nbytes, path, None, stream)
    if st != MHLA_OK:
        raise MhlaError(st, "mhla_forward_ex")
    return out


# ---------------------------------------------------------------- layer

LAYER_PARAM_NAMES = ("ln_w", "ln_b", "w_qkv", "b_qkv", "qn_w", "kn_w", "lepe_w", "lepe_b", "w_out", "b_out")


def mhla_layer_workspace_bytes(grid: mhla_grid, block: mhla_block) -> int:
    return int(lib().mhla_layer_workspace_bytes(ctypes.byref(grid), ctypes.byref(block)))


def _check_layer_tensors(x, W, grid: mhla_grid, block: mhla_block, params: dict, y):
    """Host-side shape/dtype checks of the layer's torch tensors (the C ABI
    cannot see tensor sizes)."""
    import torch
    st, M, _ = mhla_check_problem(grid, block)
    if st != MHLA_OK:
        return
    N = 1
    for a in range(grid.ndim):
        N *= grid.extent[a]
    C = grid.heads * grid.head_dim
    want = {"ln_w": ((C,), torch.float32), "ln_b": ((C,), torch.float32),
            "w_qkv": ((3 * C, C), torch.bfloat16), "b_qkv": ((3 * C,), torch.float32),
            "qn_w": ((C,), torch.float32), "kn_w": ((C,), torch.float32),
            "lepe_w": ((C, 5, 5), torch.float32), "lepe_b": ((C,), torch.float32),
            "w_out": ((C, C), torch.bfloat16), "b_out": ((C,), torch.float32)}
    tensors = [("x", x, ((grid.batch, N, C), torch.bfloat16)), ("y", y, ((grid.batch, N, C), torch.bfloat16)),
               ("W", W, ((M, M), torch.float32))]
    tensors += [(k, params.get(k), want[k]) for k in LAYER_PARAM_NAMES]
    for name, t, (shape, dt) in tensors:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor) or tuple(t.shape) != shape or t.dtype != dt \
                or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous {dt} GPU tensor of shape {shape}")


def mhla_layer_forward(x, W, grid: mhla_grid, block: mhla_block, params: dict, y, ws=None, ws_bytes: int = 0,
                       phi: int = MHLA_PHI_ELU1, phi_eps: float = 1e-6, ln_eps: float = 1e-5,
                       rms_eps: float = 1e-6, stage_events=None, stream=None) -> int:
    """The layer forward through the C ABI.  params: dict with the tensors
    named in LAYER_PARAM_NAMES (absent or None for optional ones)."""
    _check_layer_tensors(x, W, grid, block, params, y)
    P = mhla_layer_params()
    for name in LAYER_PARAM_NAMES:
        setattr(P, name, _ptr(params.get(name)))
    P.phi, P.phi_eps, P.ln_eps, P.rms_eps = int(phi), float(phi_eps), float(ln_eps), float(rms_eps)
    return lib().mhla_layer_forward(_ptr(x), _ptr(W), ctypes.byref(grid), ctypes.byref(block), ctypes.byref(P),
                                    _ptr(y), _ptr(ws), int(ws_bytes), _events(stage_events, 5), _stream(stream))
