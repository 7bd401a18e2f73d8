"""Thin ctypes binding of ``libgdn2.so`` (see ``include/gdn2.h``).

Argument marshalling only: torch provides device memory and the current HIP
stream; every step of the computation runs in the library's gfx950 kernels.
There is no CPU fallback: if the library is missing, or a tensor is not on a
GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn2.so")

GDN2_DTYPE_BF16, GDN2_DTYPE_F32, GDN2_DTYPE_I32, GDN2_DTYPE_F16, GDN2_DTYPE_I64 = 1, 2, 3, 4, 5
_DTYPES = {torch.bfloat16: GDN2_DTYPE_BF16, torch.float32: GDN2_DTYPE_F32, torch.int32: GDN2_DTYPE_I32,
           torch.float16: GDN2_DTYPE_F16, torch.int64: GDN2_DTYPE_I64}
GDN2_STATE_KV, GDN2_STATE_VK = 0, 1
_LAYOUTS = {"kv": GDN2_STATE_KV, "vk": GDN2_STATE_VK}

STATUS = {0: "OK", -1: "NULL_ARG", -2: "DTYPE", -3: "SHAPE", -4: "HEADS",
          -5: "UNSUPPORTED", -6: "LAYOUT", -7: "ALIAS", -8: "HIP"}

EXPORTED = ["gdn2_chunk_fwd", "gdn2_chunk_fwd_opts", "gdn2_chunk_fwd_noalloc", "gdn2_chunk_fwd_check",
            "gdn2_split_plan",
            "gdn2_recurrent_fwd", "gdn2_recurrent_fwd_opts", "gdn2_recurrent_fwd_check",
            "gdn2_chunk_bwd", "gdn2_chunk_bwd_check", "gdn2_last_error", "gdn2_abi_version"]


class Gdn2Tensor(ctypes.Structure):
    """Mirror of ``gdn2_tensor``."""
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class Gdn2FwdOptions(ctypes.Structure):
    """Mirror of ``gdn2_fwd_options``."""
    _fields_ = [("struct_size", ctypes.c_int32), ("seq_split_chunks", ctypes.c_int32),
                ("state_layout", ctypes.c_int32), ("qk_l2norm", ctypes.c_int32)]


def make_options(seq_split=0, state_layout="kv", qk_l2norm=False):
    """A filled ``gdn2_fwd_options`` (state_layout "kv": [N, HV, K, V],
    "vk": [N, HV, V, K])."""
    if state_layout not in _LAYOUTS:
        raise ValueError(f"state_layout must be 'kv' or 'vk', not {state_layout!r}")
    return Gdn2FwdOptions(ctypes.sizeof(Gdn2FwdOptions), int(seq_split or 0), _LAYOUTS[state_layout],
                          1 if qk_l2norm else 0)


class Gdn2Error(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"gdn2 error {code} ({STATUS.get(code, '?')}): {message}")
        self.code = code
        self.status = STATUS.get(code, "?")


_lib = None


def load_library():
    """Load libgdn2.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Gdn2Tensor)
        lib.gdn2_chunk_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P, P, ctypes.c_void_p]
        lib.gdn2_chunk_fwd.restype = ctypes.c_int
        lib.gdn2_chunk_fwd_opts.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P, P,
                                            ctypes.POINTER(Gdn2FwdOptions), ctypes.c_void_p]
        lib.gdn2_chunk_fwd_opts.restype = ctypes.c_int
        lib.gdn2_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P, P,
                                               ctypes.POINTER(Gdn2FwdOptions), ctypes.c_void_p]
        lib.gdn2_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.gdn2_recurrent_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P, P, ctypes.c_void_p]
        lib.gdn2_recurrent_fwd.restype = ctypes.c_int
        lib.gdn2_recurrent_fwd_opts.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P, P,
                                                ctypes.POINTER(Gdn2FwdOptions), ctypes.c_void_p]
        lib.gdn2_recurrent_fwd_opts.restype = ctypes.c_int
        lib.gdn2_recurrent_fwd_check.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P, P]
        lib.gdn2_recurrent_fwd_check.restype = ctypes.c_int
        lib.gdn2_split_plan.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        lib.gdn2_split_plan.restype = ctypes.c_int
        lib.gdn2_chunk_fwd_check.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P, P]
        lib.gdn2_chunk_fwd_check.restype = ctypes.c_int
        lib.gdn2_chunk_bwd.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, P,
                                       ctypes.c_void_p]
        lib.gdn2_chunk_bwd.restype = ctypes.c_int
        lib.gdn2_chunk_bwd_check.argtypes = [P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, P]
        lib.gdn2_chunk_bwd_check.restype = ctypes.c_int
        lib.gdn2_last_error.argtypes = []
        lib.gdn2_last_error.restype = ctypes.c_char_p
        lib.gdn2_abi_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def last_error() -> str:
    return load_library().gdn2_last_error().decode()


def describe(t):
    """Build a gdn2_tensor descriptor for a torch tensor (None -> NULL)."""
    if t is None:
        return None
    d = Gdn2Tensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _DTYPES.get(t.dtype, 0)
    d.ndim = t.dim()
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ptr(d):
    return None if d is None else ctypes.byref(d)


def _scale_arg(scale):
    return 0.0 if scale is None else float(scale)


def check(q, k, v, g=None, beta=None, w=None, scale=None, initial_state=None,
          cu_seqlens=None, out=None, final_state=None):
    """Run the library's host-side validation only (no GPU needed).

    Returns the status code (0 = valid); never touches device memory."""
    lib = load_library()
    ds = [describe(x) for x in (q, k, v, g, beta, w)]
    rest = [describe(x) for x in (initial_state, cu_seqlens, out, final_state)]
    return lib.gdn2_chunk_fwd_check(*[_ptr(d) for d in ds], _scale_arg(scale),
                                    *[_ptr(d) for d in rest])


def split_plan(T, N, HV, num_cu):
    """The library's automatic segment length (0 = whole sequences) for T
    tokens in N sequences with HV value heads on ``num_cu`` compute units."""
    return load_library().gdn2_split_plan(int(T), int(N), int(HV), int(num_cu))


def _prepare(q, k, v, initial_state, cu_seqlens, output_final_state, out, final_state, g, beta, w,
             state_layout="kv"):
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("w", w),
                    ("initial_state", initial_state), ("cu_seqlens", cu_seqlens)):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    T, HV, V = v.shape
    K = q.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    if out is None:
        out = torch.empty((T, HV, V), dtype=q.dtype, device=v.device)
    if final_state is None and output_final_state:
        shape = (N, HV, V, K) if state_layout == "vk" else (N, HV, K, V)
        final_state = torch.empty(shape, dtype=torch.float32, device=v.device)
    descs = [describe(x) for x in (q, k, v, g, beta, w)]
    rest = [describe(x) for x in (initial_state, cu_seqlens, out, final_state)]
    return out, final_state, descs, rest


def chunk_fwd(q, k, v, g=None, beta=None, w=None, scale=None, initial_state=None,
              cu_seqlens=None, output_final_state=True, out=None, final_state=None,
              seq_split=None, state_layout="kv", qk_l2norm=False):
    """GDN-2 chunked prefill forward on the current HIP stream.

    q, k [T, H, K] and v, w [T, HV, V], beta [T, HV, K], out: bf16 or
    float16 (q's type); g [T, HV, K] float32, bf16 or float16;
    initial_state and final_state [N, HV, K, V] float32 or bf16
    ([N, HV, V, K] with ``state_layout="vk"``); cu_seqlens [N + 1] int32 or int64 (None: one
    sequence). Strided views are accepted where the rows are contiguous.
    ``scale`` None or 0 means 1/sqrt(K). Returns (out [T, HV, V],
    final_state or None); preallocated ``out`` / ``final_state`` are written
    in place. ``seq_split``: None or 0 automatic, -1 never split sequences,
    n > 0 split every sequence into segments of n 64-token chunks.
    ``qk_l2norm``: normalise q and k rows in the kernel.
    """
    lib = load_library()
    out, final_state, descs, rest = _prepare(q, k, v, initial_state, cu_seqlens, output_final_state, out,
                                             final_state, g, beta, w, state_layout)
    stream = torch.cuda.current_stream(v.device).cuda_stream
    if seq_split is None and state_layout == "kv" and not qk_l2norm:
        rc = lib.gdn2_chunk_fwd(*[_ptr(d) for d in descs], _scale_arg(scale),
                                *[_ptr(d) for d in rest], ctypes.c_void_p(stream))
    else:
        opts = make_options(seq_split, state_layout, qk_l2norm)
        rc = lib.gdn2_chunk_fwd_opts(*[_ptr(d) for d in descs], _scale_arg(scale),
                                     *[_ptr(d) for d in rest], ctypes.byref(opts), ctypes.c_void_p(stream))
    if rc != 0:
        raise Gdn2Error(rc, last_error())
    return out, final_state


def chunk_fwd_noalloc(q, k, v, g=None, beta=None, w=None, scale=None, initial_state=None,
                      cu_seqlens=None, out=None, final_state=None, seq_split=None, state_layout="kv",
                      qk_l2norm=False):
    """:func:`chunk_fwd` through ``gdn2_chunk_fwd_noalloc``: the library
    allocates no device memory (a split run's workspace is its fixed device
    array). ``out`` and ``final_state`` must be preallocated by the caller
    (``final_state`` None: not produced)."""
    lib = load_library()
    if out is None:
        raise ValueError("chunk_fwd_noalloc needs a preallocated out")
    _, _, descs, rest = _prepare(q, k, v, initial_state, cu_seqlens, False, out, final_state, g, beta, w,
                                 state_layout)
    stream = torch.cuda.current_stream(v.device).cuda_stream
    opts = make_options(seq_split, state_layout, qk_l2norm)
    rc = lib.gdn2_chunk_fwd_noalloc(*[_ptr(d) for d in descs], _scale_arg(scale), *[_ptr(d) for d in rest],
                                    ctypes.byref(opts), ctypes.c_void_p(stream))
    if rc != 0:
        raise Gdn2Error(rc, last_error())
    return out, final_state


def recurrent_fwd(q, k, v, g=None, beta=None, w=None, scale=None, initial_state=None,
                  cu_seqlens=None, output_final_state=True, out=None, final_state=None,
                  state_layout="kv", qk_l2norm=False):
    """The same forward evaluated token by token (decode and short spans).

    Tensors and options as in :func:`chunk_fwd`. ``final_state`` may be
    ``initial_state`` itself to update the state in place.
    """
    lib = load_library()
    out, final_state, descs, rest = _prepare(q, k, v, initial_state, cu_seqlens, output_final_state, out,
                                             final_state, g, beta, w, state_layout)
    stream = torch.cuda.current_stream(v.device).cuda_stream
    if state_layout == "kv" and not qk_l2norm:
        rc = lib.gdn2_recurrent_fwd(*[_ptr(d) for d in descs], _scale_arg(scale),
                                    *[_ptr(d) for d in rest], ctypes.c_void_p(stream))
    else:
        opts = make_options(0, state_layout, qk_l2norm)
        rc = lib.gdn2_recurrent_fwd_opts(*[_ptr(d) for d in descs], _scale_arg(scale),
                                         *[_ptr(d) for d in rest], ctypes.byref(opts), ctypes.c_void_p(stream))
    if rc != 0:
        raise Gdn2Error(rc, last_error())
    return out, final_state


BWD_GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dw", "d_initial_state")


def _bwd_descs(q, k, v, g, beta, w, initial_state, cu_seqlens, d_out, d_final_state, grads):
    ins = [describe(x) for x in (q, k, v, g, beta, w)]
    mid = [describe(x) for x in (initial_state, cu_seqlens, d_out, d_final_state)]
    outs = [describe(grads.get(n)) for n in BWD_GRADS]
    return ins, mid, outs


def chunk_bwd(q, k, v, g, beta, w, d_out, scale=None, initial_state=None, cu_seqlens=None,
              d_final_state=None, need_d_initial_state=True, grads=None):
    """Backward of :func:`chunk_fwd` on the current HIP stream.

    q, k [T, H, K], v, w [T, HV, V], beta [T, HV, K], d_out [T, HV, V]: one
    16-bit type, bf16 or float16; g [T, HV, K]: float32, bf16 or float16;
    initial_state and d_final_state [N, HV, K, V]: float32 (the states may
    be None: zero). Returns a dict with dq, dk ([T, H, K]), dv, dw
    ([T, HV, V]), dbeta ([T, HV, K]) in q's type, dg ([T, HV, K]) in g's
    type and d_initial_state (float32 [N, HV, K, V], or None when not
    requested). Tensors given in ``grads`` are written in place.
    """
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("w", w), ("d_out", d_out),
                    ("initial_state", initial_state), ("cu_seqlens", cu_seqlens), ("d_final_state", d_final_state)):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (there is no CPU path)")
    T, H, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    N = 1 if cu_seqlens is None else cu_seqlens.shape[0] - 1
    dev = v.device
    out = dict(grads or {})
    io, gt = q.dtype, g.dtype
    shapes = {"dq": ((T, H, K), io), "dk": ((T, H, K), io), "dv": ((T, HV, V), io), "dw": ((T, HV, V), io),
              "dbeta": ((T, HV, K), io), "dg": ((T, HV, K), gt), "d_initial_state": ((N, HV, K, V), torch.float32)}
    for n, (shp, dt) in shapes.items():
        if out.get(n) is None and (n != "d_initial_state" or need_d_initial_state):
            out[n] = torch.empty(shp, dtype=dt, device=dev)
    out.setdefault("d_initial_state", None)
    ins, mid, outs = _bwd_descs(q, k, v, g, beta, w, initial_state, cu_seqlens, d_out, d_final_state, out)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.gdn2_chunk_bwd(*[_ptr(d) for d in ins], _scale_arg(scale), *[_ptr(d) for d in mid],
                            *[_ptr(d) for d in outs], ctypes.c_void_p(stream))
    if rc != 0:
        raise Gdn2Error(rc, last_error())
    return out


def check_bwd(q, k, v, g, beta, w, d_out, scale=None, initial_state=None, cu_seqlens=None,
              d_final_state=None, grads=None):
    """The library's host-side validation of a backward call only (no GPU needed)."""
    lib = load_library()
    ins, mid, outs = _bwd_descs(q, k, v, g, beta, w, initial_state, cu_seqlens, d_out, d_final_state, grads or {})
    return lib.gdn2_chunk_bwd_check(*[_ptr(d) for d in ins], _scale_arg(scale), *[_ptr(d) for d in mid],
                                    *[_ptr(d) for d in outs])
