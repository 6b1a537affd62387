"""Python binding of libflarepp (FLARE++ token-mixer forward on MI355X).

Argument marshalling only: tensors are passed to the C ABI as raw device
pointers together with torch's current HIP stream; every step of the
computation runs in the library's HIP kernels.  torch supplies device memory
(outputs and workspace) and the stream.  There is no fallback: if the
library is missing, loading it raises.

Entry points (same names as the C ABI in include/flarepp.h):

* ``flarepp_mixer_fwd(q0, q_fixed, gate, k0, k, v)`` -> y
* ``flarepp_mixer_fwd_noalloc(q0, q_fixed, gate, k0, k, v, y)`` -> y (no workspace;
  the library's own per-device array of FLAREPP_NOALLOC_SCRATCH_BYTES)
* ``simplified_flarepp_mixer_fwd(q0, k0, v0, k, v)`` -> y
* ``flare_mixer_fwd(q, k, v, scale)`` -> y
* ``flarepp_mixer_fwd_train(...)`` -> (y, saved); ``flarepp_mixer_bwd(..., y, dy, saved)``
  -> dict of fp32 gradients; ``flare_mixer_fwd_train`` / ``flare_mixer_bwd`` likewise
* ``flare_encode_fwd(q, k, v, scale, chunk_tokens=0)`` -> z (fp32)
* ``flare_decode_fwd(q, z, k, scale)`` -> y
* ``flarepp_workspace_size(B, H, N, M, D, dtype)`` and friends
"""

from __future__ import annotations

import ctypes
import math
import os
import re

__all__ = [
    "FlareppError", "load_library", "library_path", "dtype_code",
    "flarepp_mixer_fwd", "flarepp_mixer_fwd_noalloc", "flarepp_mixer_fwd_timed",
    "simplified_flarepp_mixer_fwd", "FLAREPP_NOALLOC_SCRATCH_BYTES",
    "flare_mixer_fwd", "flare_encode_fwd", "flare_decode_fwd",
    "flarepp_mixer_fwd_train", "flarepp_mixer_bwd", "flare_mixer_fwd_train", "flare_mixer_bwd",
    "simplified_flarepp_mixer_fwd_train", "simplified_flarepp_mixer_bwd",
    "flarepp_frontend_fwd", "flarepp_seed_norm_fwd",
    "flarepp_workspace_size", "flare_encode_workspace_size", "flare_decode_workspace_size",
    "flarepp_status_string", "flarepp_version", "declared_functions",
    "FLAREPP_OK", "FLAREPP_ERR_INVALID_ARGUMENT", "FLAREPP_ERR_UNSUPPORTED",
    "FLAREPP_ERR_WORKSPACE", "FLAREPP_ERR_HIP", "FLAREPP_F32", "FLAREPP_BF16", "FLAREPP_F16",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG), "include", "flarepp.h")

FLAREPP_OK = 0
FLAREPP_ERR_INVALID_ARGUMENT = 1
FLAREPP_ERR_UNSUPPORTED = 2
FLAREPP_ERR_WORKSPACE = 3
FLAREPP_ERR_HIP = 4
FLAREPP_F32, FLAREPP_BF16, FLAREPP_F16 = 0, 1, 2
FLAREPP_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

_lib = None


class FlareppError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {flarepp_status_string(status)} ({status})")


def library_path() -> str:
    """The in-tree libflarepp.so, or the file FLAREPP_LIBRARY names (the host
    sanitizer test points it at an instrumented build of the same sources)."""
    return os.environ.get("FLAREPP_LIBRARY") or os.path.join(_PKG, "libflarepp.so")


def load_library():
    """Load libflarepp.so (built in-tree by build_lib.py); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m rank_latent_attention_mixer_amd.build_lib`"
            " (there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    i64, sz, vp, i32, f32 = (ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                             ctypes.c_float)
    shape = [i64] * 5
    lib.flarepp_status_string.argtypes = [i32]
    lib.flarepp_status_string.restype = ctypes.c_char_p
    lib.flarepp_version.argtypes = []
    lib.flarepp_version.restype = ctypes.c_char_p
    lib.flarepp_workspace_size.argtypes = shape + [i32]
    lib.flarepp_workspace_size.restype = sz
    lib.flare_encode_workspace_size.argtypes = shape + [i32, i64]
    lib.flare_encode_workspace_size.restype = sz
    lib.flare_decode_workspace_size.argtypes = shape + [i32]
    lib.flare_decode_workspace_size.restype = sz
    lib.flarepp_mixer_fwd.argtypes = shape + [i32] + [vp] * 7 + [vp, sz, vp]
    lib.flarepp_mixer_fwd.restype = i32
    lib.flarepp_mixer_fwd_noalloc.argtypes = shape + [i32] + [vp] * 7 + [vp]
    lib.flarepp_mixer_fwd_noalloc.restype = i32
    lib.flarepp_mixer_fwd_timed.argtypes = shape + [i32] + [vp] * 7 + [vp, sz, vp, vp]
    lib.flarepp_mixer_fwd_timed.restype = i32
    lib.simplified_flarepp_mixer_fwd.argtypes = shape + [i32] + [vp] * 6 + [vp, sz, vp]
    lib.simplified_flarepp_mixer_fwd.restype = i32
    lib.flarepp_saved_size.argtypes = shape
    lib.flarepp_saved_size.restype = sz
    lib.flarepp_mixer_fwd_train.argtypes = shape + [i32] + [vp] * 7 + [vp, sz, vp, sz, vp]
    lib.flarepp_mixer_fwd_train.restype = i32
    lib.flare_mixer_fwd_train.argtypes = shape + [i32, f32] + [vp] * 4 + [vp, sz, vp, sz, vp]
    lib.flare_mixer_fwd_train.restype = i32
    lib.flarepp_bwd_workspace_size.argtypes = shape + [i32]
    lib.flarepp_bwd_workspace_size.restype = sz
    lib.flarepp_mixer_bwd.argtypes = shape + [i32] + [vp] * 8 + [vp, sz] + [vp] * 6 + [vp, sz, vp]
    lib.flarepp_mixer_bwd.restype = i32
    lib.flare_mixer_bwd.argtypes = shape + [i32, f32] + [vp] * 5 + [vp, sz] + [vp] * 3 + [vp, sz, vp]
    lib.flare_mixer_bwd.restype = i32
    lib.simplified_flarepp_mixer_fwd_train.argtypes = shape + [i32] + [vp] * 6 + [vp, sz, vp, sz, vp]
    lib.simplified_flarepp_mixer_fwd_train.restype = i32
    lib.simplified_flarepp_mixer_bwd.argtypes = shape + [i32] + [vp] * 7 + [vp, sz] + [vp] * 5 + [vp, sz, vp]
    lib.simplified_flarepp_mixer_bwd.restype = i32
    lib.flarepp_frontend_fwd.argtypes = [i64] * 5 + [i32] + [vp] * 8 + [f32, i32] + [vp] * 4
    lib.flarepp_frontend_fwd.restype = i32
    lib.flarepp_seed_norm_fwd.argtypes = [i64] * 3 + [i32, vp, vp, f32, vp, vp]
    lib.flarepp_seed_norm_fwd.restype = i32
    lib.flare_mixer_fwd.argtypes = shape + [i32, f32] + [vp] * 4 + [vp, sz, vp]
    lib.flare_mixer_fwd.restype = i32
    lib.flare_encode_fwd.argtypes = shape + [i32, f32, vp, i64, vp, vp, vp, i64, vp, sz, vp]
    lib.flare_encode_fwd.restype = i32
    lib.flare_decode_fwd.argtypes = shape + [i32, f32, vp, i64, vp, vp, vp, vp, sz, vp]
    lib.flare_decode_fwd.restype = i32
    _lib = lib
    return lib


def declared_functions():
    """Function names declared in include/flarepp.h."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(\w*flare\w*)\s*\(", text)))


def flarepp_status_string(status: int) -> str:
    return load_library().flarepp_status_string(int(status)).decode()


def flarepp_version() -> str:
    return load_library().flarepp_version().decode()


def flarepp_workspace_size(B, H, N, M, D, dtype) -> int:
    return int(load_library().flarepp_workspace_size(B, H, N, M, D, dtype))


def flare_encode_workspace_size(B, H, N, M, D, dtype, chunk_tokens=0) -> int:
    return int(load_library().flare_encode_workspace_size(B, H, N, M, D, dtype, chunk_tokens))


def flare_decode_workspace_size(B, H, N, M, D, dtype) -> int:
    return int(load_library().flare_decode_workspace_size(B, H, N, M, D, dtype))


# --------------------------------------------------------------------------
# torch marshalling
# --------------------------------------------------------------------------

def dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FLAREPP_F32, torch.bfloat16: FLAREPP_BF16, torch.float16: FLAREPP_F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _check_tensor(name, t, shape, dtype, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes, device, workspace):
    import torch
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _call(fn, where, *args):
    st = fn(*args)
    if st != FLAREPP_OK:
        raise FlareppError(st, where)


def flarepp_mixer_fwd(q0, q_fixed, gate, k0, k, v, y=None, workspace=None, stream=None):
    """FLARE++ mixer forward; see include/flarepp.h.  Returns y."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q0.shape[1]
    dev, dt = k.device, k.dtype
    for name, t, shp in (("q0", q0, (H, M, D)), ("q_fixed", q_fixed, (H, M, D)),
                         ("k0", k0, (B, H, N, D)), ("k", k, (B, H, N, D)),
                         ("v", v, (B, H, N, D))):
        _check_tensor(name, t, shp, dt, dev)
    _check_tensor("gate", gate, (H,), torch.float32, dev)
    if y is None:
        y = torch.empty((B, H, N, D), dtype=dt, device=dev)
    _check_tensor("y", y, (B, H, N, D), dt, dev)
    code = dtype_code(k)
    nbytes = lib.flarepp_workspace_size(B, H, N, M, D, code)
    if nbytes == 0:
        raise FlareppError(FLAREPP_ERR_UNSUPPORTED, "flarepp_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    _call(lib.flarepp_mixer_fwd, "flarepp_mixer_fwd", B, H, N, M, D, code, _ptr(q0),
          _ptr(q_fixed), _ptr(gate), _ptr(k0), _ptr(k), _ptr(v), _ptr(y), _ptr(ws),
          ws.numel(), _stream(stream))
    return y


def flarepp_mixer_fwd_noalloc(q0, q_fixed, gate, k0, k, v, y, stream=None):
    """FLARE++ mixer forward with no workspace argument (the library's own
    per-device array; the C call allocates nothing); see include/flarepp.h.
    y must be given.  Returns y."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q0.shape[1]
    dev, dt = k.device, k.dtype
    for name, t, shp in (("q0", q0, (H, M, D)), ("q_fixed", q_fixed, (H, M, D)),
                         ("k0", k0, (B, H, N, D)), ("k", k, (B, H, N, D)),
                         ("v", v, (B, H, N, D)), ("y", y, (B, H, N, D))):
        _check_tensor(name, t, shp, dt, dev)
    _check_tensor("gate", gate, (H,), torch.float32, dev)
    _call(lib.flarepp_mixer_fwd_noalloc, "flarepp_mixer_fwd_noalloc", B, H, N, M, D,
          dtype_code(k), _ptr(q0), _ptr(q_fixed), _ptr(gate), _ptr(k0), _ptr(k), _ptr(v),
          _ptr(y), _stream(stream))
    return y


def simplified_flarepp_mixer_fwd(q0, k0, v0, k, v, y=None, workspace=None, stream=None):
    """Simplified FLARE++ (separate synthesis values v0, q = synthesized
    query); see include/flarepp.h.  Returns y."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q0.shape[1]
    dev, dt = k.device, k.dtype
    for name, t, shp in (("q0", q0, (H, M, D)), ("k0", k0, (B, H, N, D)),
                         ("v0", v0, (B, H, N, D)), ("k", k, (B, H, N, D)),
                         ("v", v, (B, H, N, D))):
        _check_tensor(name, t, shp, dt, dev)
    if y is None:
        y = torch.empty((B, H, N, D), dtype=dt, device=dev)
    _check_tensor("y", y, (B, H, N, D), dt, dev)
    code = dtype_code(k)
    nbytes = lib.flarepp_workspace_size(B, H, N, M, D, code)
    if nbytes == 0:
        raise FlareppError(FLAREPP_ERR_UNSUPPORTED, "flarepp_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    _call(lib.simplified_flarepp_mixer_fwd, "simplified_flarepp_mixer_fwd", B, H, N, M, D, code,
          _ptr(q0), _ptr(k0), _ptr(v0), _ptr(k), _ptr(v), _ptr(y), _ptr(ws), ws.numel(),
          _stream(stream))
    return y


FLAREPP_TIMED_EVENTS = 7


def flarepp_mixer_fwd_timed(q0, q_fixed, gate, k0, k, v, events, y=None, workspace=None,
                            stream=None):
    """flarepp_mixer_fwd recording FLAREPP_TIMED_EVENTS caller-created
    hipEvent_t handles (integers) on the stream around its kernels."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q0.shape[1]
    dev, dt = k.device, k.dtype
    for name, t, shp in (("q0", q0, (H, M, D)), ("q_fixed", q_fixed, (H, M, D)),
                         ("k0", k0, (B, H, N, D)), ("k", k, (B, H, N, D)),
                         ("v", v, (B, H, N, D))):
        _check_tensor(name, t, shp, dt, dev)
    _check_tensor("gate", gate, (H,), torch.float32, dev)
    if len(events) != FLAREPP_TIMED_EVENTS:
        raise ValueError(f"need {FLAREPP_TIMED_EVENTS} events")
    if y is None:
        y = torch.empty((B, H, N, D), dtype=dt, device=dev)
    _check_tensor("y", y, (B, H, N, D), dt, dev)
    code = dtype_code(k)
    nbytes = lib.flarepp_workspace_size(B, H, N, M, D, code)
    if nbytes == 0:
        raise FlareppError(FLAREPP_ERR_UNSUPPORTED, "flarepp_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    ev = (ctypes.c_void_p * FLAREPP_TIMED_EVENTS)(*[ctypes.c_void_p(e) for e in events])
    _call(lib.flarepp_mixer_fwd_timed, "flarepp_mixer_fwd_timed", B, H, N, M, D, code,
          _ptr(q0), _ptr(q_fixed), _ptr(gate), _ptr(k0), _ptr(k), _ptr(v), _ptr(y), _ptr(ws),
          ws.numel(), _stream(stream), ev)
    return y


def flare_mixer_fwd(q, k, v, scale, y=None, workspace=None, stream=None):
    """Two-step FLARE forward with an explicit scale.  Returns y."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q.shape[1]
    dev, dt = k.device, k.dtype
    for name, t, shp in (("q", q, (H, M, D)), ("k", k, (B, H, N, D)), ("v", v, (B, H, N, D))):
        _check_tensor(name, t, shp, dt, dev)
    if y is None:
        y = torch.empty((B, H, N, D), dtype=dt, device=dev)
    _check_tensor("y", y, (B, H, N, D), dt, dev)
    code = dtype_code(k)
    nbytes = lib.flarepp_workspace_size(B, H, N, M, D, code)
    if nbytes == 0:
        raise FlareppError(FLAREPP_ERR_UNSUPPORTED, "flarepp_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    _call(lib.flare_mixer_fwd, "flare_mixer_fwd", B, H, N, M, D, code, float(scale), _ptr(q),
          _ptr(k), _ptr(v), _ptr(y), _ptr(ws), ws.numel(), _stream(stream))
    return y


def flare_encode_fwd(q, k, v, scale, chunk_tokens=0, z=None, workspace=None, stream=None):
    """Encoder alone: z = softmax(scale q k^T) v in fp32.  q is [H,M,D] (shared
    over the batch) or [B,H,M,D]."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q.shape[-2]
    dev, dt = k.device, k.dtype
    qshape = (H, M, D) if q.dim() == 3 else (B, H, M, D)
    _check_tensor("q", q, qshape, dt, dev)
    _check_tensor("k", k, (B, H, N, D), dt, dev)
    _check_tensor("v", v, (B, H, N, D), dt, dev)
    if z is None:
        z = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
    _check_tensor("z", z, (B, H, M, D), torch.float32, dev)
    code = dtype_code(k)
    nbytes = lib.flare_encode_workspace_size(B, H, N, M, D, code, chunk_tokens)
    if nbytes == 0:
        raise FlareppError(FLAREPP_ERR_INVALID_ARGUMENT, "flare_encode_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    qbs = 0 if q.dim() == 3 else H * M * D
    _call(lib.flare_encode_fwd, "flare_encode_fwd", B, H, N, M, D, code, float(scale), _ptr(q),
          qbs, _ptr(k), _ptr(v), _ptr(z), int(chunk_tokens), _ptr(ws), ws.numel(),
          _stream(stream))
    return z


def flare_decode_fwd(q, z, k, scale, y=None, workspace=None, stream=None):
    """Decoder alone: y = softmax over latents of (scale k q^T), applied to z."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q.shape[-2]
    dev, dt = k.device, k.dtype
    qshape = (H, M, D) if q.dim() == 3 else (B, H, M, D)
    _check_tensor("q", q, qshape, dt, dev)
    _check_tensor("z", z, (B, H, M, D), torch.float32, dev)
    _check_tensor("k", k, (B, H, N, D), dt, dev)
    if y is None:
        y = torch.empty((B, H, N, D), dtype=dt, device=dev)
    _check_tensor("y", y, (B, H, N, D), dt, dev)
    code = dtype_code(k)
    nbytes = lib.flare_decode_workspace_size(B, H, N, M, D, code)
    if nbytes == 0:
        raise FlareppError(FLAREPP_ERR_UNSUPPORTED, "flare_decode_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    qbs = 0 if q.dim() == 3 else H * M * D
    _call(lib.flare_decode_fwd, "flare_decode_fwd", B, H, N, M, D, code, float(scale), _ptr(q),
          qbs, _ptr(z), _ptr(k), _ptr(y), _ptr(ws), ws.numel(), _stream(stream))
    return y


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


# --------------------------------------------------------------------------
# training: forward with saved tensors, backward
# --------------------------------------------------------------------------

def _saved_buffer(B, H, N, M, D, device):
    import torch
    n = load_library().flarepp_saved_size(B, H, N, M, D)
    if n == 0:
        raise FlareppError(FLAREPP_ERR_INVALID_ARGUMENT, "flarepp_saved_size")
    return torch.empty(n // 4, dtype=torch.float32, device=device)


def flarepp_mixer_fwd_train(q0, q_fixed, gate, k0, k, v, y=None, workspace=None, stream=None):
    """FLARE++ forward that also returns the tensors its backward needs."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q0.shape[1]
    dev, dt = k.device, k.dtype
    for name, t, shp in (("q0", q0, (H, M, D)), ("q_fixed", q_fixed, (H, M, D)),
                         ("k0", k0, (B, H, N, D)), ("k", k, (B, H, N, D)),
                         ("v", v, (B, H, N, D))):
        _check_tensor(name, t, shp, dt, dev)
    _check_tensor("gate", gate, (H,), torch.float32, dev)
    if y is None:
        y = torch.empty((B, H, N, D), dtype=dt, device=dev)
    _check_tensor("y", y, (B, H, N, D), dt, dev)
    saved = _saved_buffer(B, H, N, M, D, dev)
    code = dtype_code(k)
    ws = _workspace(lib.flarepp_workspace_size(B, H, N, M, D, code), dev, workspace)
    _call(lib.flarepp_mixer_fwd_train, "flarepp_mixer_fwd_train", B, H, N, M, D, code, _ptr(q0),
          _ptr(q_fixed), _ptr(gate), _ptr(k0), _ptr(k), _ptr(v), _ptr(y), _ptr(saved),
          saved.numel() * 4, _ptr(ws), ws.numel(), _stream(stream))
    return y, saved


def flarepp_mixer_bwd(q0, q_fixed, gate, k0, k, v, y, dy, saved, workspace=None, stream=None):
    """Gradients of the FLARE++ mixer (fp32): dict(dq0, dq_fixed, dgate, dk0, dk, dv)."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q0.shape[1]
    dev, dt = k.device, k.dtype
    for name, t, shp in (("q0", q0, (H, M, D)), ("q_fixed", q_fixed, (H, M, D)),
                         ("k0", k0, (B, H, N, D)), ("k", k, (B, H, N, D)),
                         ("v", v, (B, H, N, D)), ("y", y, (B, H, N, D)),
                         ("dy", dy, (B, H, N, D))):
        _check_tensor(name, t, shp, dt, dev)
    _check_tensor("gate", gate, (H,), torch.float32, dev)
    f = dict(device=dev, dtype=torch.float32)
    g = dict(dq0=torch.empty((H, M, D), **f), dq_fixed=torch.empty((H, M, D), **f),
             dgate=torch.empty((H,), **f), dk0=torch.empty((B, H, N, D), **f),
             dk=torch.empty((B, H, N, D), **f), dv=torch.empty((B, H, N, D), **f))
    code = dtype_code(k)
    nbytes = lib.flarepp_bwd_workspace_size(B, H, N, M, D, code)
    if nbytes == 0:
        raise FlareppError(FLAREPP_ERR_UNSUPPORTED, "flarepp_bwd_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    _call(lib.flarepp_mixer_bwd, "flarepp_mixer_bwd", B, H, N, M, D, code, _ptr(q0),
          _ptr(q_fixed), _ptr(gate), _ptr(k0), _ptr(k), _ptr(v), _ptr(y), _ptr(dy), _ptr(saved),
          saved.numel() * 4, _ptr(g["dq0"]), _ptr(g["dq_fixed"]), _ptr(g["dgate"]),
          _ptr(g["dk0"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(ws), ws.numel(), _stream(stream))
    return g


def flare_mixer_fwd_train(q, k, v, scale, y=None, workspace=None, stream=None):
    """FLARE forward that also returns the tensors its backward needs."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q.shape[1]
    dev, dt = k.device, k.dtype
    for name, t, shp in (("q", q, (H, M, D)), ("k", k, (B, H, N, D)), ("v", v, (B, H, N, D))):
        _check_tensor(name, t, shp, dt, dev)
    if y is None:
        y = torch.empty((B, H, N, D), dtype=dt, device=dev)
    saved = _saved_buffer(B, H, N, M, D, dev)
    code = dtype_code(k)
    ws = _workspace(lib.flarepp_workspace_size(B, H, N, M, D, code), dev, workspace)
    _call(lib.flare_mixer_fwd_train, "flare_mixer_fwd_train", B, H, N, M, D, code, float(scale),
          _ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(saved), saved.numel() * 4, _ptr(ws),
          ws.numel(), _stream(stream))
    return y, saved


def flare_mixer_bwd(q, k, v, scale, y, dy, saved, workspace=None, stream=None):
    """Gradients of the FLARE mixer (fp32): dict(dq, dk, dv)."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q.shape[1]
    dev, dt = k.device, k.dtype
    for name, t, shp in (("q", q, (H, M, D)), ("k", k, (B, H, N, D)), ("v", v, (B, H, N, D)),
                         ("y", y, (B, H, N, D)), ("dy", dy, (B, H, N, D))):
        _check_tensor(name, t, shp, dt, dev)
    f = dict(device=dev, dtype=torch.float32)
    g = dict(dq=torch.empty((H, M, D), **f), dk=torch.empty((B, H, N, D), **f),
             dv=torch.empty((B, H, N, D), **f))
    code = dtype_code(k)
    nbytes = lib.flarepp_bwd_workspace_size(B, H, N, M, D, code)
    if nbytes == 0:
        raise FlareppError(FLAREPP_ERR_UNSUPPORTED, "flarepp_bwd_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    _call(lib.flare_mixer_bwd, "flare_mixer_bwd", B, H, N, M, D, code, float(scale), _ptr(q),
          _ptr(k), _ptr(v), _ptr(y), _ptr(dy), _ptr(saved), saved.numel() * 4, _ptr(g["dq"]),
          _ptr(g["dk"]), _ptr(g["dv"]), _ptr(ws), ws.numel(), _stream(stream))
    return g


def simplified_flarepp_mixer_fwd_train(q0, k0, v0, k, v, y=None, workspace=None, stream=None):
    """Simplified-mixer forward that also returns the tensors its backward needs."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q0.shape[1]
    dev, dt = k.device, k.dtype
    _check_tensor("q0", q0, (H, M, D), dt, dev)
    for name, t in (("k0", k0), ("v0", v0), ("k", k), ("v", v)):
        _check_tensor(name, t, (B, H, N, D), dt, dev)
    if y is None:
        y = torch.empty((B, H, N, D), dtype=dt, device=dev)
    saved = _saved_buffer(B, H, N, M, D, dev)
    code = dtype_code(k)
    ws = _workspace(lib.flarepp_workspace_size(B, H, N, M, D, code), dev, workspace)
    _call(lib.simplified_flarepp_mixer_fwd_train, "simplified_flarepp_mixer_fwd_train", B, H, N,
          M, D, code, _ptr(q0), _ptr(k0), _ptr(v0), _ptr(k), _ptr(v), _ptr(y), _ptr(saved),
          saved.numel() * 4, _ptr(ws), ws.numel(), _stream(stream))
    return y, saved


def simplified_flarepp_mixer_bwd(q0, k0, v0, k, v, y, dy, saved, workspace=None, stream=None):
    """Gradients of the simplified mixer (fp32): dict(dq0, dk0, dv0, dk, dv)."""
    import torch
    lib = load_library()
    B, H, N, D = k.shape
    M = q0.shape[1]
    dev, dt = k.device, k.dtype
    _check_tensor("q0", q0, (H, M, D), dt, dev)
    for name, t in (("k0", k0), ("v0", v0), ("k", k), ("v", v), ("y", y), ("dy", dy)):
        _check_tensor(name, t, (B, H, N, D), dt, dev)
    f = dict(device=dev, dtype=torch.float32)
    g = dict(dq0=torch.empty((H, M, D), **f), dk0=torch.empty((B, H, N, D), **f),
             dv0=torch.empty((B, H, N, D), **f), dk=torch.empty((B, H, N, D), **f),
             dv=torch.empty((B, H, N, D), **f))
    code = dtype_code(k)
    nbytes = lib.flarepp_bwd_workspace_size(B, H, N, M, D, code)
    if nbytes == 0:
        raise FlareppError(FLAREPP_ERR_UNSUPPORTED, "flarepp_bwd_workspace_size")
    ws = _workspace(nbytes, dev, workspace)
    _call(lib.simplified_flarepp_mixer_bwd, "simplified_flarepp_mixer_bwd", B, H, N, M, D, code,
          _ptr(q0), _ptr(k0), _ptr(v0), _ptr(k), _ptr(v), _ptr(y), _ptr(dy), _ptr(saved),
          saved.numel() * 4, _ptr(g["dq0"]), _ptr(g["dk0"]), _ptr(g["dv0"]), _ptr(g["dk"]),
          _ptr(g["dv"]), _ptr(ws), ws.numel(), _stream(stream))
    return g


# --------------------------------------------------------------------------
# front end: projections and head-wise normalisation
# --------------------------------------------------------------------------

def flarepp_frontend_fwd(x, w_k0, w_k, w_v, H, b_k0=None, b_k=None, b_v=None, g_k0=None,
                         eps=1e-6, normalize_k0=True, out=None, stream=None):
    """k0, k, v [B,H,N,D] from x [B,N,C] and linear-layer weights [H*D, C];
    k0 normalised head-wise (see include/flarepp.h)."""
    import torch
    lib = load_library()
    B, N, C = x.shape
    HD = w_k0.shape[0]
    if HD % H:
        raise ValueError(f"weight rows {HD} are not a multiple of H={H}")
    D = HD // H
    dev, dt = x.device, x.dtype
    _check_tensor("x", x, (B, N, C), dt, dev)
    for name, t in (("w_k0", w_k0), ("w_k", w_k), ("w_v", w_v)):
        _check_tensor(name, t, (HD, C), dt, dev)
    for name, t in (("b_k0", b_k0), ("b_k", b_k), ("b_v", b_v)):
        if t is not None:
            _check_tensor(name, t, (HD,), dt, dev)
    if g_k0 is not None:
        _check_tensor("g_k0", g_k0, (H, D), dt, dev)
    if out is None:
        out = tuple(torch.empty((B, H, N, D), dtype=dt, device=dev) for _ in range(3))
    for name, t in zip(("k0", "k", "v"), out):
        _check_tensor(name, t, (B, H, N, D), dt, dev)
    opt = lambda t: None if t is None else _ptr(t)
    _call(lib.flarepp_frontend_fwd, "flarepp_frontend_fwd", B, N, C, H, D, dtype_code(x),
          _ptr(x), _ptr(w_k0), _ptr(w_k), _ptr(w_v), opt(b_k0), opt(b_k), opt(b_v), opt(g_k0),
          float(eps), 1 if normalize_k0 else 0, _ptr(out[0]), _ptr(out[1]), _ptr(out[2]),
          _stream(stream))
    return out


def flarepp_seed_norm_fwd(q0, g=None, eps=1e-6, out=None, stream=None):
    """Head-wise normalisation of the seeds q0 [H, M, D]; out may be q0."""
    import torch
    lib = load_library()
    H, M, D = q0.shape
    _check_tensor("q0", q0, (H, M, D), q0.dtype, q0.device)
    if g is not None:
        _check_tensor("g", g, (H, D), q0.dtype, q0.device)
    if out is None:
        out = torch.empty_like(q0)
    _check_tensor("out", out, (H, M, D), q0.dtype, q0.device)
    _call(lib.flarepp_seed_norm_fwd, "flarepp_seed_norm_fwd", H, M, D, dtype_code(q0), _ptr(q0),
          None if g is None else _ptr(g), float(eps), _ptr(out), _stream(stream))
    return out
