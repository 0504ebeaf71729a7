"""ctypes binding of libscute.so (the C ABI in include/scute.h).

Argument marshalling only: every step of the forward runs in the library's
HIP kernels. PyTorch is used by callers for device memory and streams; this
module accepts torch tensors (device pointers via ``data_ptr()``) or raw
integer pointers. The library must be built first (``build()`` in
``__graft_entry__`` or ``python -m lora_normal_form_amd.build``); importing
this module without it raises.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SCUTE_LIB names another build of the library (the sanitized host build)
LIB_PATH = os.environ.get("SCUTE_LIB") or os.path.join(_HERE, "libscute.so")

OK = 0
E_INVALID, E_SHAPE, E_NOMEM, E_HIP, E_STATE, E_UNSUPPORTED = -1, -2, -3, -4, -5, -6
F32, BF16, F64 = 0, 1, 2
LORA, DORA, IA3, VERA, OFT, NORMAL_FORM = 0, 1, 2, 3, 4, 5
METHOD_IDS = {"lora": LORA, "dora": DORA, "ia3": IA3, "vera": VERA, "oft": OFT, "nf": NORMAL_FORM}
SLOT_A, SLOT_B, SLOT_S, SLOT_BIAS, SLOT_VD, SLOT_VE, SLOT_P = range(7)

_STATUS_NAMES = {E_INVALID: "SCUTE_E_INVALID", E_SHAPE: "SCUTE_E_SHAPE", E_NOMEM: "SCUTE_E_NOMEM",
                 E_HIP: "SCUTE_E_HIP", E_STATE: "SCUTE_E_STATE",
                 E_UNSUPPORTED: "SCUTE_E_UNSUPPORTED"}


class ScuteError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


class AdapterDesc(C.Structure):
    _fields_ = [("method", C.c_int32), ("dtype", C.c_int32), ("rank", C.c_int32),
                ("blk", C.c_int32), ("c", C.c_double),
                ("A", C.c_void_p), ("B", C.c_void_p), ("d", C.c_void_p), ("e", C.c_void_p),
                ("m", C.c_void_p), ("l", C.c_void_p), ("vd", C.c_void_p), ("ve", C.c_void_p),
                ("Q", C.c_void_p), ("R", C.c_void_p), ("s", C.c_void_p), ("b", C.c_void_p)]


class Cost(C.Structure):
    _fields_ = [("bytes", C.c_double), ("adapter_bytes", C.c_double), ("flops", C.c_double),
                ("base_flops", C.c_double), ("launches", C.c_int32), ("n_tokens", C.c_int32),
                ("n_segments", C.c_int32), ("n_rot_rows", C.c_int32),
                ("n_vera_rows", C.c_int32), ("n_touched", C.c_int32),
                ("gemm_bytes", C.c_double), ("prologue_bytes", C.c_double),
                ("gemm_flops", C.c_double), ("prologue_flops", C.c_double)]


class AdapterInfo(C.Structure):
    _fields_ = [("loaded", C.c_int32), ("method", C.c_int32), ("rank", C.c_int32),
                ("blk", C.c_int32), ("has_R", C.c_int32), ("has_s", C.c_int32),
                ("has_b", C.c_int32), ("has_term", C.c_int32), ("has_vera", C.c_int32)]


class BatchInfo(C.Structure):
    _fields_ = [("n", C.c_int32), ("n_segments", C.c_int32), ("n_rot_rows", C.c_int32),
                ("n_vera_rows", C.c_int32), ("max_rank", C.c_int32), ("path", C.c_int32)]


class KernelTime(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_int32), ("total_ms", C.c_double)]


# exported symbols and their signatures (must match include/scute.h)
_P = C.c_void_p
SIGNATURES = {
    "scute_layer_create": (C.c_int32, [C.c_int32, C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                                       C.POINTER(_P)]),
    "scute_layer_destroy": (C.c_int32, [_P]),
    "scute_set_vera_shared": (C.c_int32, [_P, _P, _P, C.c_int32]),
    "scute_load_adapter": (C.c_int32, [_P, C.c_int32, C.POINTER(AdapterDesc), _P, _P]),
    "scute_load_adapter_proj": (C.c_int32, [_P, C.c_int32, C.POINTER(AdapterDesc), C.POINTER(_P), _P, _P]),
    "scute_layer_set_projections": (C.c_int32, [_P, C.c_int32, C.POINTER(C.c_int64)]),
    "scute_unload_adapter": (C.c_int32, [_P, C.c_int32, _P]),
    "scute_plan_batch": (C.c_int32, [_P, _P, C.c_int32, _P, C.POINTER(_P)]),
    "scute_plan_batch_flags": (C.c_int32, [_P, _P, C.c_int32, C.c_uint32, _P, C.POINTER(_P)]),
    "scute_batch_destroy": (C.c_int32, [_P]),
    "scute_layer_forward": (C.c_int32, [_P, _P, _P, _P, _P, _P]),
    "scute_layer_forward_noalloc": (C.c_int32, [_P, _P, C.c_int32, _P, _P, _P, _P]),
    "scute_cost_model": (C.c_int32, [_P, _P, C.POINTER(Cost)]),
    "scute_adapter_info_get": (C.c_int32, [_P, C.c_int32, C.POINTER(AdapterInfo)]),
    "scute_read_slot": (C.c_int32, [_P, C.c_int32, C.c_int32, _P, C.c_int64]),
    "scute_batch_info_get": (C.c_int32, [_P, C.POINTER(BatchInfo)]),
    "scute_batch_read": (C.c_int32, [_P, _P, _P]),
    "scute_batch_wait_failures": (C.c_int32, [_P, C.c_int32, C.POINTER(C.c_int32)]),
    "scute_profile_enable": (C.c_int32, [_P, C.c_int32]),
    "scute_profile_read": (C.c_int32, [_P, C.POINTER(KernelTime), C.c_int32,
                                       C.POINTER(C.c_int32)]),
    "scute_launch_empty": (C.c_int32, [C.c_int32, _P]),
    "scute_silu_gate": (C.c_int32, [_P, _P, _P, C.c_int64, _P]),
    "scute_last_error": (C.c_char_p, []),
    "scute_version": (C.c_char_p, []),
}


def _load():
    # One HIP runtime per process: PyTorch ships its own libamdhip64 (soname
    # libamdhip64.so.7). Importing torch first makes the dynamic loader bind
    # libscute.so to that same runtime, so device pointers and streams from
    # torch are valid in the library's calls.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m lora_normal_form_amd.build` (hipcc, gfx950)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(code):
    if code != OK:
        raise ScuteError(code, lib.scute_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Device / host address of a torch tensor, numpy array or int (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except Exception:
            pass
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------------
# same-named thin wrappers (raise ScuteError on a failing status)
# --------------------------------------------------------------------------

def scute_layer_create(device: int, d_in: int, d_out: int, act_dtype: int,
                       max_adapters: int) -> int:
    h = _P()
    _check(lib.scute_layer_create(device, d_in, d_out, act_dtype, max_adapters, C.byref(h)))
    return h.value


def scute_layer_destroy(layer: int) -> None:
    _check(lib.scute_layer_destroy(layer))


def scute_set_vera_shared(layer: int, A_sh, B_sh, r_v: int) -> None:
    _check(lib.scute_set_vera_shared(layer, _ptr(A_sh), _ptr(B_sh), r_v))


def scute_load_adapter(layer: int, id: int, desc: AdapterDesc, W_host=None, stream=None) -> None:
    _check(lib.scute_load_adapter(layer, id, C.byref(desc), _ptr(W_host), _stream_ptr(stream)))


def scute_load_adapter_proj(layer: int, id: int, desc: AdapterDesc, R_proj, W_host=None,
                            stream=None) -> None:
    """R_proj: one host array per projection ([d_in/blk][blk][blk] in the
    descriptor's dtype) or None for the identity."""
    ptrs = (_P * len(R_proj))(*[_ptr(r) for r in R_proj])
    _check(lib.scute_load_adapter_proj(layer, id, C.byref(desc), ptrs, _ptr(W_host), _stream_ptr(stream)))


def scute_layer_set_projections(layer: int, col_end) -> None:
    ends = (C.c_int64 * len(col_end))(*[int(e) for e in col_end])
    _check(lib.scute_layer_set_projections(layer, len(col_end), ends))


def scute_unload_adapter(layer: int, id: int, stream=None) -> None:
    _check(lib.scute_unload_adapter(layer, id, _stream_ptr(stream)))


PLAN_DETERMINISTIC = 1
PLAN_ROUTE_EXPAND_PASS = 2
PLAN_ROUTE_SEPARATE_S = 4
PLAN_ROUTE_VERA_PASS = 8
PLAN_ROUTE_ROTATE_PASS = 16


def scute_plan_batch(layer: int, token_adapter, stream=None) -> int:
    ta = np.ascontiguousarray(np.asarray(token_adapter, dtype=np.int32))
    h = _P()
    _check(lib.scute_plan_batch(layer, ta.ctypes.data if ta.size else None, int(ta.size),
                                _stream_ptr(stream), C.byref(h)))
    return h.value


def scute_plan_batch_flags(layer: int, token_adapter, flags: int, stream=None) -> int:
    ta = np.ascontiguousarray(np.asarray(token_adapter, dtype=np.int32))
    h = _P()
    _check(lib.scute_plan_batch_flags(layer, ta.ctypes.data if ta.size else None, int(ta.size),
                                      int(flags), _stream_ptr(stream), C.byref(h)))
    return h.value


def scute_silu_gate(g, u, h, count=None, stream=None) -> None:
    """h = silu(g) (.) u on device float32 tensors."""
    n = int(h.numel() if count is None else count)
    _check(lib.scute_silu_gate(_ptr(g), _ptr(u), _ptr(h), n, _stream_ptr(stream)))


def scute_launch_empty(count: int, stream=None) -> None:
    _check(lib.scute_launch_empty(int(count), _stream_ptr(stream)))


def scute_batch_destroy(batch: int) -> None:
    _check(lib.scute_batch_destroy(batch))


def scute_layer_forward(layer: int, batch: int, x, W, y, stream=None) -> None:
    _check(lib.scute_layer_forward(layer, batch, _ptr(x), _ptr(W), _ptr(y), _stream_ptr(stream)))


def scute_layer_forward_noalloc(layer: int, token_adapter, n: int, x, W, y, stream=None) -> None:
    """token_adapter: a device int32 tensor [n] (the ids stay on the device)."""
    _check(lib.scute_layer_forward_noalloc(layer, _ptr(token_adapter), int(n), _ptr(x), _ptr(W), _ptr(y),
                                           _stream_ptr(stream)))


def scute_cost_model(layer: int, batch: int) -> Dict:
    c = Cost()
    _check(lib.scute_cost_model(layer, batch, C.byref(c)))
    return {f: getattr(c, f) for f, _ in Cost._fields_}


def scute_adapter_info_get(layer: int, id: int) -> Dict:
    i = AdapterInfo()
    _check(lib.scute_adapter_info_get(layer, id, C.byref(i)))
    return {f: getattr(i, f) for f, _ in AdapterInfo._fields_}


def scute_read_slot(layer: int, id: int, slot: int, nbytes: int) -> bytes:
    buf = C.create_string_buffer(nbytes)
    _check(lib.scute_read_slot(layer, id, slot, C.cast(buf, C.c_void_p), nbytes))
    return buf.raw


def scute_batch_info_get(batch: int) -> Dict:
    i = BatchInfo()
    _check(lib.scute_batch_info_get(batch, C.byref(i)))
    return {f: getattr(i, f) for f, _ in BatchInfo._fields_}


def scute_batch_read(batch: int):
    info = scute_batch_info_get(batch)
    perm = np.zeros(info["n"], np.int32)
    seg = np.zeros(3 * info["n_segments"], np.int32)
    _check(lib.scute_batch_read(batch, perm.ctypes.data if perm.size else None,
                                seg.ctypes.data if seg.size else None))
    return perm, seg.reshape(-1, 3)


def scute_profile_enable(layer: int, enable: bool) -> None:
    _check(lib.scute_profile_enable(layer, 1 if enable else 0))


def scute_profile_read(layer: int) -> Dict[str, Dict]:
    """{kernel name: {"launches": k, "total_ms": t}} since the last read."""
    cap = 32
    buf = (KernelTime * cap)()
    cnt = C.c_int32(0)
    _check(lib.scute_profile_read(layer, buf, cap, C.byref(cnt)))
    return {buf[i].name.decode(): {"launches": buf[i].launches, "total_ms": buf[i].total_ms}
            for i in range(min(cnt.value, cap))}


def scute_batch_wait_failures(batch: int, reset: bool = False) -> int:
    out = C.c_int32(0)
    _check(lib.scute_batch_wait_failures(batch, 1 if reset else 0, C.byref(out)))
    return out.value


def scute_last_error() -> str:
    return lib.scute_last_error().decode()


def scute_version() -> str:
    return lib.scute_version().decode()


# --------------------------------------------------------------------------
# descriptor construction from host arrays
# --------------------------------------------------------------------------

_DESC_ARRAYS = ("A", "B", "d", "e", "m", "l", "vd", "ve", "Q", "R", "s", "b")


def make_desc(method, rank=0, blk=0, c=1.0, **arrays):
    """Build an AdapterDesc over float64 host copies of the given arrays.

    Returns (desc, keepalive); keep ``keepalive`` until the load returns.
    """
    keep = []
    desc = AdapterDesc()
    desc.method = METHOD_IDS[method] if isinstance(method, str) else int(method)
    desc.dtype = F64
    desc.rank = int(rank)
    desc.blk = int(blk)
    desc.c = float(c)
    for k, v in arrays.items():
        if k not in _DESC_ARRAYS:
            raise TypeError(f"unknown descriptor array {k}")
        if v is None:
            continue
        a = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
        keep.append(a)
        setattr(desc, k, a.ctypes.data)
    return desc, keep


# --------------------------------------------------------------------------
# convenience object wrapper
# --------------------------------------------------------------------------

class Layer:
    """Owns one scute_layer handle and the plans built for it."""

    def __init__(self, d_in, d_out, dtype="bf16", max_adapters=64, device=0):
        self.d_in, self.d_out = int(d_in), int(d_out)
        self.act = BF16 if dtype == "bf16" else F32
        self.device = device
        self.h = scute_layer_create(device, d_in, d_out, self.act, max_adapters)
        self._vera_refs = None

    def close(self):
        if self.h:
            scute_layer_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_vera_shared(self, A_sh, B_sh, r_v):
        scute_set_vera_shared(self.h, A_sh, B_sh, r_v)
        self._vera_refs = (A_sh, B_sh)  # borrowed by the library: keep alive

    def load(self, id, method, rank=0, blk=0, c=1.0, W_host=None, stream=None, **arrays):
        desc, keep = make_desc(method, rank, blk, c, **arrays)
        w = None if W_host is None else np.ascontiguousarray(np.asarray(W_host, np.float64))
        scute_load_adapter(self.h, id, desc, w, stream)
        del keep

    def load_proj(self, id, R_proj, blk, rank=0, c=1.0, W_host=None, stream=None, **arrays):
        """A normal-form adapter with one rotation per projection (R_proj[p]:
        [d_in/blk][blk][blk], None for the identity)."""
        desc, keep = make_desc("nf", rank, blk, c, **arrays)
        rs = [None if r is None else np.ascontiguousarray(np.asarray(r, dtype=np.float64)) for r in R_proj]
        w = None if W_host is None else np.ascontiguousarray(np.asarray(W_host, np.float64))
        scute_load_adapter_proj(self.h, id, desc, rs, w, stream)
        del keep, rs

    def set_projections(self, col_end):
        scute_layer_set_projections(self.h, col_end)

    def unload(self, id, stream=None):
        scute_unload_adapter(self.h, id, stream)

    def plan(self, token_adapter, stream=None, deterministic=False, flags=0) -> "Batch":
        flags |= PLAN_DETERMINISTIC if deterministic else 0
        if flags:
            return Batch(self, scute_plan_batch_flags(self.h, token_adapter, flags, stream))
        return Batch(self, scute_plan_batch(self.h, token_adapter, stream))

    def forward(self, batch, x, W, y, stream=None):
        scute_layer_forward(self.h, batch.h, x, W, y, stream)
        return y

    def forward_noalloc(self, token_adapter, x, W, y, stream=None):
        scute_layer_forward_noalloc(self.h, token_adapter, token_adapter.shape[0], x, W, y, stream)
        return y

    def cost(self, batch):
        return scute_cost_model(self.h, batch.h)

    def info(self, id):
        return scute_adapter_info_get(self.h, id)

    def read_slot(self, id, slot, shape, dtype):
        """Stored slot as a numpy array; bf16 slots come back as float64."""
        count = int(np.prod(shape))
        if dtype == "bf16":
            raw = scute_read_slot(self.h, id, slot, 2 * count)
            bits = np.frombuffer(raw, np.uint16).astype(np.uint32) << 16
            return bits.view(np.float32).astype(np.float64).reshape(shape)
        dt = np.dtype(dtype)
        raw = scute_read_slot(self.h, id, slot, dt.itemsize * count)
        return np.frombuffer(raw, dt).reshape(shape).astype(np.float64)


class Batch:
    def __init__(self, layer, h):
        self.layer, self.h = layer, h

    def close(self):
        if self.h:
            scute_batch_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def info(self):
        return scute_batch_info_get(self.h)

    def read(self):
        return scute_batch_read(self.h)

    def wait_failures(self, reset=False):
        """1 if a forward of this plan had a bounded wait give up (fused decode
        path), else 0; reset clears it."""
        return scute_batch_wait_failures(self.h, reset)
