"""ctypes declarations of the C ABI in include/kvq.h.

torch is imported before the library is opened so that libkvq.so binds to the
HIP runtime torch already loaded (same soname), which makes torch's stream
handles and device pointers valid inside the library.  If the library has not
been built this module raises: there is no other implementation to fall back
to.
"""

from __future__ import annotations

import ctypes as C
import os

import torch  # noqa: F401  (loads the HIP runtime first)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

KV_OK = 0
STATUS = {
    0: "KV_OK", -1: "KV_ERR_ARG", -2: "KV_ERR_NO_SPACE", -3: "KV_ERR_BOUND", -4: "KV_ERR_FORMAT",
    -5: "KV_ERR_UNSUPPORTED", -6: "KV_ERR_WORKSPACE", -7: "KV_ERR_DEVICE",
}


class KvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status
        self.name = STATUS.get(status, str(status))


class Geom(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("n_q_heads", C.c_int32)]


class PoolStats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in
                ("pages", "free_pages", "reserved_pages", "used_pages", "page_bytes", "token_bytes", "tokens", "n_seqs")]


_P = C.c_void_p
_I32, _I64, _F = C.c_int32, C.c_int64, C.c_float
_PI32, _PI64 = C.POINTER(C.c_int32), C.POINTER(C.c_int64)

SIGNATURES = {
    "kv_token_bytes": [C.POINTER(Geom), C.c_int, _PI64, _PI64],
    "kv_pool_bytes_for_tokens": [C.POINTER(Geom), C.c_int, _I64, _PI64],
    "kv_pool_create": [_I64, C.POINTER(Geom), C.c_int, _I32, _I64, _P, C.POINTER(_P)],
    "kv_pool_destroy": [_P],
    "kv_pool_stats": [_P, C.POINTER(PoolStats)],
    "kv_pool_device_ptr": [_P, C.POINTER(_P), _PI64],
    "kv_seq_reserve": [_P, _I64, _PI32, _PI32],
    "kv_seq_fork": [_P, _I32, _I64, _I64, _P, _PI32],
    "kv_seq_release": [_P, _I32],
    "kv_seq_pages": [_P, _I32, _PI32, _I32, _PI32],
    "kv_seq_block_table": [_P, _I32, C.POINTER(_P), _PI32],
    "kv_append_quant": [_P, _I32, _I32, _PI32, _PI64, _PI32, _P, _P, _P],
    "kv_workspace_bytes": [_P, _I32, _I32, _I32, _PI64],
    "kv_decode_splits": [_P, _I32, _PI64, _PI32],
    "kv_attn_decode": [_P, _I32, _I32, _PI32, _PI64, _P, _F, _I32, _P, _I64, _P, _P, _I64, _P],
    "kv_attn_decode_static": [_P, _I32, _I32, _PI32, _PI64, _P, _F, _I32, _P, _P, _I64, _P],
    "kv_attn_prefill": [_P, _I32, _I32, _I64, _I32, _P, _F, _I32, _P, _I64, _P, _P],
    "kv_dequant_page": [_P, _I32, _I32, _I32, _I32, _P, _P],
    "kv_last_error": [],
    "kv_status_str": [C.c_int],
}


def load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m quantized_kv_attention_append_amd.build`")
    lib = C.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = C.c_char_p if name in ("kv_last_error", "kv_status_str") else C.c_int
    return lib


lib = load()


def check(status: int):
    if status != KV_OK:
        msg = lib.kv_last_error().decode()
        raise KvError(status, msg)
