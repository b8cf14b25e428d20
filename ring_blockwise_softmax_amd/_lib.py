"""ctypes binding of libra.so (argument marshalling only).

Every step of the computation runs in the HIP library; this module only turns
torch tensors into ``ra_tensor`` descriptors, allocates outputs and workspace
with torch (device memory and streams are torch's), and raises on errors.
There is no fallback: if the library is missing the import fails loudly.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libra.so")

# ra_dtype
RA_BF16, RA_F32 = 0, 1
# ra_mask
MASKS = {"none": 0, "causal": 1, "causal_bottom_right": 2}
# ra_layout_kind
LAYOUTS = {"contig": 0, "contig_causal": 1, "zigzag_causal": 2, "kv_sharded": 3, "kv_sharded_causal": 4}
ORDERS = {"ring": 0, "tokenring": 1}
KERNEL_KINDS = ("attn", "merge", "split_reduce")
# Size of the static device scratch of ra_block_attn_fwd_noalloc (RA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 32 << 20


class RaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("b", ctypes.c_int64), ("s", ctypes.c_int64), ("h", ctypes.c_int64), ("d", ctypes.c_int64),
                ("sb", ctypes.c_int64), ("ss", ctypes.c_int64), ("sh", ctypes.c_int64)]


class RaLayout(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("order", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("fuse_merge", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class RaPlanSeg(ctypes.Structure):
    _fields_ = [("kv_start", ctypes.c_int64), ("kv_len", ctypes.c_int64), ("causal", ctypes.c_int32),
                ("kv_rank", ctypes.c_int32)]


class RaPlanItem(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("rank", ctypes.c_int32), ("q_start", ctypes.c_int64),
                ("q_len", ctypes.c_int64), ("nseg", ctypes.c_int32), ("first", ctypes.c_int32),
                ("seg", RaPlanSeg * 2), ("q_pos0", ctypes.c_int64)]


EXPORTS = {
    "ra_block_attn_fwd": (ctypes.c_int, [ctypes.POINTER(RaTensor)] * 3 + [ctypes.c_int] +
                          [ctypes.POINTER(RaTensor)] * 2 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "ra_block_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(RaTensor)] * 2),
    "ra_block_attn_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(RaTensor)] * 3 + [ctypes.c_int] +
                                  [ctypes.POINTER(RaTensor)] * 2 + [ctypes.c_void_p]),
    "ra_merge": (ctypes.c_int, [ctypes.POINTER(RaTensor)] * 4 + [ctypes.c_void_p]),
    "ra_ring_forward": (ctypes.c_int, [ctypes.POINTER(RaTensor)] * 3 + [ctypes.c_int, ctypes.POINTER(RaLayout)] +
                        [ctypes.POINTER(RaTensor)] * 2 + [ctypes.c_void_p]),
    "ra_ring_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(RaTensor)] * 2 +
                                [ctypes.c_int, ctypes.POINTER(RaLayout)]),
    "ra_ring_plan": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.POINTER(RaLayout),
                                    ctypes.POINTER(RaPlanItem), ctypes.c_int]),
    "ra_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "ra_profile_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_double),
                                       ctypes.c_int]),
    "ra_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "ra_last_error": (ctypes.c_char_p, []),
    "ra_version": (ctypes.c_int, []),
}

_lib = None


def _check_single_hip_runtime():
    """The library must bind to the HIP runtime torch already loaded."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise RuntimeError(f"two HIP runtimes mapped in this process: {sorted(real)}")


def lib():
    """Load libra.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- loads torch's libamdhip64 first

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m ring_blockwise_softmax_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _check_single_hip_runtime()
    _lib = L
    return L


class RaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{lib().ra_status_str(status).decode()}: {msg}")
        self.status = status


def check(status: int):
    if status != 0:
        raise RaError(status, lib().ra_last_error().decode())


def dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bfloat16 or float32")


def bshd(t) -> RaTensor:
    """Descriptor of a [B, S, H, d] tensor with d contiguous."""
    if t.dim() != 4:
        raise ValueError("expected a [B, S, H, d] tensor")
    if t.stride(3) != 1:
        raise ValueError("the last dimension must be contiguous")
    b, s, h, d = t.shape
    return RaTensor(t.data_ptr(), dtype_code(t), 0, b, s, h, d, t.stride(0), t.stride(1), t.stride(2))


def lse_desc(t) -> RaTensor:
    """Descriptor of an lse tensor stored [B, H, S] (logical [B, S, H])."""
    if t.dim() != 3:
        raise ValueError("expected an lse tensor of shape [B, H, S]")
    b, h, s = t.shape
    return RaTensor(t.data_ptr(), dtype_code(t), 0, b, s, h, 1, t.stride(0), t.stride(2), t.stride(1))


def stream_ptr(stream=None):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)
