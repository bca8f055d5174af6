"""ctypes binding of libspecverify.so (the C ABI in include/spec_verify.h).

Argument marshalling only: every step of the verify path runs in the HIP
kernels of the library.  torch is used for device buffers and the stream
handle.  Importing this module fails loudly when the library has not been
built; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecverify.so")

SV_OK = 0
SV_ERR_INVALID_ARG = 1
SV_ERR_OUT_OF_MEMORY = 2
SV_ERR_DEVICE = 3
SV_ERR_UNSUPPORTED = 4
SV_ERR_CAPACITY = 5
SV_ERR_DEVICE_CONTRACT = 6
SV_F32 = 0
SV_BF16 = 1
SV_FLAG_PROFILE = 1
SV_FLAG_TWO_KERNEL = 2
SV_DEVERR_DRAFT_ID = 1
SV_DEVERR_OFFSETS = 2
SV_DEVERR_NONFINITE = 4
SV_DEVERR_TOPK = 16
SV_MAX_GAMMA = 128
SV_MAX_TOPK = 64


def stats_len(gamma: int) -> int:
    """Length of the acceptance-counter array for padded width ``gamma`` (SV_STATS_LEN)."""
    return 5 + 3 * int(gamma)
SV_SCHEDULE_NONE = 0
SV_SCHEDULE_SPLIT = 1
SV_SCHEDULE_FLAT = 2

SCHEDULE_FLAGS = {None: 0, "auto": 0, "twokernel": SV_FLAG_TWO_KERNEL}
SCHEDULE_NAMES = {SV_SCHEDULE_NONE: "none", SV_SCHEDULE_SPLIT: "rows-split+draw", SV_SCHEDULE_FLAT: "rows+draw"}

EXPORTS = (
    "spec_verify_create",
    "spec_verify_run",
    "spec_verify_destroy",
    "spec_verify_device_errors",
    "spec_verify_profile_read",
    "spec_verify_last_schedule",
    "spec_verify_status_string",
    "spec_verify_run_static",
)
SV_STATIC_MAX_BATCH = 256
SV_STATIC_MAX_ROWS = 4096


class SVConfig(ctypes.Structure):
    _fields_ = [
        ("max_batch", ctypes.c_int32),
        ("max_gamma", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("logits_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class SVArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("gamma", ctypes.c_int32),
        ("total_draft", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("draft_offsets", ctypes.c_void_p),
        ("target_logits", ctypes.c_void_p),
        ("draft_probs", ctypes.c_void_p),
        ("draft_ids", ctypes.c_void_p),
        ("temperature", ctypes.c_void_p),
        ("uniforms", ctypes.c_void_p),
        ("out_tokens", ctypes.c_void_p),
        ("out_num_accepted", ctypes.c_void_p),
        ("diag_row_max", ctypes.c_void_p),
        ("diag_row_norm", ctypes.c_void_p),
        ("diag_ratio", ctypes.c_void_p),
        ("draft_topk", ctypes.c_int32),
        ("draft_topk_ids", ctypes.c_void_p),
        ("draft_topk_probs", ctypes.c_void_p),
        ("stats", ctypes.c_void_p),
    ]


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: the library then binds to the HIP runtime torch has loaded,
    # so device pointers and streams from torch are valid in it
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m lossless_rejection_sampling_sampler_amd.build` "
            "(the verifier has no CPU fallback)")
    lib = ctypes.CDLL(path)
    lib.spec_verify_create.argtypes = [ctypes.POINTER(SVConfig), ctypes.c_int,
                                       ctypes.POINTER(ctypes.c_void_p)]
    lib.spec_verify_create.restype = ctypes.c_int
    lib.spec_verify_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(SVArgs), ctypes.c_void_p]
    lib.spec_verify_run.restype = ctypes.c_int
    lib.spec_verify_destroy.argtypes = [ctypes.c_void_p]
    lib.spec_verify_destroy.restype = ctypes.c_int
    lib.spec_verify_device_errors.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
    lib.spec_verify_device_errors.restype = ctypes.c_int
    lib.spec_verify_profile_read.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                             ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
    lib.spec_verify_profile_read.restype = ctypes.c_int
    lib.spec_verify_last_schedule.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)]
    lib.spec_verify_last_schedule.restype = ctypes.c_int
    lib.spec_verify_status_string.argtypes = [ctypes.c_int]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_run_static.argtypes = [ctypes.c_int, ctypes.POINTER(SVArgs), ctypes.c_void_p]
    lib.spec_verify_run_static.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().spec_verify_status_string(status).decode()


def run_static(logits_dtype: str, args: "SVArgs", stream_handle: int) -> int:
    """spec_verify_run_static: the verify step with the library's static device
    scratch (no context, nothing allocated); returns the status."""
    lib = load_library()
    return lib.spec_verify_run_static(SV_BF16 if logits_dtype == "bf16" else SV_F32, ctypes.byref(args),
                                      ctypes.c_void_p(stream_handle))


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


class SpecVerify:
    """One verifier context (device scratch for one stream).

    ``run`` takes torch CUDA tensors in the layout of the C header and
    enqueues the verify step on ``stream`` (default: torch's current stream).
    """

    def __init__(self, max_batch: int, max_gamma: int, vocab: int, logits_dtype: str = "bf16",
                 device: int = 0, profile: bool = False, schedule: Optional[str] = None):
        self._lib = load_library()
        self.vocab = int(vocab)
        self.device = int(device)
        self.logits_dtype = logits_dtype
        cfg = SVConfig(int(max_batch), int(max_gamma), int(vocab),
                       SV_BF16 if logits_dtype == "bf16" else SV_F32,
                       (SV_FLAG_PROFILE if profile else 0)
                       | SCHEDULE_FLAGS[schedule])
        handle = ctypes.c_void_p()
        st = self._lib.spec_verify_create(ctypes.byref(cfg), self.device, ctypes.byref(handle))
        if st != SV_OK:
            raise SpecVerifyError(st, "spec_verify_create")
        self._ctx = handle

    def run(self, *, target_logits, draft_probs, draft_ids, temperature, uniforms,
            out_tokens, out_num_accepted, gamma: int, draft_offsets=None, total_draft=None,
            diag_row_max=None, diag_row_norm=None, diag_ratio=None, draft_topk: int = 0,
            draft_topk_ids=None, draft_topk_probs=None, stats=None, stream=None) -> None:
        """draft_probs None selects a sparse q (draft_topk > 0 entries per row in
        draft_topk_ids / draft_topk_probs) or point-mass drafts (draft_topk == 0)."""
        import torch
        batch = int(temperature.shape[0])
        if total_draft is None:
            total_draft = int(draft_ids.shape[0])
        args = SVArgs(batch, int(gamma), int(total_draft), self.vocab,
                      _ptr(draft_offsets), _ptr(target_logits), _ptr(draft_probs), _ptr(draft_ids),
                      _ptr(temperature), _ptr(uniforms), _ptr(out_tokens), _ptr(out_num_accepted),
                      _ptr(diag_row_max), _ptr(diag_row_norm), _ptr(diag_ratio),
                      int(draft_topk), _ptr(draft_topk_ids), _ptr(draft_topk_probs), _ptr(stats))
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        st = self._lib.spec_verify_run(self._ctx, ctypes.byref(args), ctypes.c_void_p(handle))
        if st != SV_OK:
            raise SpecVerifyError(st, "spec_verify_run")

    def run_args(self, args: SVArgs, stream_handle: int) -> int:
        """Raw call with a prepared SVArgs (returns the status)."""
        return self._lib.spec_verify_run(self._ctx, ctypes.byref(args), ctypes.c_void_p(stream_handle))

    def device_errors(self, clear: bool = False) -> int:
        bits = ctypes.c_uint32(0)
        st = self._lib.spec_verify_device_errors(self._ctx, ctypes.byref(bits), 1 if clear else 0)
        if st != SV_OK:
            raise SpecVerifyError(st, "spec_verify_device_errors")
        return int(bits.value)

    def profile_read(self):
        """(rows-kernel ms, draw-kernel ms, calls) summed since the last read."""
        a, b, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int32()
        st = self._lib.spec_verify_profile_read(self._ctx, ctypes.byref(a), ctypes.byref(b), ctypes.byref(n))
        if st != SV_OK:
            raise SpecVerifyError(st, "spec_verify_profile_read")
        return a.value, b.value, n.value

    def last_schedule(self) -> int:
        """SV_SCHEDULE_* of the last successful run on this context."""
        v = ctypes.c_int32()
        st = self._lib.spec_verify_last_schedule(self._ctx, ctypes.byref(v))
        if st != SV_OK:
            raise SpecVerifyError(st, "spec_verify_last_schedule")
        return v.value

    def close(self) -> None:
        if getattr(self, "_ctx", None):
            self._lib.spec_verify_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
