"""ctypes binding of ``lib/libpa_probe.so`` (include/pa_probe.h): the
streaming-read and matrix-core probes (measurement helpers beside the
attention library) and the buffer range probe (a check of the hardware
behaviour the attention kernels rely on)."""

import ctypes
import os

from . import PaError, _dev, _stream

PROBE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libpa_probe.so")

# name -> (restype, argtypes): every symbol declared in include/pa_probe.h
SIGNATURES = {
    "pa_read_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "pa_mfma_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                     ctypes.c_void_p]),
    "pa_range_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]),
}

# Work of one pa_mfma_probe call per workgroup and iteration: 8 waves, four
# 32 x 32 x 16 products each (2 * 32 * 32 * 16 flops a product).
MFMA_PROBE_FLOPS_PER_WG_ITER = 8 * 4 * 2 * 32 * 32 * 16

_lib = None


def lib():
    """The loaded probe library (loaded on first use)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (binds the library to PyTorch's HIP runtime)
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with `python -m paged_kv_cache_382_amd.build`")
        handle = ctypes.CDLL(PROBE_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def pa_read_probe(buf, sink, stream=None):
    """Read every byte of the contiguous device tensor ``buf`` once (``sink`` is
    a one-element int32 device tensor)."""
    import torch
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    status = lib().pa_read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                 _dev(sink, torch.int32, "sink"), _stream(stream))
    if status != 0:
        raise PaError(status, "pa_read_probe failed")


def pa_mfma_probe(sink, workgroups, iters, operand=1.0, stream=None):
    """Run ``workgroups`` x 8 waves of back-to-back fp16 matrix products
    (``iters`` iterations of four independent chains per wave); ``sink`` is a
    one-element int32 device tensor, set to 1 if any accumulator differs from
    its value for ``operand`` 1.0.  Returns the flops of the call."""
    import torch
    status = lib().pa_mfma_probe(_dev(sink, torch.int32, "sink"), int(workgroups), int(iters),
                                 float(operand), _stream(stream))
    if status != 0:
        raise PaError(status, "pa_mfma_probe failed")
    return int(workgroups) * int(iters) * MFMA_PROBE_FLOPS_PER_WG_ITER


def pa_range_probe(buf, range_bytes, soffset, voffsets, out, stream=None):
    """16-byte buffer loads from the contiguous device tensor ``buf`` through a
    resource of ``range_bytes``, at lane offsets ``voffsets`` (a list of at most
    64) plus the scalar offset ``soffset``; ``out`` (int32 device tensor of
    2 * len(voffsets) * 4 elements) receives what each lane's register load
    returned, then what its LDS-writing load put in LDS."""
    import torch
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    n = len(voffsets)
    if out.numel() != 2 * n * 4:
        raise ValueError("out must hold 2 * len(voffsets) * 4 int32 values")
    arr = (ctypes.c_uint32 * max(n, 1))(*[int(v) for v in voffsets])
    status = lib().pa_range_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                  int(range_bytes), int(soffset), arr, n, _dev(out, torch.int32, "out"),
                                  _stream(stream))
    if status != 0:
        raise PaError(status, "pa_range_probe failed")
