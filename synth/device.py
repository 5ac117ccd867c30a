"""Device-side fill of synthetic expert blobs (libcolisynth.so), identical to
synth.expert_blob() byte for byte. Used for workloads too large to generate on
the host; the CPU side regenerates any single expert with synth.expert_blob()."""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcolisynth.so")


def build() -> str:
    tmp = LIB_PATH + ".tmp"
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", os.path.join(HERE, "gen_device.hip"), "-o", tmp], check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        L.coli_synth_fill_blobs.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_void_p]
        L.coli_synth_fill_blobs.restype = C.c_int
        L.coli_synth_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
        L.coli_synth_copy.restype = C.c_int
        L.coli_synth_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]
        L.coli_synth_read.restype = C.c_int
        L.coli_synth_read_sink_words.restype = C.c_int
        L.coli_synth_scaled_mfma.argtypes = [C.c_void_p, C.c_int32, C.c_void_p]
        L.coli_synth_scaled_mfma.restype = C.c_int
        L.coli_synth_scaled_mfma_out_words.restype = C.c_int
        L.coli_synth_scaled_mfma_ops.argtypes = [C.c_int32]
        L.coli_synth_scaled_mfma_ops.restype = C.c_double
        _lib = L
    return _lib


def fill_blobs(out, seed: int, layer: int, first_expert: int, n_blobs: int, blob_bytes: int, wbits: int):
    """Fill the uint8 CUDA tensor ``out`` ([n_blobs * blob_bytes]) with blobs of experts
    first_expert .. first_expert + n_blobs - 1 of (seed, layer)."""
    import torch

    assert out.is_cuda and out.dtype == torch.uint8 and out.is_contiguous()
    assert out.numel() >= n_blobs * blob_bytes
    keys = np.array([synth.derive_key(seed, synth.TAG_BLOB, layer, first_expert + i) for i in range(n_blobs)],
                    dtype=np.uint64)
    kd = torch.from_numpy(keys.view(np.int64)).to(out.device)
    stream = torch.cuda.current_stream(out.device).cuda_stream
    rc = lib().coli_synth_fill_blobs(C.c_void_p(out.data_ptr()), C.c_void_p(kd.data_ptr()), blob_bytes, n_blobs,
                                     wbits, C.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"coli_synth_fill_blobs failed: {rc}")
    torch.cuda.current_stream(out.device).synchronize()  # keys tensor lifetime


def copy(src, dst, stream=None):
    """Streaming device copy of ``src`` into ``dst`` (same byte size, multiple of 16):
    the reference kernel of known traffic for scaling hardware byte counters."""
    import torch

    assert src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()
    nbytes = src.numel() * src.element_size()
    assert nbytes == dst.numel() * dst.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(src.device)
    rc = lib().coli_synth_copy(C.c_void_p(src.data_ptr()), C.c_void_p(dst.data_ptr()), nbytes, C.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"coli_synth_copy failed: {rc}")


def read_sink(device):
    """A device buffer for read()'s per-wavefront words."""
    import torch
    return torch.empty(lib().coli_synth_read_sink_words(), dtype=torch.int32, device=device)


def read(src, sink, stream=None):
    """Streaming device read of ``src`` (byte size a multiple of 16): the measured read
    bandwidth ceiling. ``sink`` from read_sink() receives one word per wavefront."""
    import torch

    assert src.is_cuda and src.is_contiguous() and sink.is_cuda
    assert sink.numel() * sink.element_size() >= 4 * lib().coli_synth_read_sink_words()
    nbytes = src.numel() * src.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(src.device)
    rc = lib().coli_synth_read(C.c_void_p(src.data_ptr()), nbytes, C.c_void_p(sink.data_ptr()),
                               C.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"coli_synth_read failed: {rc}")


def scaled_mfma_out(device):
    """A device buffer for scaled_mfma()'s per-thread results."""
    import torch
    return torch.empty(lib().coli_synth_scaled_mfma_out_words(), dtype=torch.float32, device=device)


def scaled_mfma_ops(iters: int) -> float:
    """int8 operations of one scaled_mfma launch."""
    return float(lib().coli_synth_scaled_mfma_ops(iters))


def scaled_mfma(out, iters: int, stream=None):
    """int8 matrix-core loop with every block dot converted to fp32 and multiply-added
    with a scale: the device's rate for exactly scaled Q8_0 block dots."""
    import torch

    assert out.is_cuda and out.dtype == torch.float32
    assert out.numel() >= lib().coli_synth_scaled_mfma_out_words()
    s = stream if stream is not None else torch.cuda.current_stream(out.device)
    rc = lib().coli_synth_scaled_mfma(C.c_void_p(out.data_ptr()), iters, C.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"coli_synth_scaled_mfma failed: {rc}")
