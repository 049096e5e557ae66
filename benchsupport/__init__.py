"""Reference kernels used by bench.py: streaming-read ceiling and a known-size copy."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(HERE, "libbenchsupport.so")
_lib = None


def build():
    import subprocess
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "stream.hip",
           "-o", SO + ".tmp"]
    r = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("benchsupport build failed:\n" + r.stderr)
    os.replace(SO + ".tmp", SO)


def lib():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (bind to torch's HIP runtime)
        if not os.path.exists(SO):
            raise RuntimeError("libbenchsupport.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(SO)
        L.bs_stream_read.restype = ctypes.c_int
        L.bs_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.c_void_p]
        L.bs_copy.restype = ctypes.c_int
        L.bs_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                              ctypes.c_void_p]
        _lib = L
    return _lib


def stream_read(buf, sink, blocks, stream):
    rc = lib().bs_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                              blocks, stream)
    if rc:
        raise RuntimeError("bs_stream_read failed (%d)" % rc)


def copy(src, dst, blocks, stream):
    rc = lib().bs_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(), blocks,
                       stream)
    if rc:
        raise RuntimeError("bs_copy failed (%d)" % rc)
