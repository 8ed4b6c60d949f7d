"""ctypes binding of libkda.so (include/kda.h). Argument marshalling only.

Loading fails loudly when the library has not been built; there is no other
compute path.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# KDA_LIB points at an alternative build of the same library (tuning experiments)
LIB_PATH = os.environ.get("KDA_LIB") or os.path.join(PKG, "libkda.so")

KDA_OK = 0
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_UNSUPPORTED",
          4: "KDA_ERR_ALLOC", 5: "KDA_ERR_LAUNCH", 6: "KDA_ERR_DEVICE", 7: "KDA_ERR_ALIAS",
          8: "KDA_ERR_SCRATCH"}
VARIANTS = {"auto": 0, "split": 1, "fused": 2, "recurrent": 3}

#: every symbol include/kda.h declares
EXPORTS = ("kda_fwd", "kda_fwd_ex", "kda_fwd_noalloc", "kda_workspace_bytes", "kda_select_variant",
           "kda_launch_plan", "kda_decode", "kda_decode_ex", "kda_bwd", "kda_bwd_workspace_bytes",
           "kda_device_errors", "kda_status_string", "kda_version")
#: KDA_DEVERR_* bits of the device error word
DEVERR = {1: "fused hand-off wait gave up (outputs invalid)", 2: "malformed cu_seqlens (sanitised)"}
STATE_DTYPES = {"f32": 0, "bf16": 1}
DTYPES = STATE_DTYPES   # KDA_DTYPE_* of kda_options.g_dtype / state_dtype
SEGMENT_ONE = 65536   # KDA_SEGMENT_ONE: unit of the launch plan's segment fractions
NOALLOC_MAX_SEQS = 16384   # KDA_NOALLOC_MAX_SEQS
KERNEL_KINDS = {0: "chunk_map", 1: "prep", 2: "recur", 3: "fused", 4: "recur_prep", 5: "recurrent", 6: "parts"}


class KdaOptions(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("n_stage_events", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stage_events", ctypes.POINTER(ctypes.c_void_p)), ("g_dtype", ctypes.c_int32),
                ("state_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class KdaLaunchInfo(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("prep_begin", ctypes.c_int32), ("prep_end", ctypes.c_int32),
                ("recur_begin", ctypes.c_int32), ("recur_end", ctypes.c_int32),
                ("chunk_len", ctypes.c_int32)]


class KdaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path=LIB_PATH):
    """Load libkda.so; raises if it is missing (build it with chunked_gated_delta_kda_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m chunked_gated_delta_kda_amd.build`")
    # Load torch's HIP runtime first: libkda.so then binds to that same runtime
    # (same SONAME), so torch streams and events are valid handles for the library.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the library also works without torch
        pass
    lib = ctypes.CDLL(path)
    vp, i32, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p
    fwd_args = [vp, vp, vp, f32p, f32p, ctypes.c_float, vp, i32, i32, i32, i32, f32p, f32p, f32p, vp]
    lib.kda_fwd.argtypes = fwd_args
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_fwd_ex.argtypes = fwd_args + [ctypes.POINTER(KdaOptions)]
    lib.kda_fwd_ex.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = fwd_args
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.kda_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_select_variant.argtypes = [i32, i32, i32]
    lib.kda_select_variant.restype = ctypes.c_int
    lib.kda_launch_plan.argtypes = [i32, i32, i32, i32, ctypes.POINTER(KdaLaunchInfo), i32]
    lib.kda_launch_plan.restype = ctypes.c_int32
    lib.kda_decode.argtypes = [vp, vp, vp, f32p, f32p, ctypes.c_float, i32, i32, i32, f32p, f32p, f32p, vp]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode_ex.argtypes = [vp, vp, vp, f32p, f32p, ctypes.c_float, i32, i32, i32, vp, vp, f32p, vp, i32]
    lib.kda_decode_ex.restype = ctypes.c_int
    lib.kda_bwd.argtypes = [vp, vp, vp, f32p, f32p, ctypes.c_float, vp, i32, i32, i32, i32, f32p, f32p, f32p,
                            f32p, f32p, f32p, f32p, f32p, f32p, vp, vp, ctypes.c_size_t]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_bwd_workspace_bytes.argtypes = [i32, i32, i32]
    lib.kda_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_device_errors.argtypes = [vp, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]
    lib.kda_device_errors.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status):
    return load_library().kda_status_string(status).decode()


def check(status):
    if status != KDA_OK:
        raise KdaError(status, status_string(status))


class KdaDeviceError(RuntimeError):
    def __init__(self, bits):
        names = [m for b, m in DEVERR.items() if bits & b]
        super().__init__(f"device error bits {bits}: {'; '.join(names)}")
        self.bits = bits


def device_errors(stream_handle=None, clear=True):
    """The device error word (KDA_DEVERR_* bits) of the current device, after
    synchronising ``stream_handle`` (a hipStream_t as int, or None); cleared when
    ``clear``."""
    bits = ctypes.c_int32(0)
    check(load_library().kda_device_errors(ctypes.c_void_p(stream_handle), ctypes.byref(bits), int(clear)))
    return bits.value


def error_word_offset(num_seqs):
    """Byte offset of the device error word inside a kda_fwd_ex workspace. After a call
    it holds 0, or bit 0 (1): a fused-kernel wait gave up and the outputs are not valid,
    or bit 1 (2): cu_seqlens was not 0 = c_0 <= ... <= c_N = T (the offsets were clamped
    to [0, T] and made non-decreasing before use)."""
    a = lambda x: (x + 255) // 256 * 256
    return a(4 * (num_seqs + 1)) + a(4 * num_seqs)


def launch_plan(num_seqs, total_tokens, num_heads, variant="auto"):
    """Kernel launches one kda_fwd_ex call makes for this shape, in order: a list of
    (kind name, (prep_begin, prep_end), (recur_begin, recur_end), chunk_len). A range is
    a segment: a fraction of every sequence in units of 1/SEGMENT_ONE (of a sequence with
    c chunks, chunks c*begin//SEGMENT_ONE to c*end//SEGMENT_ONE - 1)."""
    lib = load_library()
    info = (KdaLaunchInfo * 64)()
    n = lib.kda_launch_plan(num_seqs, total_tokens, num_heads, VARIANTS[variant], info, 64)
    return [(KERNEL_KINDS[x.kind], (x.prep_begin, x.prep_end), (x.recur_begin, x.recur_end), x.chunk_len)
            for x in info[:n]]
