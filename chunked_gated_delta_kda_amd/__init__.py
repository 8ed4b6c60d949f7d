"""MI355X-native Kimi Delta Attention (KDA) forward.

``fwd`` marshals torch tensors into the C ABI of libkda.so (include/kda.h).
PyTorch only allocates device memory and provides the stream; every step of
the computation runs in the library's HIP kernels.
"""
import ctypes
import math

from . import native

__all__ = ["fwd", "decode", "workspace_bytes", "select_variant", "version", "native"]

HEAD_DIM = 128


def version():
    return native.load_library().kda_version().decode()


def workspace_bytes(num_seqs, total_tokens, num_heads, variant="auto"):
    return int(native.load_library().kda_workspace_bytes(num_seqs, total_tokens, num_heads,
                                                         native.VARIANTS[variant]))


def select_variant(num_seqs, total_tokens, num_heads):
    v = native.load_library().kda_select_variant(num_seqs, total_tokens, num_heads)
    return {b: a for a, b in native.VARIANTS.items()}[v]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def fwd(q, k, v, g, beta, scale=None, cu_seqlens=None, initial_state=None,
        output_final_state=True, *, variant="auto", out=None, final_state=None,
        workspace=None, stream=None, stage_events=None):
    """KDA forward on the current HIP device.

    q, k, v: bf16 [T, H, 128]; g: fp32 [T, H, 128] (log-decay, clamped at -5);
    beta: fp32 [T, H]; cu_seqlens: int32 [N+1] on the device or None (one sequence);
    initial_state: fp32 [N, H, 128, 128] or None.
    Returns (o fp32 [T, H, 128], final_state fp32 [N, H, 128, 128] or None).
    """
    import torch

    lib = native.load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda.fwd needs device tensors")
    T, H, Dk = q.shape
    if Dk != HEAD_DIM:
        raise ValueError("head_dim must be 128")
    for name, t, dt, shape in (("q", q, torch.bfloat16, (T, H, Dk)), ("k", k, torch.bfloat16, (T, H, Dk)),
                               ("v", v, torch.bfloat16, (T, H, Dk)), ("g", g, torch.float32, (T, H, Dk)),
                               ("beta", beta, torch.float32, (T, H))):
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name}: expected contiguous {dt} {shape} on {dev}, "
                             f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or cu_seqlens.dim() != 1 \
                or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens: expected a contiguous int32 vector on the device")
        N = cu_seqlens.shape[0] - 1
    else:
        N = 1
    if initial_state is not None:
        if initial_state.dtype != torch.float32 or tuple(initial_state.shape) != (N, H, Dk, Dk) \
                or not initial_state.is_contiguous() or initial_state.device != dev:
            raise ValueError("initial_state: expected contiguous fp32 [N, H, 128, 128]")
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((T, H, Dk), dtype=torch.float32, device=dev)
    if output_final_state and final_state is None:
        final_state = torch.empty((N, H, Dk, Dk), dtype=torch.float32, device=dev)
    if not output_final_state:
        final_state = None
    var = native.VARIANTS[variant]
    if workspace is None:
        nbytes = lib.kda_workspace_bytes(N, T, H, var)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    opt = native.KdaOptions(var, 0, ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None,
                            workspace.numel() if workspace is not None else 0, None, 0)
    if stage_events is not None:   # profiling: a ctypes array of hipEvent_t handles
        opt.n_stage_events = len(stage_events)
        opt.stage_events = ctypes.cast(stage_events, ctypes.POINTER(ctypes.c_void_p))
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    rc = lib.kda_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(cu_seqlens),
                        N, T, H, Dk, _ptr(initial_state), _ptr(out), _ptr(final_state),
                        ctypes.c_void_p(st.cuda_stream), ctypes.byref(opt))
    native.check(rc)
    return out, final_state


def decode(q, k, v, g, beta, scale=None, state=None, *, out=None, state_out="inplace", state_dtype=None,
           stream=None):
    """One recurrence step per sequence (decode) on the current HIP device.

    q, k, v: bf16 [N, H, 128] (one token per sequence); g: fp32 [N, H, 128];
    beta: fp32 [N, H]; state: [N, H, 128, 128] fp32 or bf16 (the BF16-state form), or
    None (zeros). state_out: "inplace" (update ``state``; a new tensor when state is
    None), None (state not written), or a tensor of the state's dtype.
    state_dtype: torch.float32 or torch.bfloat16; by default the dtype of ``state``
    (or of ``state_out``), else float32.
    Returns (o fp32 [N, H, 128], the updated state or None).
    """
    import torch

    lib = native.load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda.decode needs device tensors")
    N, H, Dk = q.shape
    if Dk != HEAD_DIM:
        raise ValueError("head_dim must be 128")
    for name, t, dt, shape in (("q", q, torch.bfloat16, (N, H, Dk)), ("k", k, torch.bfloat16, (N, H, Dk)),
                               ("v", v, torch.bfloat16, (N, H, Dk)), ("g", g, torch.float32, (N, H, Dk)),
                               ("beta", beta, torch.float32, (N, H))):
        if t.dtype != dt or tuple(t.shape) != shape or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name}: expected contiguous {dt} {shape} on {dev}, "
                             f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    if state_dtype is None:
        state_dtype = (state.dtype if state is not None else
                       state_out.dtype if isinstance(state_out, torch.Tensor) else torch.float32)
    codes = {torch.float32: native.STATE_DTYPES["f32"], torch.bfloat16: native.STATE_DTYPES["bf16"]}
    if state_dtype not in codes:
        raise ValueError("state_dtype: torch.float32 or torch.bfloat16")
    sshape = (N, H, Dk, Dk)
    for name, t in (("state", state), ("state_out", state_out)):
        if isinstance(t, torch.Tensor) and (t.dtype != state_dtype or tuple(t.shape) != sshape
                                            or not t.is_contiguous() or t.device != dev):
            raise ValueError(f"{name}: expected contiguous {state_dtype} {sshape} on {dev}")
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((N, H, Dk), dtype=torch.float32, device=dev)
    if isinstance(state_out, str):
        if state_out != "inplace":
            raise ValueError('state_out: "inplace", None or a tensor')
        state_out = state if state is not None else torch.empty(sshape, dtype=state_dtype, device=dev)
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    rc = lib.kda_decode_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), N, H, Dk,
                           _ptr(state), _ptr(state_out), _ptr(out), ctypes.c_void_p(st.cuda_stream),
                           codes[state_dtype])
    native.check(rc)
    return out, state_out
