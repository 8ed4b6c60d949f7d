"""MI355X-native Kimi Delta Attention (KDA) forward.

``fwd`` marshals torch tensors into the C ABI of libkda.so (include/kda.h).
PyTorch only allocates device memory and provides the stream; every step of
the computation runs in the library's HIP kernels.
"""
import ctypes
import math

from . import native

__all__ = ["fwd", "fwd_noalloc", "bwd", "decode", "workspace_bytes", "select_variant", "device_errors", "version", "native"]

HEAD_DIM = 128


def version():
    return native.load_library().kda_version().decode()


def workspace_bytes(num_seqs, total_tokens, num_heads, variant="auto"):
    return int(native.load_library().kda_workspace_bytes(num_seqs, total_tokens, num_heads,
                                                         native.VARIANTS[variant]))


def device_errors(clear=True, stream=None):
    """KDA_DEVERR_* bits raised on the current device since the last clear (synchronises
    ``stream``, by default torch's current stream)."""
    import torch

    st = stream if stream is not None else torch.cuda.current_stream()
    return native.device_errors(st.cuda_stream, clear=clear)


def select_variant(num_seqs, total_tokens, num_heads):
    v = native.load_library().kda_select_variant(num_seqs, total_tokens, num_heads)
    return {b: a for a, b in native.VARIANTS.items()}[v]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _expect(name, t, dtype, shape, dev):
    """Raise unless ``t`` is a contiguous ``dtype`` tensor of ``shape`` on ``dev``: the
    kernels write whole rows through raw pointers, so a wrong buffer must be caught here."""
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != dev:
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {dev}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}"
                         f"{'' if t.is_contiguous() else ' (not contiguous)'}")


def check_fwd_args(q, k, v, g, beta, cu_seqlens=None, initial_state=None, out=None, final_state=None,
                   state_dtype=None):
    """Every check fwd makes on its tensors before anything is launched (dtype, shape,
    contiguity, one device); returns (T, H, N, state dtype). g may be fp32 or bf16 (the
    input-byte diet form); initial and final state share one dtype, fp32 or bf16 (by
    default that of initial_state, else of final_state, else fp32)."""
    import torch

    dev = q.device
    if q.dim() != 3:
        raise ValueError("q: expected [T, H, 128]")
    T, H, Dk = q.shape
    if Dk != HEAD_DIM:
        raise ValueError("head_dim must be 128")
    gdt = g.dtype if g.dtype in (torch.float32, torch.bfloat16) else torch.float32
    for name, t, dt, shape in (("q", q, torch.bfloat16, (T, H, Dk)), ("k", k, torch.bfloat16, (T, H, Dk)),
                               ("v", v, torch.bfloat16, (T, H, Dk)), ("g", g, gdt, (T, H, Dk)),
                               ("beta", beta, torch.float32, (T, H))):
        _expect(name, t, dt, shape, dev)
    if state_dtype is None:
        state_dtype = (initial_state.dtype if initial_state is not None else
                       final_state.dtype if final_state is not None else torch.float32)
    if state_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"states: dtype {state_dtype}; initial_state and final_state must be fp32 or bf16")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.device != dev or cu_seqlens.dim() != 1 \
                or not cu_seqlens.is_contiguous() or cu_seqlens.shape[0] < 2:
            raise ValueError("cu_seqlens: expected a contiguous int32 vector of N+1 >= 2 offsets on the device")
        N = cu_seqlens.shape[0] - 1
    else:
        N = 1
    if initial_state is not None:
        _expect("initial_state", initial_state, state_dtype, (N, H, Dk, Dk), dev)
    if out is not None:
        _expect("out", out, torch.float32, (T, H, Dk), dev)
    if final_state is not None:
        _expect("final_state", final_state, state_dtype, (N, H, Dk, Dk), dev)
    return T, H, N, state_dtype


def fwd(q, k, v, g, beta, scale=None, cu_seqlens=None, initial_state=None,
        output_final_state=True, *, variant="auto", out=None, final_state=None,
        workspace=None, stream=None, stage_events=None, check=False, state_dtype=None):
    """KDA forward on the current HIP device.

    q, k, v: bf16 [T, H, 128]; g: fp32 or bf16 [T, H, 128] (log-decay, clamped at -5);
    beta: fp32 [T, H]; cu_seqlens: int32 [N+1] on the device or None (one sequence);
    initial_state: [N, H, 128, 128] fp32 or bf16, or None; out: fp32 [T, H, 128] caller
    buffer or None; final_state: caller buffer of the state dtype or None. state_dtype
    (torch.float32 or torch.bfloat16): the states' dtype, by default that of the given
    states, else fp32. bf16 g or states run the split variant's 32-token forms or the
    token loop (the fused variant rejects them).
    check: clear the device error word before the call and read it after (both
    synchronise the stream); raise native.KdaDeviceError if the kernels raised a bit
    (malformed cu_seqlens, a fused hand-off timeout).
    Returns (o fp32 [T, H, 128], final_state fp32 [N, H, 128, 128] or None).
    """
    import torch

    lib = native.load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda.fwd needs device tensors")
    T, H, N, sdt = check_fwd_args(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, state_dtype)
    Dk = HEAD_DIM
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    if out is None:
        out = torch.empty((T, H, Dk), dtype=torch.float32, device=dev)
    if not output_final_state:
        final_state = None
    elif final_state is None:
        final_state = torch.empty((N, H, Dk, Dk), dtype=sdt, device=dev)
    dtypes = {torch.float32: native.DTYPES["f32"], torch.bfloat16: native.DTYPES["bf16"]}
    var = native.VARIANTS[variant]
    if workspace is None:
        nbytes = lib.kda_workspace_bytes(N, T, H, var)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    opt = native.KdaOptions(variant=var, n_stage_events=0,
                            workspace=ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None,
                            workspace_bytes=workspace.numel() * workspace.element_size() if workspace is not None
                            else 0,
                            g_dtype=dtypes[g.dtype], state_dtype=dtypes[sdt])
    if stage_events is not None:   # profiling: a ctypes array of hipEvent_t handles
        opt.n_stage_events = len(stage_events)
        opt.stage_events = ctypes.cast(stage_events, ctypes.POINTER(ctypes.c_void_p))
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    if check:
        native.device_errors(st.cuda_stream, clear=True)
    rc = lib.kda_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(cu_seqlens),
                        N, T, H, Dk, _ptr(initial_state), _ptr(out), _ptr(final_state),
                        ctypes.c_void_p(st.cuda_stream), ctypes.byref(opt))
    native.check(rc)
    if check:
        bits = native.device_errors(st.cuda_stream, clear=True)
        if bits:
            raise native.KdaDeviceError(bits)
    return out, final_state


def check_bwd_args(q, k, v, g, beta, d_out, cu_seqlens=None, initial_state=None, d_final_state=None):
    """Every check bwd makes on its inputs before anything is launched; returns (T, H, N).
    The backward reads g, the states and the gradients in fp32."""
    import torch

    T, H, N, _ = check_fwd_args(q, k, v, g, beta, cu_seqlens, initial_state, state_dtype=torch.float32)
    dev = q.device
    _expect("g", g, torch.float32, (T, H, HEAD_DIM), dev)
    _expect("d_out", d_out, torch.float32, (T, H, HEAD_DIM), dev)
    if d_final_state is not None:
        _expect("d_final_state", d_final_state, torch.float32, (N, H, HEAD_DIM, HEAD_DIM), dev)
    return T, H, N


def bwd(q, k, v, g, beta, d_out, scale=None, cu_seqlens=None, initial_state=None, d_final_state=None, *,
        need_d_initial_state=True, workspace=None, stream=None):
    """Gradients of fwd (kda_bwd): given d_out = dL/do (fp32 [T, H, 128]) and optionally
    d_final_state = dL/dS_final (fp32 [N, H, 128, 128]), returns a dict of fp32 tensors dq,
    dk, dv, dg ([T, H, 128]), dbeta ([T, H]) and d_initial_state ([N, H, 128, 128], or None
    when need_d_initial_state is False). Inputs as for fwd, with g and initial_state fp32."""
    import torch

    lib = native.load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda.bwd needs device tensors")
    T, H, N = check_bwd_args(q, k, v, g, beta, d_out, cu_seqlens, initial_state, d_final_state)
    Dk = HEAD_DIM
    if scale is None:
        scale = 1.0 / math.sqrt(Dk)
    f32 = dict(dtype=torch.float32, device=dev)
    gr = dict(dq=torch.empty((T, H, Dk), **f32), dk=torch.empty((T, H, Dk), **f32),
              dv=torch.empty((T, H, Dk), **f32), dg=torch.empty((T, H, Dk), **f32),
              dbeta=torch.empty((T, H), **f32),
              d_initial_state=torch.empty((N, H, Dk, Dk), **f32) if need_d_initial_state else None)
    if workspace is None:
        workspace = torch.empty(lib.kda_bwd_workspace_bytes(N, T, H), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    rc = lib.kda_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(cu_seqlens), N, T, H, Dk,
                     _ptr(initial_state), _ptr(d_out), _ptr(d_final_state), _ptr(gr["dq"]), _ptr(gr["dk"]),
                     _ptr(gr["dv"]), _ptr(gr["dg"]), _ptr(gr["dbeta"]), _ptr(gr["d_initial_state"]),
                     ctypes.c_void_p(st.cuda_stream), _ptr(workspace), workspace.numel() * workspace.element_size())
    native.check(rc)
    return gr


def check_decode_args(q, k, v, g, beta, state=None, state_out="inplace", out=None, state_dtype=None):
    """Every check decode makes on its tensors before the launch; returns (N, H, state dtype)."""
    import torch

    dev = q.device
    if q.dim() != 3:
        raise ValueError("q: expected [N, H, 128]")
    N, H, Dk = q.shape
    if Dk != HEAD_DIM:
        raise ValueError("head_dim must be 128")
    for name, t, dt, shape in (("q", q, torch.bfloat16, (N, H, Dk)), ("k", k, torch.bfloat16, (N, H, Dk)),
                               ("v", v, torch.bfloat16, (N, H, Dk)), ("g", g, torch.float32, (N, H, Dk)),
                               ("beta", beta, torch.float32, (N, H))):
        _expect(name, t, dt, shape, dev)
    if state_dtype is None:
        state_dtype = (state.dtype if state is not None else
                       state_out.dtype if isinstance(state_out, torch.Tensor) else torch.float32)
    if state_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("state_dtype: torch.float32 or torch.bfloat16")
    for name, t in (("state", state), ("state_out", state_out)):
        if isinstance(t, torch.Tensor):
            _expect(name, t, state_dtype, (N, H, Dk, Dk), dev)
    if out is not None:
        _expect("out", out, torch.float32, (N, H, Dk), dev)
    return N, H, state_dtype


def fwd_noalloc(q, k, v, g, beta, scale=None, cu_seqlens=None, initial_state=None, *, out, final_state=None,
                stream=None):
    """KDA forward through kda_fwd_noalloc: the library allocates nothing (its kernels use a
    fixed per-device scratch; at most native.NOALLOC_MAX_SEQS sequences). The caller passes
    the outputs: ``out`` fp32 [T, H, 128] and, optionally, ``final_state`` fp32
    [N, H, 128, 128]. Calls that overlap in time on one device race on the scratch.
    Returns (out, final_state)."""
    import torch

    lib = native.load_library()
    if q.device.type != "cuda":
        raise ValueError("kda.fwd_noalloc needs device tensors")
    T, H, N, sdt = check_fwd_args(q, k, v, g, beta, cu_seqlens, initial_state, out, final_state)
    if g.dtype != torch.float32 or sdt != torch.float32:
        raise ValueError("fwd_noalloc: fp32 g and states only (it runs the fused variant)")
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    rc = lib.kda_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale), _ptr(cu_seqlens),
                             N, T, H, HEAD_DIM, _ptr(initial_state), _ptr(out), _ptr(final_state),
                             ctypes.c_void_p(st.cuda_stream))
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
    N, H, state_dtype = check_decode_args(q, k, v, g, beta, state, state_out, out, state_dtype)
    Dk = HEAD_DIM
    codes = {torch.float32: native.STATE_DTYPES["f32"], torch.bfloat16: native.STATE_DTYPES["bf16"]}
    sshape = (N, H, Dk, Dk)
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
