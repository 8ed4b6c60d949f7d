"""The Python binding's checks of caller tensors, on the CPU: every buffer the kernels read
or write through a raw pointer is checked for dtype, shape, contiguity and device before
anything is launched, so a wrong caller buffer is a ValueError, not a device write past
the end of an allocation."""
import pytest

torch = pytest.importorskip("torch")

from chunked_gated_delta_kda_amd import check_decode_args, check_fwd_args  # noqa: E402

T, H, D, N = 40, 2, 128, 3


def _inputs():
    bf, f32 = torch.bfloat16, torch.float32
    return dict(q=torch.zeros(T, H, D, dtype=bf), k=torch.zeros(T, H, D, dtype=bf),
                v=torch.zeros(T, H, D, dtype=bf), g=torch.zeros(T, H, D, dtype=f32),
                beta=torch.zeros(T, H, dtype=f32),
                cu_seqlens=torch.tensor([0, 10, 25, T], dtype=torch.int32))


def test_fwd_good_buffers():
    a = _inputs()
    out = torch.empty(T, H, D)
    fin = torch.empty(N, H, D, D)
    assert check_fwd_args(**a, initial_state=torch.zeros(N, H, D, D), out=out, final_state=fin) == \
        (T, H, N, torch.float32)
    assert check_fwd_args(**a) == (T, H, N, torch.float32)
    # the input-byte diet forms: bf16 g, bf16 states
    a["g"] = a["g"].to(torch.bfloat16)
    sb = torch.zeros(N, H, D, D, dtype=torch.bfloat16)
    assert check_fwd_args(**a, initial_state=sb, final_state=sb.clone()) == (T, H, N, torch.bfloat16)


@pytest.mark.parametrize("name,bad", [
    ("out", lambda: torch.empty(T, H, D, dtype=torch.bfloat16)),          # half the bytes
    ("out", lambda: torch.empty(T - 1, H, D)),                            # one row short
    ("out", lambda: torch.empty(H, T, D).transpose(0, 1)),                # not contiguous
    ("final_state", lambda: torch.empty(N - 1, H, D, D)),
    ("final_state", lambda: torch.empty(N, H, D, D).transpose(2, 3)),
    ("initial_state", lambda: torch.empty(N, H, D, 64)),
    ("beta", lambda: torch.empty(T, H, dtype=torch.float64)),
    ("g", lambda: torch.empty(T, H, D, dtype=torch.float16)),
    ("final_state", lambda: torch.empty(N, H, D, D, dtype=torch.float16)),
    ("v", lambda: torch.empty(T, H, D)),
])
def test_fwd_rejects(name, bad):
    a = _inputs()
    a[name] = bad()
    with pytest.raises(ValueError, match=name):
        check_fwd_args(**a)


def test_fwd_rejects_mixed_state_dtypes():
    a = _inputs()
    with pytest.raises(ValueError, match="final_state"):
        check_fwd_args(**a, initial_state=torch.zeros(N, H, D, D), final_state=torch.empty(N, H, D, D,
                                                                                            dtype=torch.bfloat16))


def test_fwd_rejects_bad_offsets_vector():
    a = _inputs()
    a["cu_seqlens"] = torch.tensor([0, 10, 25, T], dtype=torch.int64)
    with pytest.raises(ValueError, match="cu_seqlens"):
        check_fwd_args(**a)
    a["cu_seqlens"] = torch.tensor([0], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens"):
        check_fwd_args(**a)


def _dec():
    bf, f32 = torch.bfloat16, torch.float32
    return dict(q=torch.zeros(N, H, D, dtype=bf), k=torch.zeros(N, H, D, dtype=bf),
                v=torch.zeros(N, H, D, dtype=bf), g=torch.zeros(N, H, D, dtype=f32),
                beta=torch.zeros(N, H, dtype=f32))


def test_decode_good_buffers():
    s = torch.zeros(N, H, D, D, dtype=torch.bfloat16)
    assert check_decode_args(**_dec(), state=s, out=torch.empty(N, H, D)) == (N, H, torch.bfloat16)
    assert check_decode_args(**_dec()) == (N, H, torch.float32)


@pytest.mark.parametrize("kw", [
    dict(out=torch.empty(N, H, D, dtype=torch.bfloat16)),
    dict(out=torch.empty(N, H, D - 1)),
    dict(state=torch.zeros(N, H, D, D), state_out=torch.zeros(N, H, D, D, dtype=torch.bfloat16)),
    dict(state=torch.zeros(N, H, D, D).transpose(2, 3)),
    dict(state_out=torch.zeros(N + 1, H, D, D)),
])
def test_decode_rejects(kw):
    with pytest.raises(ValueError):
        check_decode_args(**_dec(), **kw)
