"""Helpers for the GPU parity tests: host <-> device copies of the seeded
inputs and the tolerance checks.  No arithmetic of the method lives here."""
import numpy as np
import torch


def dev_bf16(bits: np.ndarray, ld: int = None) -> torch.Tensor:
    """uint16 BF16 bits [r, c] -> GPU bfloat16 tensor, optionally inside a
    wider [r, ld] buffer whose padding holds a NaN sentinel."""
    bits = np.ascontiguousarray(bits)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    if ld is None or ld == bits.shape[1]:
        return t.cuda()
    buf = torch.full((bits.shape[0], ld), float("nan"), dtype=torch.bfloat16, device="cuda")
    buf[:, : bits.shape[1]] = t.cuda()
    return buf[:, : bits.shape[1]]


def dev_f32(a: np.ndarray, ld: int = None) -> torch.Tensor:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if ld is None or ld == a.shape[1]:
        return torch.from_numpy(a).cuda()
    buf = torch.full((a.shape[0], ld), float("nan"), dtype=torch.float32, device="cuda")
    buf[:, : a.shape[1]] = torch.from_numpy(a).cuda()
    return buf[:, : a.shape[1]]


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """GPU bfloat16 tensor -> uint16 bits (numpy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy()


def padded_out(rows: int, cols: int, ld: int, dtype) -> torch.Tensor:
    """Output view [rows, cols] inside a [rows, ld] buffer pre-filled with a
    sentinel (NaN) so that writes into the padding are caught."""
    buf = torch.full((rows, ld), float("nan"), dtype=dtype, device="cuda")
    return buf[:, :cols]


def padding_untouched(view: torch.Tensor) -> bool:
    base = view.as_strided((view.shape[0], view.stride(0)), (view.stride(0), 1))
    pad = base[:, view.shape[1]:]
    return bool(torch.isnan(pad.float()).all().item()) if pad.numel() else True


def assert_gemm_close(gpu: np.ndarray, L: np.ndarray, S: np.ndarray, rel: float = 1e-5, what=""):
    """|gpu - L| <= rel * S elementwise (S = sum |a b|), the FP32-accumulation
    error bound used for random operands."""
    err = np.abs(gpu.astype(np.float64) - L)
    bound = rel * S + 1e-30
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside {rel}*S; first at "
                             f"{tuple(i)}: gpu={gpu[tuple(i)]!r} ref={L[tuple(i)]!r} S={S[tuple(i)]!r}")


def assert_loss_close(gpu, ref, rel=1e-5, what="loss"):
    """|gpu - ref| <= rel * max(|ref|, 1): relative error with an absolute
    floor below |loss| = 1 (a row can have loss ~0)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    bound = rel * np.maximum(np.abs(ref), 1.0)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} bad; first at {tuple(i)} gpu={gpu[tuple(i)]} "
                             f"ref={ref[tuple(i)]}")
