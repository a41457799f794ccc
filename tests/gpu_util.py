"""Helpers for GPU tests: moving seeded inputs to the device, poison fills, ulp distances."""
import numpy as np
import torch

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
NAN_BITS = {"f32": 0x7FC00000, "bf16": 0x7FC0}


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32/float64 numpy -> device tensor of the storage type (torch's RNE cast)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(TORCH_DTYPE[dtype]).cuda()


def host64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (exact for bf16 and f32)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def poisoned(shape, dtype: str) -> torch.Tensor:
    """A device tensor every element of which is a quiet NaN."""
    if dtype == "bf16":
        return torch.full(shape, NAN_BITS["bf16"], dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns as int64 numpy (for bit-exact comparisons)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().astype(np.int64) & 0xFFFF
    return t.view(torch.int32).cpu().numpy().astype(np.int64) & 0xFFFFFFFF


def ulp_distance(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """|a - b| in units in the last place of the storage type (a, b float64 holding storage values)."""
    if dtype == "bf16":
        ia = (a.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
        ib = (b.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
        sign = 0x8000
    else:
        ia = a.astype(np.float32).view(np.uint32).astype(np.int64)
        ib = b.astype(np.float32).view(np.uint32).astype(np.int64)
        sign = 0x80000000
    # map sign-magnitude to a monotonic integer line
    ia = np.where(ia & sign, -(ia & (sign - 1)), ia)
    ib = np.where(ib & sign, -(ib & (sign - 1)), ib)
    return np.abs(ia - ib)


def make_cache(kvc, n_layers, batch, max_seq, n_kv, d, dtype: str, poison=True):
    shape = (n_layers, batch, max_seq, n_kv, d)
    if poison:
        k, v = poisoned(shape, dtype), poisoned(shape, dtype)
    else:
        k = torch.zeros(shape, dtype=TORCH_DTYPE[dtype], device="cuda")
        v = torch.zeros(shape, dtype=TORCH_DTYPE[dtype], device="cuda")
    return kvc.KVCache(k, v, torch.zeros(batch, dtype=torch.int32, device="cuda"))


def _rope_err(got: np.ndarray, ref: np.ndarray, x_in: np.ndarray, dtype: str):
    half = x_in.shape[-1] // 2
    pair = np.sqrt(x_in[..., :half] ** 2 + x_in[..., half:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1)
    _, e = np.frexp(np.abs(ref))
    ulp = np.ldexp(1.0, e - (8 if dtype == "bf16" else 24))
    return np.abs(got - ref), ulp, pair


def rope_error_ok(got: np.ndarray, ref: np.ndarray, x_in: np.ndarray, dtype: str) -> bool:
    """Is a rotated vector within the error a float32 rotation can have?

    The kernel rotates in float32 with float32 cos/sin (each within an ulp),
    so an output's error scales with the pair's length |(a, b)|, not with the
    output itself (which may be tiny by cancellation).  Allowed: one ulp of
    the storage type at the output, or 2^-20 |(a, b)|, whichever is larger.
    x_in: the unrotated input (..., D) in storage precision.
    """
    err, ulp, pair = _rope_err(got, ref, x_in, dtype)
    return bool(np.all(err <= np.maximum(ulp, pair * 2.0 ** -20)))


def rope_excess_ratio(got: np.ndarray, ref: np.ndarray, x_in: np.ndarray, dtype: str):
    """How close a rotated tensor comes to the 2^-20 |(a, b)| allowance: the largest
    |got - ref| / |(a, b)| over the elements that are more than one storage ulp off, and how
    many such elements there are ((0.0, 0) when every element is within an ulp)."""
    err, ulp, pair = _rope_err(got, ref, x_in, dtype)
    over = err > ulp
    if not np.any(over):
        return 0.0, 0
    return float(np.max(err[over] / pair[over])), int(np.count_nonzero(over))
