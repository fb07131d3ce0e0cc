"""Helpers shared by the GPU tests: moving seeded numpy inputs to the device
and comparing results with the oracle's."""
import numpy as np
import torch

import oracle as O


def dev(a):
    """numpy (float32, or uint16 bf16 bits, or uint32 codes) -> cuda tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return torch.from_numpy(a).cuda()
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).cuda()
    raise TypeError(a.dtype)


def host(t):
    """cuda tensor -> numpy in the same representation `dev` takes."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    raise TypeError(t.dtype)


def values(a):
    """float64 values of a float32 or bf16-bits array."""
    if a.dtype == np.uint16:
        return O.bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def tolerance(y_dtype):
    """Per-row bound on max_n |y - y_ref| / max_n |y_ref|."""
    return 1e-3 if y_dtype in (np.float32, torch.float32) else 1e-2


def assert_rows_close(y, y_ref, tol, what=""):
    """y [.., n] (numpy values) against the fp64 oracle, row by row."""
    y = np.asarray(y, dtype=np.float64).reshape(-1, y_ref.shape[-1])
    r = np.asarray(y_ref, dtype=np.float64).reshape(-1, y_ref.shape[-1])
    assert y.shape == r.shape
    assert np.all(np.isfinite(y)), what
    for i in range(r.shape[0]):
        den = np.max(np.abs(r[i]))
        err = np.max(np.abs(y[i] - r[i]))
        if den == 0:
            assert err == 0, (what, i, err)
        else:
            assert err / den <= tol, (what, i, err / den)


def bits_equal(a, b):
    return a.shape == b.shape and bool(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16
                                                  else a.view(torch.int32),
                                                  b.view(torch.int16) if b.dtype == torch.bfloat16
                                                  else b.view(torch.int32)))
