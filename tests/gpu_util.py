"""Helpers shared by the GPU parity tests: host <-> device copies and the
comparisons the parity bar uses.  No arithmetic of the method lives here."""
import numpy as np
import torch

DEV = torch.device("cuda:0")


def to_dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(DEV)


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.cpu().numpy()


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def singular_values(x):
    x = np.asarray(x, np.float64)
    if x.shape[0] > x.shape[1]:
        x = x.T
    return np.sqrt(np.clip(np.linalg.eigvalsh(x @ x.T), 0, None))[::-1]


def same_band(x, y, tol=0.05):
    """Sorted singular values agree within tol, endpoint by endpoint."""
    sx, sy = singular_values(x), singular_values(y)
    return float(np.max(np.abs(sx - sy))), (sx[0], sx[-1]), (sy[0], sy[-1])
