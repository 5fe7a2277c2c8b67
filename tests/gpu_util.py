"""Helpers for the GPU parity tests: device upload, the library handle, and
a marker that every GPU case prints (and flushes) before it launches."""
import sys

import numpy as np


def announce(msg: str):
    print(f"[gpu case] {msg}", flush=True)
    sys.stdout.flush()


def cuda(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32))).to("cuda:0")


def host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.detach().to("cpu").numpy().astype(np.float64)


def cuda_dict(d):
    return {k: cuda(v) for k, v in d.items()}
