"""Helpers for GPU parity tests: move seeded numpy inputs onto the device in
their storage dtype, and bring results back as float64."""
import numpy as np
import torch

TOL = {"bf16": 2e-3, "f32": 1e-5}


def dev(x, dtype):
    """float64 numpy array holding exactly-representable values -> device tensor."""
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def dev_f32(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def flush(msg):
    print(msg, flush=True)
