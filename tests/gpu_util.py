"""Host <-> device conversion for GPU tests (numpy arrays from the generator,
bf16 kept as uint16 bit patterns on the host)."""
import os
import sys

import numpy as np


def torch():
    import torch as t
    return t


def announce(what):
    """Name the case (and report measured errors) on the process's stderr, which
    output capture does not hold back; also appended to the file named by
    WKV7_TEST_LOG when that is set."""
    sys.__stderr__.write(f"[gpu] {what}\n")
    sys.__stderr__.flush()
    path = os.environ.get("WKV7_TEST_LOG")
    if path:
        with open(path, "a") as f:
            f.write(f"{what}\n")


def to_dev(x):
    t = torch()
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return t.from_numpy(x.view(np.int16)).view(t.bfloat16).cuda()
    return t.from_numpy(x).cuda()


def to_host(tensor):
    """Device tensor -> float64 numpy (bf16 widened exactly)."""
    t = torch()
    if tensor.dtype == t.bfloat16:
        bits = tensor.view(t.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return tensor.cpu().numpy().astype(np.float64)


def dev_inputs(x):
    return {k: to_dev(v) for k, v in x.items()}
