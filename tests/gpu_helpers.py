"""Helpers for the GPU parity tests: host <-> device marshalling and case announcements."""

import sys

import numpy as np


def announce(msg: str):
    """Name the case on the real stderr (visible under pytest capture) before a GPU step."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def to_device(p: dict):
    import torch
    dev = torch.device("cuda", 0)
    x = torch.from_numpy(np.ascontiguousarray(p["x"]).view(np.int16)).view(torch.bfloat16).to(dev)
    wq = torch.from_numpy(np.ascontiguousarray(p["wq"]).view(np.int32)).to(dev)
    s = torch.from_numpy(np.ascontiguousarray(p["scales"]).view(np.int16)).view(torch.bfloat16).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(p["biases"]).view(np.int16)).view(torch.bfloat16).to(dev)
    return x, wq, s, b


def bits(y) -> np.ndarray:
    """bf16 torch tensor -> numpy uint16 bit patterns (synchronizes)."""
    import torch
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_from_bits(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to("cuda:0")
