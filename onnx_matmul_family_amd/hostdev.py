"""Host <-> device copies of the seeded inputs and of results.

numpy has no bfloat16, so bf16 data travels as uint16 bit patterns: `dev`
reinterprets them as a torch bfloat16 tensor on the GPU, `host_f64` turns any
float result (bf16 / fp16 / fp32 / fp64) back into exact float64 values.
Copies only: no arithmetic of the operators happens here.
"""
import numpy as np
import torch

from . import synth


def dev(arr, dt=None):
    """numpy array -> GPU tensor (bf16 arrays are uint16 bit patterns, pass dt='bf16')."""
    arr = np.ascontiguousarray(arr)
    if dt == "bf16":
        return torch.from_numpy(arr.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(arr.copy()).cuda()


def host_f64(t):
    """GPU tensor -> float64 numpy (exact for bf16 / fp16 / fp32 / fp64)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_to_f32(bits).astype(np.float64).reshape(t.shape)
    return t.cpu().numpy().astype(np.float64)


def host_f32(t):
    """GPU tensor of bf16 / fp16 / fp32 -> float32 numpy (exact; half the memory of host_f64)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return synth.bf16_to_f32(bits).reshape(t.shape)
    return t.float().cpu().numpy()
