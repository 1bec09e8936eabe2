"""Host <-> device marshalling for the GPU tests (no layer arithmetic here)."""
import numpy as np
import torch

import synth


def to_dev(a, dtype="f32"):
    """numpy -> cuda tensor.  bf16 data arrives as uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "bf16" and a.dtype in (np.float32, np.float64):
        return torch.from_numpy(synth.f32_to_bf16_bits(a.astype(np.float32)).view(np.int16)).view(
            torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def to_host(t):
    """cuda tensor -> numpy (bf16 widened exactly to float32)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def f64(a, dtype):
    """The float64 values the layer sees for an input array."""
    return synth.as_f32(a, dtype).astype(np.float64)
