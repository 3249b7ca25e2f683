"""Shared test inputs: degenerate weight blocks and helpers to move numpy
arrays to and from the GPU.  Seeded; no method arithmetic here."""
import numpy as np


def edge_matrix():
    """64 x 256 fp32 matrix mixing ordinary and degenerate blocks."""
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    W[0, :64] = 0.0                     # zero block
    W[1, :64] = -0.0                    # negative-zero block
    W[2, :64] = 1e-9                    # absmax under half the smallest fp16 subnormal
    W[3, :64] = rng.standard_normal(64) * 1e-6   # subnormal fp16 scale
    W[4, :64] = rng.standard_normal(64) * 1e3    # large scale
    W[5, 64:128] = 65519.0              # rounds to 65504
    W[6, :64] = rng.standard_normal(64).astype(np.float32) * np.float32(2.0 ** -14)
    W[7, :] = np.exp2(rng.integers(-30, 10, 256)).astype(np.float32) * \
        np.sign(rng.standard_normal(256)).astype(np.float32)
    W[8, :64] = 0.0
    W[8, 5] = 1.0                       # one nonzero in a block
    W[9, :64] = 1.0                     # constant block
    W[10, :64] = -1.0
    W[11, 128:192] = 2.0 ** -24         # smallest fp16 subnormal exactly
    W[12, 192:256] = 2.0 ** -25         # tie at half the smallest subnormal -> 0
    W[13, :] = 65504.0                  # largest finite half
    return W


def to_dev(a, torch, device):
    """numpy -> torch on `device`, keeping the bits (uint16 -> fp16/bf16 as asked)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits16(t, torch):
    """fp16/bf16 tensor -> numpy uint16 bit patterns."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)
