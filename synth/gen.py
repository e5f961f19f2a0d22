"""Counter-free seeded generators built on torch's own RNG.

Every tensor is named by ``(workload_id, tensor_id, slot)``; its seed depends
on nothing else, so a tensor can be regenerated alone and a batch of B rows is
drawn one row (``slot``) at a time, which bounds host/device temporaries to a
single sequence.  The generator runs on whatever device it is given.  A given
test or benchmark draws each tensor once and hands the very same bytes to both
sides (the HIP path and the CPU oracle), so CPU and GPU streams never need to
agree with each other.

Storage formats:

* ``f32``  – IEEE binary32.
* ``bf16`` – the value rounded to bfloat16 by torch (round-to-nearest-even).
* ``e4m3`` – OCP FP8 E4M3FN codes (torch.float8_e4m3fn) plus one fp32 scale
  per row, ``scale = absmax(row) / 448`` (``1.0`` for an all-zero row).  The
  row is divided by its scale, clamped to the finite range and rounded by
  torch; ``decode(code) * scale`` approximates the drawn value.
"""
from __future__ import annotations

import torch

SEED_BASE = 0x0C5A  # fixed so results are reproducible across runs and machines

_TORCH_DTYPES = {
    "f32": torch.float32,
    "bf16": torch.bfloat16,
}

E4M3_MAX = 448.0


def quantize_rows_e4m3(x: torch.Tensor):
    """Per-row absmax scaling of an fp32 tensor to e4m3fn codes.

    Returns ``(codes, scale)`` with ``codes`` a float8_e4m3fn tensor shaped
    like ``x`` and ``scale`` fp32 shaped ``x.shape[:-1]``.
    """
    x = x.float()
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn), scale.contiguous()


class Gen:
    """Seeded tensor factory for one workload on one device."""

    def __init__(self, workload_id: int, device: str | torch.device = "cpu"):
        self.workload_id = int(workload_id)
        self.device = torch.device(device)

    # -- seeds -------------------------------------------------------------
    def _gen(self, tensor_id: int, slot: int) -> torch.Generator:
        g = torch.Generator(device=self.device)
        seed = ((SEED_BASE * 1_000_003 + self.workload_id) * 1_000_033
                + int(tensor_id)) * 1_000_037 + int(slot)
        g.manual_seed(seed & ((1 << 63) - 1))
        return g

    # -- draws -------------------------------------------------------------
    def _draw(self, kind: str, tensor_id: int, shape, per_slot: bool):
        shape = tuple(int(s) for s in shape)
        if not per_slot or len(shape) == 0:
            return self._draw_one(kind, tensor_id, 0, shape)
        out = torch.empty(shape, dtype=torch.float32, device=self.device)
        for b in range(shape[0]):
            out[b] = self._draw_one(kind, tensor_id, b, shape[1:])
        return out

    def _draw_one(self, kind, tensor_id, slot, shape):
        g = self._gen(tensor_id, slot)
        if kind == "normal":
            return torch.randn(shape, generator=g, device=self.device, dtype=torch.float32)
        if kind == "uniform":
            return torch.rand(shape, generator=g, device=self.device, dtype=torch.float32)
        raise ValueError(kind)

    def normal(self, tensor_id: int, shape, dtype: str = "f32", per_slot: bool = True):
        """N(0,1) values stored as ``dtype`` ('f32' or 'bf16')."""
        x = self._draw("normal", tensor_id, shape, per_slot)
        return x.to(_TORCH_DTYPES[dtype]).contiguous()

    def uniform(self, tensor_id: int, shape, per_slot: bool = True):
        """U(0,1) values in fp32."""
        return self._draw("uniform", tensor_id, shape, per_slot).contiguous()

    def normal_e4m3(self, tensor_id: int, shape):
        """N(0,1) rows quantised to e4m3fn with a per-row fp32 scale.

        Quantised one leading slot at a time to bound temporaries.
        """
        shape = tuple(int(s) for s in shape)
        codes = torch.empty(shape, dtype=torch.float8_e4m3fn, device=self.device)
        scale = torch.empty(shape[:-1], dtype=torch.float32, device=self.device)
        for b in range(shape[0]):
            x = self._draw_one("normal", tensor_id, b, shape[1:])
            c, s = quantize_rows_e4m3(x)
            codes[b] = c
            scale[b] = s
            del x, c, s
        return codes, scale

    def const(self, value: float, shape, dtype: str = "f32"):
        return torch.full(tuple(shape), float(value), dtype=_TORCH_DTYPES[dtype],
                          device=self.device)
