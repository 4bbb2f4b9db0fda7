"""Seeded synthetic inputs for the attention workloads.

This module holds the workload shapes, seeds and the value recipe, and nothing
of the attention arithmetic itself.  Both sides draw their inputs from here:
the float64 CPU oracle (as upcasts of exactly the values the GPU receives) and
the HIP library.

Recipe: a CPU ``torch.Generator`` seeded per workload draws ``torch.randn``
float32 tensors of shape [B, H, N, d] in the order q, k, v, then dO (only when
a backward is wanted); the GPT-2-medium-shaped workload multiplies every 7th
query row (0-based rows i with i % 7 == 6) by 4 so later key tiles keep raising
the running max; finally the tensors are cast to the workload's dtype (bf16
rounds to nearest even; x4 is exact in bf16, so the order does not matter).
The default softmax scale is 1/sqrt(d).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                      # "bf16" or "f32"
    causal: Tuple[bool, ...]
    seed: int
    boost_every: int = 0            # every k-th query row scaled ...
    boost: float = 1.0              # ... by this factor
    backward: bool = False
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


WORKLOADS = {
    w.name: w
    for w in (
        Workload("single_head_fp32_n256", 1, 1, 256, 64, "f32", (False,), 0,
                 note="single head, non-causal, fp32 end to end"),
        Workload("gpt2_medium_n1024", 8, 16, 1024, 64, "bf16", (False, True), 1,
                 boost_every=7, boost=4.0,
                 note="GPT-2-medium shape; every 7th query row x4"),
        Workload("llama8b_n4096", 1, 32, 4096, 128, "bf16", (True,), 2,
                 note="Llama-3.1-8B shape, causal"),
        Workload("long_context_n16384", 1, 8, 16384, 128, "bf16", (True,), 3,
                 note="long context, causal"),
        Workload("long_context_n32768", 1, 8, 32768, 128, "bf16", (True,), 4,
                 note="long context, causal"),
        Workload("train_step_n2048", 4, 16, 2048, 64, "bf16", (True,), 5,
                 backward=True,
                 note="forward plus backward, causal"),
    )
}


def make_inputs(B: int, H: int, N: int, d: int, dtype=torch.bfloat16,
                seed: int = 0, with_do: bool = False, boost_every: int = 0,
                boost: float = 1.0):
    """Return CPU tensors (q, k, v[, do]) of shape [B, H, N, d] in ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32) if with_do else None
    if boost_every:
        q[:, :, boost_every - 1::boost_every] *= boost
    out = [q.to(dtype), k.to(dtype), v.to(dtype)]
    if with_do:
        out.append(do.to(dtype))
    return tuple(out)



def make_device_inputs(B: int, H: int, N: int, d: int, dtype=torch.bfloat16,
                       seed: int = 0, with_do: bool = False, device: str = "cuda"):
    """``make_inputs`` drawn on the device, for sizes whose host-side draw
    would dominate a test (the longest sequences).

    Same recipe (torch.randn float32 in the order q, k, v, dO, then the cast),
    from torch's generator of that device seeded with ``seed``; its stream of
    numbers differs from the CPU generator's, so these are other inputs of the
    same distribution, not the same inputs.
    """
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    out = [torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(dtype)
           for _ in range(4 if with_do else 3)]
    return tuple(out)

def workload_inputs(w: Workload, with_do: bool = None):
    """Inputs for a named workload (dO included for backward workloads)."""
    if with_do is None:
        with_do = w.backward
    return make_inputs(w.B, w.H, w.N, w.d, w.torch_dtype, w.seed, with_do,
                       w.boost_every, w.boost)


def make_gqa_inputs(B: int, H: int, Hkv: int, N: int, d: int, dtype=torch.bfloat16,
                    seed: int = 0, with_do: bool = False):
    """Grouped-query inputs: q (and dO) [B, H, N, d], k and v [B, Hkv, N, d].

    Same recipe as ``make_inputs`` (torch.randn float32 in the order q, k, v,
    dO, then the cast), with the key/value tensors drawn at their own head count.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, N, d), generator=g, dtype=torch.float32)
    out = [q.to(dtype), k.to(dtype), v.to(dtype)]
    if with_do:
        out.append(torch.randn((B, H, N, d), generator=g, dtype=torch.float32).to(dtype))
    return tuple(out)


def make_fp8_inputs(B: int, H: int, N: int, d: int, seed: int = 0):
    """e4m3 inputs: (q8, k8, v8) as uint8 byte codes [B, H, N, d] and their
    dequantisation factors (q_scale, k_scale, v_scale).

    torch.randn float32 tensors (q, k, v in that order) are scaled by
    448 / max|x| (the largest e4m3 value) and cast to torch.float8_e4m3fn
    (round to nearest even); the factor that maps the codes back is
    max|x| / 448.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    out, scales = [], []
    for _ in range(3):
        x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
        amax = float(x.abs().max()) if x.numel() else 1.0
        s = (amax / 448.0) if amax > 0 else 1.0
        out.append((x / s).to(torch.float8_e4m3fn).view(torch.uint8))
        scales.append(s)
    return out[0], out[1], out[2], scales[0], scales[1], scales[2]
