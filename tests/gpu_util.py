"""Helpers shared by the GPU parity tests: move BF16 bit patterns to and from the device,
run the library through its binding, compare with the FP64 oracle."""
import numpy as np
import torch

from oracle import bf16_bits_to_f64, compare


def dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 BF16 bit patterns -> contiguous bfloat16 tensor on cuda:0 (same bits)."""
    a = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(a).to("cuda:0").view(torch.bfloat16)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to("cuda:0")


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of(t: torch.Tensor) -> np.ndarray:
    return bf16_bits_to_f64(bits_of(t))


def check(o_gpu, o_ref, lse_gpu=None, lse_ref=None, label=""):
    m = compare(o_gpu, o_ref, lse_gpu, lse_ref)
    print(f"[parity] {label}: rel_l2={m['rel_l2']:.3e} max_abs={m['max_abs']:.3e} "
          f"lse_max_abs={m.get('lse_max_abs', float('nan')):.3e} n={m['n_elems']}", flush=True)
    assert m["ok"], (label, m)
    return m


def device_normal_bf16(shape, seed: int) -> torch.Tensor:
    """Seeded N(0, 1) values rounded to BF16, generated on cuda:0 for inputs too large to build
    on the host. Tests copy back the rows the oracle needs, so both sides read the same bits."""
    g = torch.Generator(device="cuda:0").manual_seed(seed)
    x = torch.randn(shape, generator=g, device="cuda:0", dtype=torch.float32)
    return x.to(torch.bfloat16)
