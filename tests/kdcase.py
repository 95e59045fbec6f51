"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP path through the C ABI, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

# Parity bars (loss and per-row values: relative 1e-3; gradients: relative L2 1e-2).
LOSS_RTOL = 1e-3
GRAD_RTOL = 1e-2


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: dict, device="cuda"):
    import torch
    H = torch.from_numpy(np.ascontiguousarray(inp["H"]).view(np.int16)).view(torch.bfloat16).to(device)
    W = torch.from_numpy(np.ascontiguousarray(inp["W"]).view(np.int16)).view(torch.bfloat16).to(device)
    idx = torch.from_numpy(np.ascontiguousarray(inp["idx"], dtype=np.int32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(inp["t"], dtype=np.float32)).to(device)
    return H, W, idx, t


def bf16_tensor_to_f64(x) -> np.ndarray:
    import torch
    bits = x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def run_gpu(inp: dict, T: float, chunk: int, grad_loss: float | None = None, want_grads=True):
    """Forward (+ backward) on the GPU; returns numpy fp64 results."""
    import torch
    import lm_head_top_amd as kd
    H, W, idx, t = to_device(inp)
    loss, lse, row_kl = kd.forward(H, W, idx, t, T, chunk, want_row_kl=True)
    out = {"loss": float(loss.item()), "lse": lse.double().cpu().numpy(),
           "row_kl": row_kl.double().cpu().numpy(), "loss_t": loss, "lse_t": lse}
    if want_grads:
        g = None if grad_loss is None else torch.tensor([grad_loss], dtype=torch.float32,
                                                          device=H.device)
        dH, dW = kd.backward(H, W, idx, t, lse, g, T, chunk)
        torch.cuda.synchronize()
        out["dH"] = bf16_tensor_to_f64(dH)
        out["dW"] = dW.double().cpu().numpy()
    return out


def rel(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_parity(gpu: dict, ref: dict, grads=True, what=""):
    lr = abs(gpu["loss"] - ref["loss"]) / abs(ref["loss"])
    say(f"  {what} loss gpu={gpu['loss']:.7g} oracle={ref['loss']:.7g} rel={lr:.2e}")
    assert lr <= LOSS_RTOL, (what, gpu["loss"], ref["loss"])
    lse_err = np.max(np.abs(gpu["lse"] - ref["lse"]) / np.maximum(np.abs(ref["lse"]), 1.0))
    kl_err = np.max(np.abs(gpu["row_kl"] - ref["row_kl"]) / np.maximum(np.abs(ref["row_kl"]), 1.0))
    say(f"  {what} max rel err lse={lse_err:.2e} row_kl={kl_err:.2e}")
    assert lse_err <= LOSS_RTOL and kl_err <= LOSS_RTOL
    if grads:
        eh, ew = rel(gpu["dH"], ref["dH"]), rel(gpu["dW"], ref["dW"])
        say(f"  {what} rel L2 dH={eh:.2e} dW={ew:.2e}")
        assert eh <= GRAD_RTOL and ew <= GRAD_RTOL
