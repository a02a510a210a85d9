"""Move synthetic inputs to the GPU for the library (test and benchmark helper).

Only copies the generator's bytes into device tensors with the dtype the C ABI
expects; it computes nothing.
"""
import numpy as np
import torch

import routed_grouped_gemm_amd as moe


def tensor(a, device="cuda"):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.uint8:  # e4m3 codes
        t = torch.from_numpy(a).view(torch.float8_e4m3fn)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


WEIGHT_KEYS = ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down",
               "sh_s_gate", "sh_s_up", "sh_s_down")


def to_device(inp, device="cuda", layout="packed", act_quant=False):
    """Returns (problem, hidden, w_router, bias, weights dict) on the device.  layout
    "packed" converts the expert matrices with the library's moe_pack_weights (the
    problem then says so); "rowmajor" passes them as generated.  act_quant: the problem's
    fp8-activation mode."""
    c = inp.cfg
    p = moe.problem(c["T"], c["d"], c["n"], c["E"], c["k"], c["shared"], c["act"], c["w"], layout=layout,
                    act_quant=act_quant)
    weights = {k: tensor(getattr(inp, k), device) for k in WEIGHT_KEYS if getattr(inp, k) is not None}
    if layout == "packed":
        weights = moe.pack_weights(p, weights)  # the row-major copies are released here
    return p, tensor(inp.hidden, device), tensor(inp.w_router, device), tensor(inp.bias, device), weights


def out_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)
