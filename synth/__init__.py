"""Seeded synthetic inputs for the MoE-layer forward.

This module only *draws and stores* inputs.  It holds none of the layer's
arithmetic (no routing, no dequantisation, no matmul): the CPU oracle and the
HIP path each interpret the stored bits on their own.  Both sides consume the
exact same bytes produced here.

Storage formats (what the arrays hold):
  * "f32"  -> numpy float32
  * "bf16" -> numpy uint16, the upper half of an IEEE float32 (round to nearest even)
  * "fp8"  -> numpy uint8, OCP FP8 E4M3 ("e4m3fn") codes, with one float32 scale
             per 128x128 block of each [out, in] weight matrix

Tensor layouts (row-major):
  hidden   [T, d]        activations
  w_router [E, d]        one row of router weights per expert
  w_gate   [E, n, d]     one row per intermediate channel (input dim d contiguous)
  w_up     [E, n, d]
  w_down   [E, d, n]     one row per output channel (input dim n contiguous)
  s_gate, s_up [E, n/128, d/128] float32   (fp8 only)
  s_down       [E, d/128, n/128] float32   (fp8 only)
  sh_*     the always-on shared expert, same layouts without the leading E
  bias     [E] float32 router bias (skewed-load workload only)

Random streams: numpy PCG64, one SeedSequence([seed, tag, idx]) per tensor, tags
0 hidden, 1 router, 2 gate, 3 up, 4 down, 5 Zipf rank permutation; idx is the
expert index (the shared expert uses idx = E).  Values are drawn in float32 and
then rounded to the storage dtype.

The workloads follow the shapes the pages name: 256 experts choosing 8 with a
512-wide expert intermediate (the vLLM fused-MoE config page, section 02 and the
E/N table of section 05), M from 1 to 4096 tokens per step (same page, section
03), fp8 weights with 128x128 block scales (same page, the fp8_w8a8 config
file of section 03), Zipf-like expert popularity (Weave review, section 1.1),
and an always-on shared expert (GC-MoE article, "two MMA implementations").
"""
from __future__ import annotations

import json
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TAG_HIDDEN, TAG_ROUTER, TAG_GATE, TAG_UP, TAG_DOWN, TAG_ZIPF = 0, 1, 2, 3, 4, 5
FP8_BLOCK = 128
FP8_MAX = 448.0

_HERE = os.path.dirname(os.path.abspath(__file__))
_REPO = os.path.dirname(_HERE)
ZIPF_BIAS_FILE = os.path.join(_REPO, "tests", "golden", "skewed_router_bias.json")

# name -> workload.  "T_gen" is how many token rows are drawn; a workload with a
# smaller T takes the first T rows, so workloads sharing a seed share tokens.
CONFIGS = {
    "tiny_fp32": dict(seed=1, T=64, T_gen=64, d=256, E=8, k=2, n=512,
                      act="f32", w="f32", shared=0, zipf=False),
    "decode_bf16": dict(seed=2, T=16, T_gen=32768, d=2048, E=256, k=8, n=512,
                        act="bf16", w="bf16", shared=0, zipf=False),
    "prefill_bf16": dict(seed=2, T=4096, T_gen=32768, d=2048, E=256, k=8, n=512,
                         act="bf16", w="bf16", shared=0, zipf=False),
    "skewed_bf16": dict(seed=4, T=2048, T_gen=2048, d=4096, E=64, k=4, n=1536,
                        act="bf16", w="bf16", shared=0, zipf=True, zipf_s=1.1),
    "large_fp8": dict(seed=5, T=4096, T_gen=16384, d=7168, E=256, k=8, n=2048,
                      act="bf16", w="fp8", shared=1, zipf=False),
}
# T_gen above a workload's own T serves the compute-bound points of the same shapes (the
# prefill shape at T = 16384 and 32768, the fp8 shape at T = 16384): a stream's first values
# do not depend on how many are drawn, so every smaller T gets the same rows as before.
LARGE_FP8_T = (1, 8, 64, 512, 4096)


def config(name: str, T: int | None = None) -> dict:
    """Return a copy of a named workload, optionally with another token count."""
    c = dict(CONFIGS[name])
    c["name"] = name
    if T is not None:
        if T > c["T_gen"]:
            raise ValueError(f"{name}: T={T} exceeds the {c['T_gen']} drawn rows")
        c["T"] = int(T)
    return c


def _rng(seed: int, tag: int, idx: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, idx])))


def normal_f32(seed: int, tag: int, idx: int, shape, std: float) -> np.ndarray:
    a = _rng(seed, tag, idx).standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a.reshape(shape)


# ----------------------------------------------------------------------------
# storage encoders (input generation only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def fp8_block_quantize(w: np.ndarray):
    """[R, C] float32 -> (uint8 e4m3 codes [R, C], float32 scales [R/128, C/128]).

    Scale = block amax / 448, codes = round-to-nearest-even of w / scale with
    saturation to +-448 (the encoder is torch's float8_e4m3fn cast).
    """
    import torch  # encoder only

    R, C = w.shape
    if R % FP8_BLOCK or C % FP8_BLOCK:
        raise ValueError("fp8 weights need both dims divisible by 128")
    blocks = w.reshape(R // FP8_BLOCK, FP8_BLOCK, C // FP8_BLOCK, FP8_BLOCK)
    amax = np.abs(blocks).max(axis=(1, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    q = blocks / scale[:, None, :, None]
    np.clip(q, -FP8_MAX, FP8_MAX, out=q)
    codes = torch.from_numpy(np.ascontiguousarray(q.reshape(R, C), dtype=np.float32))
    codes = codes.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def encode(a: np.ndarray, dtype: str):
    """float32 array -> (storage array, scales or None) for a storage dtype."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32), None
    if dtype == "bf16":
        return f32_to_bf16_bits(a), None
    if dtype == "fp8":
        return fp8_block_quantize(a)
    raise ValueError(dtype)


def storage_np_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]


# ----------------------------------------------------------------------------
# inputs
# ----------------------------------------------------------------------------
@dataclass
class MoEInputs:
    cfg: dict
    hidden: np.ndarray
    w_router: np.ndarray
    bias: np.ndarray | None
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    s_gate: np.ndarray | None = None
    s_up: np.ndarray | None = None
    s_down: np.ndarray | None = None
    sh_gate: np.ndarray | None = None
    sh_up: np.ndarray | None = None
    sh_down: np.ndarray | None = None
    sh_s_gate: np.ndarray | None = None
    sh_s_up: np.ndarray | None = None
    sh_s_down: np.ndarray | None = None
    experts_filled: tuple = field(default_factory=tuple)


def make_hidden(cfg: dict) -> np.ndarray:
    x = normal_f32(cfg["seed"], TAG_HIDDEN, 0, (cfg["T_gen"], cfg["d"]), 1.0)[: cfg["T"]]
    return encode(x, cfg["act"])[0]


def make_router(cfg: dict) -> np.ndarray:
    w = normal_f32(cfg["seed"], TAG_ROUTER, 0, (cfg["E"], cfg["d"]), 1.0 / np.sqrt(cfg["d"]))
    return encode(w, cfg["act"])[0]


def load_zipf_bias(cfg: dict) -> np.ndarray:
    """The frozen per-expert router bias of a Zipf-skewed workload."""
    with open(ZIPF_BIAS_FILE) as f:
        rec = json.load(f)
    if rec["config"] != cfg["name"]:
        raise ValueError("bias file is for another workload")
    b = np.array([float.fromhex(h) for h in rec["bias_f32_hex"]], dtype=np.float32)
    assert b.shape == (cfg["E"],)
    return b


def zipf_rank_permutation(cfg: dict) -> np.ndarray:
    """Seeded map rank r -> expert id, so hot experts are not simply the low ids."""
    return _rng(cfg["seed"], TAG_ZIPF, 0).permutation(cfg["E"])


def _expert_matrices(cfg: dict, idx: int):
    d, n = cfg["d"], cfg["n"]
    s = cfg["seed"]
    g = normal_f32(s, TAG_GATE, idx, (n, d), 1.0 / np.sqrt(d))
    u = normal_f32(s, TAG_UP, idx, (n, d), 1.0 / np.sqrt(d))
    dn = normal_f32(s, TAG_DOWN, idx, (d, n), 1.0 / np.sqrt(n))
    return [encode(g, cfg["w"]), encode(u, cfg["w"]), encode(dn, cfg["w"])]


def make_inputs(cfg: dict, experts=None, with_bias: bool = True, threads: int | None = None) -> MoEInputs:
    """Draw every input of a workload.

    experts: None for all routed experts, or an iterable of expert ids to draw;
    the rows of other experts are left zero (a caller passes only experts that
    the routing can reach).  The shared expert, if any, is always drawn.
    """
    E, d, n = cfg["E"], cfg["d"], cfg["n"]
    wdt = storage_np_dtype(cfg["w"])
    ids = list(range(E)) if experts is None else sorted(set(int(e) for e in experts))
    w_gate = np.zeros((E, n, d), dtype=wdt)
    w_up = np.zeros((E, n, d), dtype=wdt)
    w_down = np.zeros((E, d, n), dtype=wdt)
    fp8 = cfg["w"] == "fp8"
    if fp8:
        s_gate = np.zeros((E, n // FP8_BLOCK, d // FP8_BLOCK), np.float32)
        s_up = np.zeros_like(s_gate)
        s_down = np.zeros((E, d // FP8_BLOCK, n // FP8_BLOCK), np.float32)
    else:
        s_gate = s_up = s_down = None

    def fill(e):
        (g, sg), (u, su), (dn, sd) = _expert_matrices(cfg, e)
        w_gate[e], w_up[e], w_down[e] = g, u, dn
        if fp8:
            s_gate[e], s_up[e], s_down[e] = sg, su, sd

    nthr = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(max(1, nthr)) as ex:
        list(ex.map(fill, ids))

    inp = MoEInputs(cfg=cfg, hidden=make_hidden(cfg), w_router=make_router(cfg),
                    bias=(load_zipf_bias(cfg) if (cfg.get("zipf") and with_bias) else None),
                    w_gate=w_gate, w_up=w_up, w_down=w_down,
                    s_gate=s_gate, s_up=s_up, s_down=s_down, experts_filled=tuple(ids))
    if cfg["shared"]:
        (g, sg), (u, su), (dn, sd) = _expert_matrices(cfg, E)
        inp.sh_gate, inp.sh_up, inp.sh_down = g, u, dn
        inp.sh_s_gate, inp.sh_s_up, inp.sh_s_down = sg, su, sd
    return inp


def make_tiny(seed: int, T: int, d: int, n: int, E: int, k: int, act="f32", w="f32",
              shared: int = 0, bias: bool = False, x_scale: float = 1.0) -> MoEInputs:
    """A small ad-hoc workload with the same generators (for tests)."""
    cfg = dict(seed=seed, T=T, T_gen=T, d=d, E=E, k=k, n=n, act=act, w=w, shared=shared,
               zipf=False, name=f"adhoc_{seed}")
    inp = make_inputs(cfg, threads=1)
    if x_scale != 1.0:
        x = normal_f32(seed, TAG_HIDDEN, 0, (T, d), 1.0) * np.float32(x_scale)
        inp.hidden = encode(x, act)[0]
    if bias:
        inp.bias = normal_f32(seed, 9, 0, (E,), 1.0)
    return inp
