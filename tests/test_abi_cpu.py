"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and its host-only entry points validate arguments.  No compute
call is made (validation returns before anything is enqueued)."""
import ctypes
import os
import re

import pytest

import routed_grouped_gemm_amd as moe

INVALID, UNSUPPORTED, TOO_SMALL = 1, 2, 3


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from routed_grouped_gemm_amd import build
        build.build()
    return moe.lib()


def test_exports_every_header_function(L):
    names = moe.header_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(L, name), f"libmoe.so does not export {name}"


def test_version_and_strings(L):
    assert moe.abi_version() == 4
    for code, name in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARGUMENT"), (2, "MOE_ERR_UNSUPPORTED"),
                       (3, "MOE_ERR_WORKSPACE_TOO_SMALL"), (4, "MOE_ERR_HIP"), (5, "MOE_ERR_DEVICE_FAULT")]:
        assert moe.status_string(code) == name
    assert moe.status_string(77) == "MOE_ERR_UNKNOWN"


def ws_size(p):
    out = ctypes.c_size_t(0)
    return moe.lib().moe_workspace_size(ctypes.byref(p), ctypes.byref(out)), out.value


@pytest.mark.parametrize("kw,code", [
    (dict(T=16, d=2048, n=512, E=256, k=8), 0),
    (dict(T=0, d=2048, n=512, E=256, k=8), 0),
    (dict(T=64, d=256, n=512, E=8, k=2, act="f32", w="f32"), 0),
    (dict(T=4, d=7168, n=2048, E=256, k=8, n_shared=1, w="fp8"), 0),
    (dict(T=16, d=2048, n=512, E=256, k=0), INVALID),
    (dict(T=16, d=2048, n=512, E=4, k=5), INVALID),
    (dict(T=-1, d=2048, n=512, E=8, k=2), INVALID),
    (dict(T=16, d=2048, n=512, E=8, k=2, n_shared=2), INVALID),
    (dict(T=16, d=2000, n=512, E=8, k=2), UNSUPPORTED),
    (dict(T=16, d=2048, n=500, E=8, k=2), UNSUPPORTED),
    (dict(T=16, d=2048, n=512, E=2048, k=2), UNSUPPORTED),
    (dict(T=16, d=2048, n=512, E=8, k=2, act="f32", w="bf16"), UNSUPPORTED),
    (dict(T=16, d=2048, n=512, E=8, k=2, act="f32", w="fp8"), UNSUPPORTED),
    # fp8: the 16-row units keep at most 128 scale blocks of their K range per wave
    (dict(T=16, d=32768, n=16384, E=8, k=2, w="fp8"), 0),
    (dict(T=16, d=33024, n=512, E=8, k=2, w="fp8"), UNSUPPORTED),
    (dict(T=16, d=2048, n=16640, E=8, k=2, w="fp8"), UNSUPPORTED),
    (dict(T=16, d=33024, n=16640, E=8, k=2, w="bf16"), 0),
    # activation tensors (hidden, and the T*k + shared rows of the intermediate) stay below 4 GB
    (dict(T=(1 << 19) - 1, d=4096, n=512, E=256, k=1), 0),
    (dict(T=1 << 19, d=4096, n=512, E=256, k=1), UNSUPPORTED),
    (dict(T=131071, d=2048, n=2048, E=256, k=8), 0),
    (dict(T=131072, d=2048, n=2048, E=256, k=8), UNSUPPORTED),
])
def test_workspace_size_validation(L, kw, code):
    p = moe.problem(**kw)
    rc, size = ws_size(p)
    assert rc == code
    if code == 0:
        assert size >= 4096 and size % 256 == 0


def _table_rows(w, aq, mean_rows):
    """The m-tile rows the compiled-in tile table (csrc/moe_tuned.h) gives: the first rule of the
    dtype's list whose bound is at least the mean rows per routed expert."""
    src = open(os.path.join(os.path.dirname(moe.__file__), "csrc", "moe_tuned.h")).read()
    lists = re.findall(r"// (\w+)\n    \{(.*)\},", src)
    body = dict(lists)["fp8a" if aq else w]
    for bound, rows, _ in re.findall(r"\{([0-9.e+]+)f, (\d+), (\d+)\}", body):
        if mean_rows <= float(bound):
            return int(rows)
    raise AssertionError("no rule covers the mean")


@pytest.mark.parametrize("kw", [
    dict(T=16, d=2048, n=512, E=256, k=8),            # decode: mean 0.5 rows per expert
    dict(T=512, d=7168, n=2048, E=256, k=8, n_shared=1, w="fp8"),
    dict(T=300, d=1024, n=512, E=64, k=6, n_shared=1, w="fp8"),
    dict(T=300, d=256, n=512, E=16, k=4, act="f32", w="f32"),
    dict(T=4096, d=2048, n=512, E=256, k=8),          # prefill: mean 128
    dict(T=4096, d=7168, n=2048, E=256, k=8, n_shared=1, w="fp8"),
])
def test_plan_describe_reports_the_m_tile(L, kw):
    info = moe.plan_describe(moe.problem(**kw))
    rows = _table_rows(kw.get("w", "bf16"), False, kw["T"] * kw["k"] / kw["E"])
    assert info["m_tile_rows"] == rows
    if rows == 16:
        assert (info["gateup_cols"], info["down_cols"]) == (16, 128)
    else:
        assert (info["gateup_cols"], info["down_cols"]) == (128, 256)
    assert info["router_k_split"] in (1, 2, 4, 8)
    T, k, E = kw["T"], kw["k"], kw["E"]
    assert info["max_m_tiles"] >= min(T * k, E)


@pytest.mark.parametrize("kw,split", [
    (dict(T=16, d=2048, n=512, E=256, k=8), 2),                       # decode: few 16-row tiles, K > 1024
    (dict(T=16, d=1024, n=512, E=256, k=8), 1),                       # short K: not split
    (dict(T=1, d=7168, n=2048, E=256, k=8, n_shared=1, w="fp8"), 4),  # K > 4096: four parts
    (dict(T=2048, d=1024, n=512, E=256, k=1), 1),                     # many tiles: not split
    (dict(T=4096, d=2048, n=512, E=256, k=8), 4),                     # tile core: up to 256 items
])
def test_router_k_split_rule(L, kw, split):
    # the router's K is split over several items when its tiles are too few to spread the
    # router weights' loads over the GPU (the partial logits are added in part order)
    assert moe.plan_describe(moe.problem(**kw))["router_k_split"] == split


def test_fp8_activation_mode_rules(L):
    """act_quant: 0 or 1 (else INVALID), 1 only with fp8 weights (else UNSUPPORTED); the plan
    reports fp8 activations exactly when the m-tiles are above 16 rows."""
    for bad in (2, -1):
        p = moe.problem(512, 7168, 2048, 256, 8, 1, w="fp8")
        p.act_quant = bad
        assert ws_size(p)[0] == INVALID
    assert ws_size(moe.problem(512, 2048, 512, 256, 8, act_quant=True))[0] == UNSUPPORTED
    assert ws_size(moe.problem(64, 256, 256, 8, 2, act="f32", w="f32", act_quant=True))[0] == UNSUPPORTED
    for T in (1, 8, 64, 512, 4096):
        plan = moe.plan_describe(moe.problem(T, 7168, 2048, 256, 8, 1, w="fp8", act_quant=True))
        assert plan["fp8_activations"] == int(plan["m_tile_rows"] > 16), T
        assert moe.plan_describe(moe.problem(T, 7168, 2048, 256, 8, 1, w="fp8"))["fp8_activations"] == 0
    assert moe.plan_describe(moe.problem(1, 7168, 2048, 256, 8, 1, w="fp8", act_quant=True))["fp8_activations"] == 0
    assert moe.plan_describe(moe.problem(4096, 7168, 2048, 256, 8, 1, w="fp8", act_quant=True))["fp8_activations"] == 1
    # the fp8-activation workspace holds the E4M3 hidden rows and block scales; H shrinks to one
    # byte per value
    rc0, plain = ws_size(moe.problem(4096, 7168, 2048, 256, 8, 1, w="fp8"))
    rc1, quant = ws_size(moe.problem(4096, 7168, 2048, 256, 8, 1, w="fp8", act_quant=True))
    assert rc0 == rc1 == 0
    rows_h = 4096 * 9
    assert quant == pytest.approx(plain - rows_h * 2048 + 4096 * 7168 + 4096 * 56 + rows_h * 16, abs=4096)


def test_tile_overrides_are_validated(L):
    """m_tile_rows / group_m overrides: invalid values are refused before any launch."""
    VP = ctypes.c_void_p
    p = moe.problem(16, 2048, 512, 256, 8, layout="packed")
    W = moe.Weights(*([1 << 21] * 3 + [None] * 9))
    for rows, gm, want in ((48, 0, INVALID), (0, -1, INVALID), (0, 65, INVALID)):
        o = moe.LaunchOptions(0, 0, None, 0, rows, gm)
        assert L.moe_forward_ex(ctypes.byref(p), VP(1 << 20), VP(1 << 20), None, ctypes.byref(W), VP(3 << 20), None,
                                VP(1 << 24), 1 << 30, None, ctypes.byref(o)) == want


def test_tile_table_is_well_formed(L):
    """The compiled-in tile table: mean-row bounds increase, tiles are valid for the dtype, and the
    chosen tile grows with the mean rows per expert."""
    for w, aq in (("f32", False), ("bf16", False), ("fp8", False), ("fp8", True)):
        act = "f32" if w == "f32" else "bf16"
        prev = 0
        for T in (1, 16, 64, 256, 1024, 4096, 16384, 65536):
            info = moe.plan_describe(moe.problem(T, 2048, 512, 256, 8, act=act, w=w, act_quant=aq))
            assert info["m_tile_rows"] in (16, 32, 64, 128, 160)
            assert 1 <= info["group_m"] <= 64
            assert info["m_tile_rows"] >= prev
            assert info["fp8_activations"] == int(aq and info["m_tile_rows"] > 16)
            prev = info["m_tile_rows"]


def test_plan_describe_validates(L):
    bad = moe.problem(16, 2000, 512, 256, 8)
    with pytest.raises(moe.MoEError) as ei:
        moe.plan_describe(bad)
    assert ei.value.code == UNSUPPORTED
    assert L.moe_plan_describe(ctypes.byref(moe.problem(16, 2048, 512, 256, 8)), None) == INVALID


def test_workspace_size_monotone_in_T(L):
    sizes = [ws_size(moe.problem(T, 2048, 512, 256, 8))[1] for T in (1, 16, 256, 4096)]
    assert sizes == sorted(sizes)
    # H and Y alone for T=4096: rows T*k, n and d bf16 columns
    assert sizes[-1] > 4096 * 8 * (512 + 2048) * 2


def test_weight_layout_rules(L):
    assert ws_size(moe.problem(16, 2048, 512, 256, 8, layout="packed"))[0] == 0
    p = moe.problem(16, 2048, 512, 256, 8)
    p.w_layout = 2
    assert ws_size(p)[0] == INVALID
    # the forward reads packed weights only; row-major ones are refused before any launch
    VP = ctypes.c_void_p
    fake = VP(1 << 20)
    W = moe.Weights(*([1 << 21] * 3 + [None] * 9))
    rm = moe.problem(16, 2048, 512, 256, 8, layout="rowmajor")
    assert L.moe_forward(ctypes.byref(rm), fake, fake, None, ctypes.byref(W), VP(3 << 20), None, fake, 1 << 30,
                         None) == UNSUPPORTED


def test_noalloc_refuses_oversized_and_invalid_problems_before_any_hip_call(L):
    """moe_forward_noalloc's fixed scratch has a stated size; larger problems are refused on the
    host, like invalid ones, before the device is touched."""
    import re
    hdr = open(moe.HEADER_PATH).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == moe.NOALLOC_SCRATCH_BYTES
    VP = ctypes.c_void_p
    W = moe.Weights(*([1 << 21] * 3 + [None] * 9))
    big = moe.problem(4096, 2048, 512, 256, 8, layout="packed")
    assert ws_size(big)[1] > moe.NOALLOC_SCRATCH_BYTES
    assert L.moe_forward_noalloc(ctypes.byref(big), VP(1 << 20), VP(1 << 20), None, ctypes.byref(W), VP(3 << 20),
                                 None, None) == TOO_SMALL
    bad = moe.problem(16, 2000, 512, 256, 8, layout="packed")
    assert L.moe_forward_noalloc(ctypes.byref(bad), VP(1 << 20), VP(1 << 20), None, ctypes.byref(W), VP(3 << 20),
                                 None, None) == UNSUPPORTED
    empty = moe.problem(0, 2048, 512, 256, 8, layout="packed")
    assert L.moe_forward_noalloc(ctypes.byref(empty), None, None, None, None, None, None, None) == 0


def test_pack_weights_rejects_bad_arguments_before_launch(L):
    """moe_pack_weights validates everything on the host (no HIP call on these paths)."""
    VP = ctypes.c_void_p
    p = moe.problem(16, 2048, 512, 256, 8)
    nbytes = 256 * 512 * 2048 * 2
    src = moe.Weights(*([1 << 40, (1 << 40) + nbytes, (1 << 40) + 2 * nbytes] + [None] * 9))
    dst = moe.Weights(*([1 << 41, (1 << 41) + nbytes, (1 << 41) + 2 * nbytes] + [None] * 9))
    assert L.moe_pack_weights(None, ctypes.byref(src), ctypes.byref(dst), None) == INVALID
    assert L.moe_pack_weights(ctypes.byref(p), None, ctypes.byref(dst), None) == INVALID
    assert L.moe_pack_weights(ctypes.byref(p), ctypes.byref(src), None, None) == INVALID
    # a missing matrix, a misaligned one, and a destination that overlaps its source
    miss = moe.Weights(*([1 << 41, None, (1 << 41) + 2 * nbytes] + [None] * 9))
    assert L.moe_pack_weights(ctypes.byref(p), ctypes.byref(src), ctypes.byref(miss), None) == INVALID
    odd = moe.Weights(*([(1 << 41) + 8, (1 << 41) + nbytes, (1 << 41) + 2 * nbytes] + [None] * 9))
    assert L.moe_pack_weights(ctypes.byref(p), ctypes.byref(src), ctypes.byref(odd), None) == INVALID
    lap = moe.Weights(*([(1 << 40) + 4096, (1 << 41) + nbytes, (1 << 41) + 2 * nbytes] + [None] * 9))
    assert L.moe_pack_weights(ctypes.byref(p), ctypes.byref(src), ctypes.byref(lap), None) == INVALID
    # the shared expert's matrices are required when the problem has one
    ps = moe.problem(16, 2048, 512, 256, 8, n_shared=1)
    assert L.moe_pack_weights(ctypes.byref(ps), ctypes.byref(src), ctypes.byref(dst), None) == INVALID
    # shapes are validated like the compute calls
    bad = moe.problem(16, 2000, 512, 256, 8)
    assert L.moe_pack_weights(ctypes.byref(bad), ctypes.byref(src), ctypes.byref(dst), None) == UNSUPPORTED


def test_scale_block_rules(L):
    p = moe.problem(4, 256, 256, 4, 2, w="fp8")
    p.scale_block = 64
    assert ws_size(p)[0] == UNSUPPORTED
    p = moe.problem(4, 256, 256, 4, 2)
    p.scale_block = 128
    assert ws_size(p)[0] == INVALID


def test_compute_calls_reject_bad_arguments_before_launch(L):
    """Host-side validation returns before any HIP call, so this runs without a GPU."""
    p = moe.problem(16, 2048, 512, 256, 8, layout="packed")
    W = moe.Weights()
    VP = ctypes.c_void_p
    fake = VP(1 << 20)  # never dereferenced: validation fails first
    # null hidden
    assert L.moe_forward(ctypes.byref(p), None, fake, None, ctypes.byref(W), fake, None, fake, 1 << 30, None) == INVALID
    # null weights
    assert L.moe_forward(ctypes.byref(p), fake, fake, None, ctypes.byref(W), VP(2 << 20), None, fake, 1 << 30, None) == INVALID
    # misaligned hidden
    assert L.moe_forward(ctypes.byref(p), VP((1 << 20) + 4), fake, None, ctypes.byref(W), fake, None, fake, 1 << 30, None) == INVALID
    # out aliases hidden
    W2 = moe.Weights(*([1 << 21] * 3 + [None] * 9))
    assert L.moe_forward(ctypes.byref(p), fake, fake, None, ctypes.byref(W2), fake, None, fake, 1 << 30, None) == INVALID
    # workspace too small (checked before any device query)
    rc = L.moe_forward(ctypes.byref(p), fake, fake, None, ctypes.byref(W2), VP(3 << 20), None, fake, 4096, None)
    assert rc == TOO_SMALL
    # workspace misaligned
    rc = L.moe_forward(ctypes.byref(p), fake, fake, None, ctypes.byref(W2), VP(3 << 20), None, VP((1 << 20) + 16), 1 << 30, None)
    assert rc == INVALID
    # fp8 without scales
    p8 = moe.problem(4, 256, 256, 4, 2, w="fp8", layout="packed")
    assert L.moe_forward(ctypes.byref(p8), fake, fake, None, ctypes.byref(W2), VP(3 << 20), None, fake, 1 << 30, None) == INVALID
    # shared expert requested but missing
    ps = moe.problem(4, 256, 256, 4, 2, n_shared=1, layout="packed")
    assert L.moe_forward(ctypes.byref(ps), fake, fake, None, ctypes.byref(W2), VP(3 << 20), None, fake, 1 << 30, None) == INVALID
    # route/permute argument checks
    assert L.moe_route(ctypes.byref(p), fake, fake, None, None, fake, None, fake, 1 << 30, None) == INVALID
    assert L.moe_permute(ctypes.byref(p), fake, None, fake, fake, fake, fake, 1 << 30, None) == INVALID
    bad = moe.problem(16, 2048, 512, 4, 8)
    assert L.moe_route(ctypes.byref(bad), fake, fake, None, fake, fake, None, fake, 1 << 30, None) == INVALID
    # workspace init argument checks
    assert L.moe_workspace_init(None, 1 << 20, None) == INVALID
    assert L.moe_workspace_init(fake, 100, None) == INVALID


def test_binding_refuses_undersized_tensors():
    """The binding checks tensor sizes and element widths against the problem before any
    pointer reaches the library (host tensors here: the check comes first)."""
    import torch
    T, d, n, E, k = 4, 256, 256, 8, 2
    p = moe.problem(T, d, n, E, k)
    x = torch.zeros(T * d, dtype=torch.bfloat16)
    wr = torch.zeros(E * d, dtype=torch.bfloat16)
    W = {key: torch.zeros(E * n * d, dtype=torch.bfloat16) for key in ("w_gate", "w_up", "w_down")}
    with pytest.raises(ValueError, match="hidden"):
        moe.forward(p, x[:-1], wr, None, W, None)
    with pytest.raises(ValueError, match="w_router"):
        moe.route(p, x, wr.float(), None, None)
    with pytest.raises(ValueError, match="bias"):
        moe.forward(p, x, wr, torch.zeros(E, dtype=torch.bfloat16), W, None)
    with pytest.raises(ValueError, match="w_down"):
        moe.forward(p, x, wr, None, dict(W, w_down=W["w_down"][:-1]), None)
    with pytest.raises(ValueError, match="ids"):
        moe.permute(p, torch.zeros(T * k - 1, dtype=torch.int32), None)
    p8 = moe.problem(T, d, n, E, k, w="fp8")
    W8 = {key: torch.zeros(E * n * d, dtype=torch.uint8) for key in ("w_gate", "w_up", "w_down")}
    W8.update({key: torch.zeros(E * 4, dtype=torch.float32) for key in ("s_gate", "s_up")})
    W8["s_down"] = torch.zeros(E * 4 - 1, dtype=torch.float32)
    with pytest.raises(ValueError, match="s_down"):
        moe.forward(p8, x, wr, None, W8, None)
