"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
the headers under include/ declare, and rejects bad arguments before touching any device."""
import ctypes
import os
import re

import pytest

import bit_diffusion_amd as bd
from bit_diffusion_amd import _abi

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def _declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(INCLUDE, h), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text,
                                flags=re.M))
    return sorted(names)


def test_header_and_library_exports_agree():
    names = _declared_functions()
    assert set(names) == set(_abi.EXPORTS), names
    L = bd.lib()
    for n in names:
        assert hasattr(L, n), n
    assert bd.svdq_version() == 100


def test_arch_check_strings():
    assert bd.svdq_check_arch("gfx950") == bd.SVDQ_OK
    assert bd.svdq_check_arch("gfx950:sramecc+:xnack-") == bd.SVDQ_OK
    for bad in ("gfx942", "gfx9500", "gfx90a:xnack+", "sm_90", ""):
        assert bd.svdq_check_arch(bad) == bd.SVDQ_ERR_UNSUPPORTED_DEVICE, bad
        assert "not gfx950" in bd.svdq_last_error()
    assert bd.lib().svdq_check_arch(None) == bd.SVDQ_ERR_INVALID_ARG


def test_status_strings():
    for s in range(5):
        assert bd.svdq_status_string(s).startswith("SVDQ_")
    assert "unknown" in bd.svdq_status_string(99)


# A fake, 256-byte aligned address: validation must fail before it is ever dereferenced.
FAKE = 1 << 20


def _quant(cfg, M=16, **kw):
    args = dict(x=FAKE, smooth_inv=FAKE, l1=FAKE, S=1.0, codes=FAKE, scales=FAKE, lora=FAKE)
    args.update(kw)
    return bd.lib().svdq_quantize_act(
        ctypes.byref(cfg) if cfg is not None else None, M, args["x"], args["smooth_inv"],
        args["l1"], args["S"], args["codes"], args["scales"], args["lora"], None)


@pytest.mark.parametrize("field,value,status", [
    ("in_features", 100, bd.SVDQ_ERR_INVALID_ARG),
    ("in_features", 0, bd.SVDQ_ERR_INVALID_ARG),
    ("out_features", 0, bd.SVDQ_ERR_INVALID_ARG),
    ("rank", 8, bd.SVDQ_ERR_INVALID_ARG),
    ("rank", 144, bd.SVDQ_ERR_UNSUPPORTED_CONFIG),
    ("group_size", 128, bd.SVDQ_ERR_INVALID_ARG),
    ("precision", 7, bd.SVDQ_ERR_INVALID_ARG),
])
def test_quantize_rejects_bad_cfg(field, value, status):
    cfg = bd.LayerCfg.make(512, 512, 16)
    setattr(cfg, field, value)
    assert _quant(cfg) == status
    assert bd.svdq_last_error() != ""


def test_quantize_rejects_null_misaligned_and_negative():
    cfg = bd.LayerCfg.make(512, 512, 16)
    assert _quant(None) == bd.SVDQ_ERR_INVALID_ARG
    assert _quant(cfg, x=None) == bd.SVDQ_ERR_INVALID_ARG and "x is NULL" in bd.svdq_last_error()
    assert _quant(cfg, x=FAKE + 8) == bd.SVDQ_ERR_INVALID_ARG
    assert "aligned" in bd.svdq_last_error()
    assert _quant(cfg, l1=None) == bd.SVDQ_ERR_INVALID_ARG
    assert _quant(cfg, M=-1) == bd.SVDQ_ERR_INVALID_ARG
    nv = bd.LayerCfg.make(512, 512, 16, "nvfp4")
    for S in (0.0, -1.0, float("inf"), float("nan")):
        assert _quant(nv, S=S) == bd.SVDQ_ERR_INVALID_ARG


def test_gemm_rejects_bad_args():
    L = bd.lib()
    cfg = bd.LayerCfg.make(512, 512, 16)

    def call(cfg=cfg, act=0, dt=0, out=FAKE, lora=FAKE, M=16, Sa=1.0, Sw=1.0):
        return L.svdq_gemm_w4a4(ctypes.byref(cfg), M, FAKE, FAKE, Sa, FAKE, FAKE, Sw, lora, FAKE,
                                None, act, dt, out, None)

    assert call(act=2) == bd.SVDQ_ERR_INVALID_ARG
    assert call(dt=3) == bd.SVDQ_ERR_INVALID_ARG
    assert call(out=None) == bd.SVDQ_ERR_INVALID_ARG
    assert call(lora=None) == bd.SVDQ_ERR_INVALID_ARG
    assert call(M=-5) == bd.SVDQ_ERR_INVALID_ARG
    nv = bd.LayerCfg.make(512, 512, 16, "nvfp4")
    assert call(cfg=nv, Sw=0.0) == bd.SVDQ_ERR_INVALID_ARG


def test_awq_rejects_bad_args():
    L = bd.lib()

    def call(M=2, K=3072, N=64, gs=64, dt=0, x=FAKE):
        return L.awq_gemm_w4a16(M, K, N, gs, x, FAKE, FAKE, FAKE, None, dt, FAKE, None)

    assert call(K=100) == bd.SVDQ_ERR_INVALID_ARG
    assert call(N=0) == bd.SVDQ_ERR_INVALID_ARG
    assert call(gs=128) == bd.SVDQ_ERR_UNSUPPORTED_CONFIG
    assert call(dt=9) == bd.SVDQ_ERR_INVALID_ARG
    assert call(x=None) == bd.SVDQ_ERR_INVALID_ARG
    assert call(M=-1) == bd.SVDQ_ERR_INVALID_ARG


def test_prepacked_l1_size_and_bad_args():
    # ceil(K / 128) 128-channel steps x rank x 2 bytes; K / 64 odd rounds up by one group
    assert bd.svdq_prepacked_l1_bytes(bd.LayerCfg.make(3072, 3072, 32)) == 3072 * 32 * 2
    assert bd.svdq_prepacked_l1_bytes(bd.LayerCfg.make(192, 64, 16)) == 256 * 16 * 2
    assert bd.svdq_prepacked_l1_bytes(bd.LayerCfg.make(512, 64, 0)) == 0
    L = bd.lib()
    cfg = bd.LayerCfg.make(512, 512, 16)
    assert L.svdq_prepack_l1(ctypes.byref(cfg), None, FAKE, None) == bd.SVDQ_ERR_INVALID_ARG
    assert L.svdq_prepack_l1(ctypes.byref(cfg), FAKE, FAKE + 4, None) == bd.SVDQ_ERR_INVALID_ARG
    nv = bd.LayerCfg.make(512, 512, 16, "nvfp4")
    assert L.svdq_prepack_l1(ctypes.byref(nv), FAKE, FAKE, None) != bd.SVDQ_OK
    # the packed activation kernel needs the prepacked factor whenever the rank is non-zero
    assert L.svdq_quantize_act_packed(ctypes.byref(cfg), 16, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                      None) == bd.SVDQ_ERR_INVALID_ARG
    assert "l1_packed" in bd.svdq_last_error()


def test_merge_lora_rank_rules():
    assert bd.svdq_merged_rank(32, 16) == 48 and bd.svdq_merged_rank(16, 5) == 32
    assert bd.svdq_merged_rank(0, 1) == 16 and bd.svdq_merged_rank(-1, 4) == -1
    L = bd.lib()
    cfg = bd.LayerCfg.make(512, 512, 112)
    # 112 + 32 -> 144 > 128
    assert L.svdq_merge_lora(ctypes.byref(cfg), 32, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE, FAKE,
                             None) == bd.SVDQ_ERR_UNSUPPORTED_CONFIG
    assert L.svdq_merge_lora(ctypes.byref(cfg), 0, FAKE, FAKE, FAKE, FAKE, 1.0, FAKE, FAKE,
                             None) == bd.SVDQ_ERR_INVALID_ARG
    cfg16 = bd.LayerCfg.make(512, 512, 16)
    assert L.svdq_merge_lora(ctypes.byref(cfg16), 8, FAKE, FAKE, None, FAKE, 1.0, FAKE, FAKE,
                             None) == bd.SVDQ_ERR_INVALID_ARG
    assert L.svdq_merge_lora(ctypes.byref(cfg16), 8, FAKE, FAKE, FAKE, FAKE, float("nan"), FAKE,
                             FAKE, None) == bd.SVDQ_ERR_INVALID_ARG


def test_quantize_next_argument_rules():
    """The fused MLP entry point rejects a next layer whose width is not this layer's output
    width, a bad act code, a missing packed output and, at next rank > 0, a missing
    workspace, before touching the device."""
    L = bd.lib()
    f = L.svdq_gemm_w4a4_packed_quantize_next
    cfg = bd.LayerCfg.make(256, 384, 16)

    def call(ncfg, act=1, packed=FAKE, work=FAKE, lora=FAKE):
        return f(ctypes.byref(cfg), 300, FAKE, FAKE, FAKE, FAKE, FAKE, act, ctypes.byref(ncfg),
                 FAKE, FAKE, packed, None, lora, work, None)

    assert call(bd.LayerCfg.make(448, 1, 32)) == bd.SVDQ_ERR_INVALID_ARG
    assert "in_features" in bd.svdq_last_error()
    ok = bd.LayerCfg.make(384, 1, 32)
    assert call(ok, act=2) == bd.SVDQ_ERR_INVALID_ARG
    assert call(ok, packed=None) == bd.SVDQ_ERR_INVALID_ARG
    assert "next_act_packed" in bd.svdq_last_error()
    assert call(ok, work=None) == bd.SVDQ_ERR_INVALID_ARG
    assert "lora_workspace" in bd.svdq_last_error()
    assert call(ok, lora=None) == bd.SVDQ_ERR_INVALID_ARG
    assert call(bd.LayerCfg.make(384, 1, 32, "nvfp4")) == bd.SVDQ_ERR_UNSUPPORTED_CONFIG


def test_weight_quantizer_argument_rules():
    L = bd.lib()
    assert L.svdq_calib_absmax(10, 100, FAKE, FAKE, None) == bd.SVDQ_ERR_INVALID_ARG
    assert L.svdq_calib_absmax(-1, 128, FAKE, FAKE, None) == bd.SVDQ_ERR_INVALID_ARG
    assert L.svdq_calib_absmax(10, 128, None, FAKE, None) == bd.SVDQ_ERR_INVALID_ARG
    cfg = bd.LayerCfg.make(256, 128, 16)
    assert L.svdq_smoothing_factors(ctypes.byref(cfg), FAKE, FAKE, None, FAKE, None) == bd.SVDQ_ERR_INVALID_ARG
    assert "w_absmax" in bd.svdq_last_error()
    assert L.svdq_quantize_residual(ctypes.byref(cfg), FAKE, FAKE, None, FAKE, FAKE, FAKE, None,
                                    None) == bd.SVDQ_ERR_INVALID_ARG
    assert "l1" in bd.svdq_last_error()
    nv = bd.LayerCfg.make(256, 128, 16, "nvfp4")
    assert L.svdq_quantize_residual(ctypes.byref(nv), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                    None) == bd.SVDQ_ERR_INVALID_ARG
    assert "wgt_global_scale" in bd.svdq_last_error()


def test_lowrank_factor_argument_rules():
    L = bd.lib()
    f = L.svdq_lowrank_factors
    big = bd.LayerCfg.make(512, 256, 80)
    assert f(ctypes.byref(big), FAKE, FAKE, FAKE, 80, 2, FAKE, FAKE, None, FAKE, None) == bd.SVDQ_ERR_UNSUPPORTED_CONFIG
    cfg = bd.LayerCfg.make(512, 256, 32)
    assert f(ctypes.byref(cfg), FAKE, FAKE, FAKE, 16, 2, FAKE, FAKE, None, FAKE, None) == bd.SVDQ_ERR_INVALID_ARG
    assert "block" in bd.svdq_last_error()
    assert f(ctypes.byref(cfg), FAKE, FAKE, FAKE, 48, 99, FAKE, FAKE, None, FAKE, None) == bd.SVDQ_ERR_INVALID_ARG
    assert f(ctypes.byref(cfg), FAKE, FAKE, FAKE, 48, 2, FAKE, FAKE, None, None, None) == bd.SVDQ_ERR_INVALID_ARG
    assert "workspace" in bd.svdq_last_error()
    assert bd.svdq_lowrank_workspace_bytes(cfg) > 0


def test_python_binding_raises_with_message():
    cfg = bd.LayerCfg.make(100, 512, 16)
    with pytest.raises(bd.SvdqError) as e:
        bd.svdq_quantize_act(cfg, 4, FAKE, FAKE, FAKE, 1.0, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == bd.SVDQ_ERR_INVALID_ARG and "in_features" in e.value.message


def test_workspace_queries_and_rules():
    """The fused MLP's workspace size is ceil(N / 192) column tiles x the rows padded to 256
    x the next rank x 4 bytes; the K-split GEMM rejects a NULL workspace with a positive
    size, a negative size and a misaligned workspace before touching the device."""
    cfg = bd.LayerCfg.make(3072, 12288, 32)
    ncfg = bd.LayerCfg.make(12288, 3072, 32)
    assert bd.svdq_quantize_next_workspace_bytes(cfg, ncfg, 4608) == 64 * 4608 * 32 * 4
    assert bd.svdq_quantize_next_workspace_bytes(cfg, ncfg, 300) == 64 * 512 * 32 * 4
    assert bd.svdq_quantize_next_workspace_bytes(cfg, bd.LayerCfg.make(12288, 3072, 0), 300) == 0
    odd = bd.LayerCfg.make(256, 448, 16)
    assert bd.svdq_quantize_next_workspace_bytes(odd, bd.LayerCfg.make(448, 1, 16), 1) == 3 * 256 * 16 * 4
    L = bd.lib()
    n = ctypes.c_int64(0)
    assert L.svdq_quantize_next_workspace_bytes(ctypes.byref(cfg), ctypes.byref(cfg), 10,
                                                ctypes.byref(n)) == bd.SVDQ_OK
    assert L.svdq_quantize_next_workspace_bytes(ctypes.byref(cfg), ctypes.byref(ncfg), -1,
                                                ctypes.byref(n)) == bd.SVDQ_ERR_INVALID_ARG
    f = L.svdq_gemm_w4a4_packed_ws
    c = bd.LayerCfg.make(1024, 3072, 32)
    args = (ctypes.byref(c), 4352, FAKE, FAKE, FAKE, FAKE, None, 0, bd.SVDQ_DT_F32, FAKE)
    assert f(*args, None, 1024, None) == bd.SVDQ_ERR_INVALID_ARG
    assert "workspace" in bd.svdq_last_error()
    assert f(*args, FAKE, -16, None) == bd.SVDQ_ERR_INVALID_ARG
    assert f(*args, FAKE + 4, 1024, None) == bd.SVDQ_ERR_INVALID_ARG
    assert "aligned" in bd.svdq_last_error()
    assert L.svdq_gemm_w4a4_packed_workspace_bytes(ctypes.byref(c), -1, 0, 0,
                                                   ctypes.byref(n)) == bd.SVDQ_ERR_INVALID_ARG
    assert L.svdq_gemm_w4a4_packed_workspace_bytes(ctypes.byref(c), 10, 0, 0,
                                                   None) == bd.SVDQ_ERR_INVALID_ARG
