"""The C-ABI library loads and exports every symbol include/fql.h declares (CPU).

No compute calls: only host-side entry points (version, size queries,
format checks, argument validation that fails before any launch).
"""

import ctypes
import os
import re

import pytest

import fp8_quantized_linear_amd as fql

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "fql.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fql_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = fql.lib()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def test_binding_covers_every_declared_symbol():
    assert set(_declared()) == set(fql.SIGNATURES)


def test_version_and_sizes():
    lib = fql.lib()
    assert lib.fql_version() >= 100
    # packed blob: N padded to 16, K to 128; codes Np*Kp/2 bytes, then scales in
    # 512-byte groups of four 128-deep chunks per 16-row tile
    def expect(N, K):
        Np, Kp = -(-N // 16) * 16, -(-K // 128) * 128
        kc4 = -(-(Kp // 128) // 4)
        return Np * Kp // 2 + (Np // 16) * kc4 * 512
    assert fql.packed_nvfp4_bytes(512, 256) == expect(512, 256) == 512 * 128 + 32 * 512
    assert fql.packed_nvfp4_bytes(100, 272) == expect(100, 272)
    assert fql.packed_nvfp4_bytes(4096, 4096) == 4096 * 4096 // 2 + 4096 * 4096 // 16
    assert fql.linear_workspace_bytes(1, 6144, 4096) > 0


def test_can_implement_rules():
    assert fql.can_implement(4096, 4096, 0) == (True, "")
    assert fql.can_implement(5120, 25600, 128)[0]
    ok, why = fql.can_implement(4096, 4100, 0)
    assert not ok and "16" in why
    ok, why = fql.can_implement(4096, 4096, 24)
    assert not ok and "hadamard" in why
    ok, why = fql.can_implement(4096, 4112, 32)
    assert not ok and "multiple" in why


def test_is_supported_without_gpu_reports_reason():
    try:
        import torch

        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except Exception:
        pass
    ok, why = fql.is_supported(0)
    assert not ok and why


@pytest.mark.parametrize("K,hb", [(4100, 0), (4096, 24), (48, 32), (0, 0)])
def test_invalid_shapes_rejected_before_launch(K, hb):
    lib = fql.lib()
    null = ctypes.c_void_p(0)
    st = lib.fql_quant_nvfp4(ctypes.c_void_p(16), 4, K, max(K, 16), 1.0, hb, ctypes.c_void_p(16),
                             ctypes.c_void_p(16), null)
    assert st == -1
    assert lib.fql_last_error().decode()


def test_invalid_scalars_rejected():
    lib = fql.lib()
    p = ctypes.c_void_p(256)
    null = ctypes.c_void_p(0)
    for g in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.fql_quant_nvfp4(p, 4, 64, 64, g, 0, p, p, null) == -1
    # null pointers
    assert lib.fql_quant_nvfp4(null, 4, 64, 64, 1.0, 0, p, p, null) == -1
    # ldx < K
    assert lib.fql_quant_nvfp4(p, 4, 64, 32, 1.0, 0, p, p, null) == -1
    # linear: ldy < N, tiny workspace
    assert lib.fql_linear_nvfp4(p, 1, 64, 64, 1.0, 0, p, 64, 1.0, null, p, 32, p, 1 << 20, null) == -1
    assert lib.fql_linear_nvfp4(p, 1, 64, 64, 1.0, 0, p, 64, 1.0, null, p, 64, p, 16, null) == -4
    # pack into a buffer that is too small
    assert lib.fql_pack_weight_nvfp4(p, p, 64, 64, p, 10, null) == -1


def test_mxfp4_sizes_and_rules():
    # packed MXFP4: N padded to 16, K to 128; codes Np*Kp/2, then one 256-byte
    # scale block (64 lanes x 4 row tiles) per 64-row quad and 128-deep chunk
    def expect(N, K):
        Np, Kp = -(-N // 16) * 16, -(-K // 128) * 128
        return Np * Kp // 2 + (-(-Np // 64)) * (Kp // 128) * 256
    assert fql.packed_mxfp4_bytes(4096, 4096) == expect(4096, 4096) == 4096 * 2048 + 4096 * 128
    assert fql.packed_mxfp4_bytes(100, 96) == expect(100, 96)
    assert fql.linear_mxfp4_workspace_bytes(1, 6144, 4096) > 0
    assert "gemm_sc_kernel<mxfp4," in fql.linear_mxfp4_plan(8192, 4096, 4096)
    assert fql.can_implement(4096, 4096, 0, fmt=fql.FMT_MXFP4) == (True, "")
    ok, why = fql.can_implement(4096, 4112, 0, fmt=fql.FMT_MXFP4)
    assert not ok and "32" in why
    ok, why = fql.can_implement(4096, 4096, 32, fmt=fql.FMT_MXFP4)
    assert not ok and "rotation" in why
    ok, why = fql.can_implement(4096, 4096, 0, fmt=7)
    assert not ok and "unknown" in why


def test_mxfp4_invalid_arguments_rejected():
    lib = fql.lib()
    p = ctypes.c_void_p(256)
    null = ctypes.c_void_p(0)
    assert lib.fql_quant_mxfp4(p, 4, 48, 48, p, p, null) == -1        # K % 32
    assert lib.fql_quant_mxfp4(p, 4, 64, 32, p, p, null) == -1        # ldx < K
    assert lib.fql_quant_mxfp4(null, 4, 64, 64, p, p, null) == -1     # null x
    assert lib.fql_quant_mxfp4(p, 0, 64, 64, p, p, null) == -1        # M = 0
    assert lib.fql_quant_mxfp4(p, 4, 64, 64, ctypes.c_void_p(258), p, null) == -1  # codes alignment
    assert lib.fql_pack_weight_mxfp4(p, p, 64, 64, p, 10, null) == -1  # buffer too small
    assert lib.fql_linear_mxfp4(p, 1, 64, 64, p, 64, 1.0, null, p, 32, p, 1 << 20, null) == -1
    assert lib.fql_linear_mxfp4(p, 1, 64, 64, p, 64, 1.0, null, p, 64, p, 16, null) == -4
    assert lib.fql_linear_mxfp4(p, 1, 64, 64, p, 64, float("nan"), null, p, 64, p, 1 << 20, null) == -1
    assert lib.fql_last_error().decode()


@pytest.mark.parametrize("fmt", ["mxfp8", "fp8", "fp8_block"])
def test_fp8_family_sizes(fmt):
    N, K = 14336, 4096
    Np, KC = N, K // 128
    code = N * K
    scale = {"mxfp8": (-(-Np // 64)) * KC * 256, "fp8": 0,
             "fp8_block": -(-((N // 128) * KC * 4) // 256) * 256}[fmt]
    assert fql._size_query(f"fql_packed_{fmt}_bytes", N, K) == code + scale
    assert fql.linear_sc_workspace_bytes(fmt, 4096, N, K) >= 64 * 1024 + 4096 * K
    assert f"gemv_sc_kernel<{fmt}," in fql.linear_sc_plan(fmt, 1, N, K)
    assert f"gemm_sc_kernel<{fmt}," in fql.linear_sc_plan(fmt, 4096, N, K)


def test_fp8_family_can_implement():
    assert fql.can_implement(14336, 4096, 0, fmt=fql.FMT_MXFP8)[0]
    assert fql.can_implement(14336, 4096, 0, fmt=fql.FMT_FP8)[0]
    assert fql.can_implement(14336, 4096, 0, fmt=fql.FMT_FP8_BLOCK)[0]
    ok, why = fql.can_implement(14336 + 64, 4096, 0, fmt=fql.FMT_FP8_BLOCK)
    assert not ok and "128" in why
    ok, why = fql.can_implement(14336, 4096 + 32, 0, fmt=fql.FMT_FP8_BLOCK)
    assert not ok and "128" in why
    assert fql.can_implement(100, 4096 + 32, 0, fmt=fql.FMT_FP8)[0]


def test_fp8_family_invalid_arguments_rejected():
    lib = fql.lib()
    p = ctypes.c_void_p(256)
    null = ctypes.c_void_p(0)
    # per-tensor: bad scales, K % 32
    for s in (0.0, -2.0, float("inf"), float("nan")):
        assert lib.fql_quant_fp8(p, 4, 64, 64, s, p, null) == -1
    assert lib.fql_quant_fp8(p, 4, 48, 48, 1.0, p, null) == -1
    assert lib.fql_linear_fp8(p, 1, 64, 64, 0.0, p, 64, 1.0, null, p, 64, p, 1 << 20, null) == -1
    # block: K and N multiples of 128
    assert lib.fql_quant_fp8_block(p, 4, 96, 96, p, p, null) == -1
    assert lib.fql_quant_fp8_block_weight_f32(p, 100, 128, 128, p, p, null) == -1
    assert lib.fql_pack_weight_fp8_block(p, p, 64, 128, p, 1 << 20, null) == -1
    assert lib.fql_linear_fp8_block(p, 1, 128, 128, p, 128, 1.0, null, p, 128, p, 16, null) == -4
    # MXFP8: workspace too small, ldy < N
    assert lib.fql_linear_mxfp8(p, 1, 64, 64, p, 64, 1.0, null, p, 64, p, 16, null) == -4
    assert lib.fql_linear_mxfp8(p, 1, 64, 64, p, 64, 1.0, null, p, 32, p, 1 << 20, null) == -1
    assert lib.fql_last_error().decode()


def test_warmup_token_counts():
    # 1 (a decode step), every positive graph-capture size, and the largest batch,
    # each once (B12X write-up, Implementation: the warmup token set)
    import fp8_quantized_linear_amd as fql

    assert fql.token_counts_for_warmup(8192) == [1, 8192]
    assert fql.token_counts_for_warmup(512, graph_sizes=(4, 1, 0, -2, 256, 4)) == [1, 4, 256, 512]


def test_dynamic_scalar_buffer_size_matches_header():
    import fp8_quantized_linear_amd as fql

    text = open(os.path.join(ROOT, "include", "fql.h")).read()
    m = re.search(r"#define FQL_DYNAMIC_SCALARS (\d+)", text)
    assert m and int(m.group(1)) == fql.DYNAMIC_SCALARS


def test_sibling_decode_plan_fuses_the_quantizer():
    # M <= 16 runs one launch (the activation quantized inside the GEMV's
    # workgroups) when the operand fits in LDS next to the weight ring
    import fp8_quantized_linear_amd as fql

    for fmt in ("mxfp4", "mxfp8", "fp8", "fp8_block"):
        assert ",FQ=1>" in fql.linear_sc_plan(fmt, 1, 14336, 4096)
        assert "sc_quant_operand_kernel" not in fql.linear_sc_plan(fmt, 16, 14336, 4096)
        assert "sc_quant_operand_kernel" in fql.linear_sc_plan(fmt, 17, 14336, 4096)
    # an operand too large for LDS keeps the two-launch path
    assert ",FQ=1>" in fql.linear_sc_plan("mxfp8", 1, 4096, 65536)  # compact: M rows only
    assert "sc_quant_operand_kernel" in fql.linear_sc_plan("mxfp8", 16, 4096, 65536)


def test_small_m_plans_pack_the_activation():
    # the per-wave-ring kernel reads the activation packed like a weight, written by
    # the quantizer pass, or under a transform by the transform kernel; the
    # workspace covers every plan of the shape
    import fp8_quantized_linear_amd as fql

    for M, N, K in ((8, 4096, 14336), (32, 4096, 14336), (32, 6144, 4096), (8, 28672, 4096)):
        plain = fql.linear_plan(M, N, K)
        assert plain.startswith("quant_nvfp4_apack_kernel + gemv_ring_kernel<"), plain
        tr = fql.linear_plan(M, N, K, aligned=False, transform=True)
        assert tr.startswith("transform_quant_kernel + gemv_ring_kernel<"), tr
        assert "apack" in fql.linear_plan(M, N, K, aligned=False)  # dynamic scale, no transform
        assert fql.linear_workspace_bytes(M, N, K) >= 64 * 1024 + 16 * ((M + 15) // 16) * K * 2


# ---------------------------------------------------------------------------
# host-side scalars of the layer: the library's formulas against the oracle's
# and against closed forms (no GPU needed)
# ---------------------------------------------------------------------------

def _amax_values():
    import numpy as np

    r = np.random.default_rng(31)
    vals = np.concatenate([r.uniform(1e-3, 1e3, 2000), np.exp(r.uniform(-80, 80, 2000)),
                           [1.0, 3.0, 6.0, 448.0, 2688.0, 1e-45, 1e-38, 3.4e38, 7.0 / 3.0]])
    return vals.astype(np.float32)


def test_global_scale_matches_oracle_and_closed_forms():
    import numpy as np
    from oracle import nvfp4 as Q

    for a in _amax_values():
        assert np.float32(fql.global_scale_from_amax(a)) == Q.global_scale_from_amax(a), a
    assert fql.global_scale_from_amax(0.0) == 1.0
    assert fql.global_scale_from_amax(2688.0) == 1.0
    assert fql.global_scale_from_amax(1.0) == 2688.0
    assert fql.global_scale_from_amax(6.0) == 448.0
    assert fql.global_scale_from_amax(1e-40) == 2.0 ** 118      # the cap


def test_alpha_matches_oracle_and_closed_forms():
    import numpy as np
    from oracle import transform as TR

    r = np.random.default_rng(32)
    for gx, gw in np.exp(r.uniform(-20, 20, (2000, 2))).astype(np.float32):
        assert np.float32(fql.nvfp4_alpha(gx, gw)) == TR.dynamic_alpha(gx, gw)
    assert fql.nvfp4_alpha(1.0, 1.0) == 1.0
    assert fql.nvfp4_alpha(2.0, 0.25) == 2.0
    assert fql.nvfp4_alpha(2688.0, 1.0) == float(np.float32(1.0 / 2688.0))


def test_fp8_scales_match_oracle_and_closed_forms():
    import numpy as np
    from oracle import fp8 as P

    for a in _amax_values():
        s = P.scale_from_amax(a)
        assert np.float32(fql.fp8_scale_from_amax(a)) == (s if s > 0 else np.float32(1.0)), a
    assert fql.fp8_scale_from_amax(448.0) == 1.0
    assert fql.fp8_scale_from_amax(0.0) == 1.0
    assert fql.fp8_scale_from_amax(896.0) == 2.0
    r = np.random.default_rng(33)
    for sx, sw in np.exp(r.uniform(-30, 30, (2000, 2))).astype(np.float32):
        assert np.float32(fql.fp8_output_scale(sx, sw)) == P.output_scale(sx, sw)
    assert fql.fp8_output_scale(0.5, 0.25) == 0.125


@pytest.mark.parametrize("name,args", [("fql_nvfp4_global_scale", (-1.0,)),
                                       ("fql_nvfp4_global_scale", (float("inf"),)),
                                       ("fql_nvfp4_global_scale", (float("nan"),)),
                                       ("fql_nvfp4_alpha", (0.0, 1.0)),
                                       ("fql_nvfp4_alpha", (1.0, float("inf"))),
                                       ("fql_fp8_scale", (-2.0,)),
                                       ("fql_fp8_output_scale", (1.0, -1.0))])
def test_host_scalars_reject_invalid_inputs(name, args):
    out = ctypes.c_float()
    assert getattr(fql.lib(), name)(*[ctypes.c_float(a) for a in args], ctypes.byref(out)) == -1
    assert fql.lib().fql_last_error().decode()


def test_plan_override_set_and_cleared():
    default = fql.linear_plan(100, 4096, 4096)
    fql.set_plan_override("kind=1")
    try:
        assert "gemm_tiled_kernel<MT=4,NT=2,WM=2>" in fql.linear_plan(100, 4096, 4096)
    finally:
        fql.set_plan_override(None)
    assert fql.linear_plan(100, 4096, 4096) == default
    with fql.plan_override("8,1,3,0", which="sc_gemv"):
        pass  # not a built GEMV: the default stays
    assert fql.lib().fql_set_plan_override(7, None) == -1


def test_lds32_layouts_and_tile_order_in_the_plan():
    # above 128 rows: 128 x 256 tiles on 8 column waves in XCD bands of 4 row
    # groups (clamped to the row groups there are); up to 128 rows 4 waves
    assert ("gemm_lds32_kernel<MT=4,NT=1,ST=3,WN=8> grid=7168 splits=1 xcd_bands=4"
            in fql.linear_plan(8192, 28672, 4096))
    assert "xcd_bands=2" in fql.linear_plan(256, 51200, 5120)
    assert "gemm_lds32_kernel<MT=2,NT=1,ST=4> grid=192 splits=2" in fql.linear_plan(128, 6144, 4096)
    # the band is selectable; a configuration that is not built falls back to kind 1
    with fql.plan_override("kind=3,mt=4,nt=1,st=3,cw=4,splits=1,xg=0"):
        plan = fql.linear_plan(1100, 2100, 1152)
        assert "gemm_lds32_kernel<MT=4,NT=1,ST=3> grid=153 splits=1" in plan and "xcd" not in plan
    with fql.plan_override("kind=3,mt=2,nt=2,st=3,splits=1"):
        assert "gemm_tiled_kernel" in fql.linear_plan(1100, 2100, 1152)
    with fql.plan_override("kind=3,mt=4,nt=1,st=3,wm=1,cw=8,splits=1,xg=3"):
        assert "WN=8> grid=81 splits=1 xcd_bands=3" in fql.linear_plan(1100, 2100, 1152)


def test_last_round_tiles_split_along_k():
    # 640 tiles of 128 x 256 leave the third round of 256 half full: its 128
    # tiles take two workgroups each; full rounds and short K stay whole
    assert "grid=768 splits=1 xcd_bands=4 tail=128x2" in fql.linear_plan(4096, 5120, 25600)
    assert "tail" not in fql.linear_plan(2048, 6144, 4096)    # 32 chunks of K: kept whole
    assert "tail" not in fql.linear_plan(8192, 28672, 4096)   # 7168 tiles: 28 full rounds
    assert "tail" not in fql.linear_plan(256, 51200, 5120)    # 400 tiles: last round 56% full
    with fql.plan_override("tail=2"):
        assert "grid=512 splits=1 xcd_bands=4 tail=128x2" in fql.linear_plan(2048, 6144, 4096)
        assert "tail" not in fql.linear_plan(2048, 6144, 512)  # 4 chunks of K: too short to split
    with fql.plan_override("tail=4"):
        assert "grid=272 splits=1 xcd_bands=4 tail=4x4" in fql.linear_plan(1650, 5120, 2048)
    with fql.plan_override("tail=1"):
        assert "grid=640 splits=1 xcd_bands=4" in fql.linear_plan(4096, 5120, 25600)
    with fql.plan_override("tail=3"):
        assert "grid=896 splits=1 xcd_bands=4 tail=128x3" in fql.linear_plan(4096, 5120, 25600)
    # the split tiles' partial sums are part of the workspace
    with fql.plan_override("tail=1"):
        whole = fql.linear_workspace_bytes(4096, 5120, 25600)
    assert fql.linear_workspace_bytes(4096, 5120, 25600) == whole + 128 * 2 * 8 * 16 * 64 * 16


def test_sibling_last_round_tiles_split_along_k():
    # MXFP4 at M = 4096: 896 tiles of 256 x 256, the last 128 in two halves
    # MXFP4 at M = 4096: 896 tiles of 256 x 256, the last 128 split in two
    # along K when K is long; at K = 4096 (32 chunks) they stay whole
    assert "grid=1024 splits=1 tail=128x2" in fql.linear_sc_plan("mxfp4", 4096, 14336, 8192)
    assert "grid=896 splits=1" in fql.linear_sc_plan("mxfp4", 4096, 14336, 4096)
    assert "tail" not in fql.linear_sc_plan("fp8", 4096, 14336, 8192)  # 1792 tiles: 7 rounds
    assert "tail" not in fql.linear_sc_plan("mxfp4", 2048, 14336, 8192)  # last round 75% full
    with fql.plan_override("2,4,8,4,4,0,2", which="sc_gemm"):
        assert "grid=1024 splits=1 tail=128x2" in fql.linear_sc_plan("mxfp4", 4096, 14336, 4096)
    with fql.plan_override("2,4,8,4,4,0,1", which="sc_gemm"):
        assert "grid=896 splits=1" in fql.linear_sc_plan("mxfp4", 4096, 14336, 8192)


def test_rotation_widens_the_fused_kernels_workgroups_at_m1():
    # with a Hadamard rotation every workgroup of the fused kernel also rotates
    # the activation: two column tiles per workgroup on the narrow layers, and
    # the wide layers (>= 1024 column tiles) quantize and rotate once instead
    assert "NTW=1" in fql.linear_plan(1, 5120, 25600)
    assert "linear_gemv_kernel<W=8,NTW=2," in fql.linear_plan(1, 5120, 25600, hadamard_block=64)
    assert "linear_gemv_kernel<W=4,NTW=1," in fql.linear_plan(1, 51200, 5120)
    for hb in (16, 32, 64, 128):
        assert ("quant_nvfp4_apack_kernel + gemv_ring_kernel<W=4,MT=1,NT=4,D=3>"
                in fql.linear_plan(1, 51200, 5120, hadamard_block=hb))
    assert "NTW=1" in fql.linear_plan(1, 4096, 14336)
    # plans with a quantizer pass, and the transform's plan, do not depend on it
    for M, N, K in [(32, 5120, 25600), (256, 5120, 25600), (4096, 51200, 5120)]:
        assert fql.linear_plan(M, N, K) == fql.linear_plan(M, N, K, hadamard_block=128)
    assert (fql.linear_plan(1, 5120, 25600, aligned=False, transform=True)
            == fql.linear_plan(1, 5120, 25600, aligned=False, transform=True, hadamard_block=64))


def test_binding_holds_no_numeric_formula():
    # every scale and alpha of the layer comes from the library; the binding
    # only marshals arguments: no numpy, no float literal but the unit alpha,
    # no float division or power
    import ast

    src = open(os.path.join(ROOT, "fp8_quantized_linear_amd", "__init__.py")).read()
    tree = ast.parse(src)
    for node in ast.walk(tree):
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module]
            assert not any(m and m.startswith("numpy") for m in mods)
        if isinstance(node, ast.Constant) and isinstance(node.value, float):
            assert node.value == 1.0, node.value
        if isinstance(node, ast.BinOp):
            assert not isinstance(node.op, (ast.Div, ast.Pow)), ast.unparse(node)
