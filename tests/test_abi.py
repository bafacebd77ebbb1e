"""The C ABI on a host without a GPU: the library loads, exports every entry
point include/qmm.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from bit_quantized_matmul_affine_amd import binding as b

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qmm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for must in ("qmm_create", "qmm_run", "qmm_destroy", "qmm_prepack", "qmm_debug_unpack",
                 "qmm_workspace_bytes", "qmm_last_error", "qmm_get_stats"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = b.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in b.SIGNATURES, name


@pytest.mark.parametrize("kw,status", [
    (dict(bits=7), b.QMM_ERR_INVALID_ARG),          # not an MLX width
    (dict(bits=5), b.QMM_ERR_UNSUPPORTED),          # MLX width, no kernel here
    (dict(bits=6), b.QMM_ERR_UNSUPPORTED),
    (dict(group_size=48), b.QMM_ERR_INVALID_ARG),
    (dict(K=500), b.QMM_ERR_INVALID_ARG),           # not a multiple of the group
    (dict(K=192), b.QMM_ERR_UNSUPPORTED),           # group-aligned, not 128-aligned
    (dict(N=24), b.QMM_ERR_UNSUPPORTED),
    (dict(N=0), b.QMM_ERR_INVALID_ARG),
    (dict(max_rows=0), b.QMM_ERR_INVALID_ARG),
    (dict(x_dtype="f16"), b.QMM_ERR_INVALID_ARG),
])
def test_create_rejects(kw, status):
    args = dict(bits=4, K=512, N=512, max_rows=4, x_dtype="bf16", group_size=64)
    args.update(kw)
    if args["x_dtype"] == "f16":
        d = b.QmmDesc(args["bits"], 64, args["K"], args["N"], args["max_rows"], 7, 1, 0)
        h = ctypes.c_void_p()
        assert b.lib().qmm_create(ctypes.byref(d), ctypes.byref(h)) == status
        assert h.value is None
        return
    with pytest.raises(b.QmmError) as ei:
        b.Plan(args["bits"], args["K"], args["N"], args["max_rows"], args["x_dtype"],
               group_size=args["group_size"])
    assert ei.value.status == status


def test_create_accepts_every_workload_shape():
    for bits, K, N in [(4, 512, 512), (4, 5120, 10240), (3, 5120, 10240), (4, 3840, 15360),
                       (4, 15360, 3840), (4, 8192, 28672)]:
        p = b.Plan(bits, K, N, 128, "bf16")
        cb, sbb = p.packed_bytes()
        assert cb == N * K * bits // 8          # same byte count as the MLX layout
        assert sbb == 2 * N * (K // 64) * 2


def test_run_validation_without_gpu():
    L = b.lib()
    p = b.Plan(3, 5120, 10240, 16, "bf16")
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first
    # rows out of range: the page's "no rows" error
    assert L.qmm_run(p.handle, fake, fake, fake, fake, 0, None, 0, None) == b.QMM_ERR_INVALID_ARG
    assert L.qmm_run(p.handle, fake, fake, fake, fake, 17, None, 0, None) == b.QMM_ERR_INVALID_ARG
    # NULL and misaligned pointers
    assert L.qmm_run(p.handle, None, fake, fake, fake, 1, None, 0, None) == b.QMM_ERR_INVALID_ARG
    assert L.qmm_run(p.handle, ctypes.c_void_p((1 << 20) + 2), fake, fake, fake, 1, None, 0,
                     None) == b.QMM_ERR_INVALID_ARG
    # a forced K split needs a workspace
    assert L.qmm_run_ex(p.handle, b.VARIANT_MFMA, 1, 1, 4, fake, fake, fake, fake, 4, None, 0,
                        None) == b.QMM_ERR_WORKSPACE
    assert b"workspace" in L.qmm_last_error()
    # MFMA takes bf16 activations only
    pf = b.Plan(4, 512, 512, 1, "f32")
    assert L.qmm_run_ex(pf.handle, b.VARIANT_MFMA, 0, 0, 0, fake, fake, fake, fake, 1, None, 0,
                        None) == b.QMM_ERR_UNSUPPORTED
    assert L.qmm_run(None, fake, fake, fake, fake, 1, None, 0, None) == b.QMM_ERR_INVALID_ARG


def test_workspace_sizes_are_bounded():
    """Partial sums only: far below the size of a materialized W."""
    p = b.Plan(3, 5120, 10240, 64, "bf16")
    for rows in (1, 9, 16, 32, 64):
        ws = p.workspace_bytes(rows)
        assert ws <= 16 * rows * 10240 * 4 + 65536
        assert ws < 10240 * 5120 * 2 // 8


def test_automatic_workspace_follows_the_row_blocks():
    """Host dispatch, no GPU: the automatic choice's workspace is the split
    slab form's partial tiles at 33..64 rows (48-row blocks needing less than
    64-row ones), none for the streaming and resident kernels, and for a long
    call the largest of its blocks (a 65- or 80-row call: one 64-row block,
    then a tail on the streaming or resident kernel); a wide-kernel call on
    a shape whose grid fills the chip needs none."""
    p = b.Plan(3, 5120, 208, 128, "bf16")
    auto = lambda rows: b.lib().qmm_workspace_bytes_ex(p.handle, 0, 0, 0, 0, rows)
    assert auto(1) == 0 and auto(9) == 0 and auto(16) == 0
    w48, w64 = auto(48), auto(64)
    assert 0 < w48 < w64
    assert auto(33) == w48
    assert auto(65) == w64 and auto(80) == w64 and auto(128) == w64
    q = b.Plan(4, 8192, 28672, 128, "bf16")
    assert b.lib().qmm_workspace_bytes_ex(q.handle, 0, 0, 0, 0, 128) == 0


@pytest.mark.parametrize("bits,gs", [(2, 32), (2, 64), (2, 128), (3, 32), (3, 128), (4, 32),
                                     (4, 128), (8, 32), (8, 64), (8, 128)])
def test_format_variants_plan_on_the_generic_kernel(bits, gs):
    """Every other MLX format builds a plan whose packed codes keep MLX's
    byte count and that needs no workspace; its scales and biases keep their
    count too.  3- and 4-bit groups of 128 go to the native layout, which
    stores the pair once per 64 values (the group's pair for each half), with
    the group-64 plan's workspace."""
    for sb_dtype, size in (("bf16", 2), ("f32", 4)):
        p = b.Plan(bits, 512, 64, 4, "bf16", sb_dtype=sb_dtype, group_size=gs)
        cb, sbb = p.packed_bytes()
        assert cb == 64 * 512 * bits // 8
        native = bits in (3, 4) and gs == 128
        assert sbb == 2 * 64 * (512 // (64 if native else gs)) * size
        if native:  # the workspace of the group-64 plan of the same shape
            q = b.Plan(bits, 512, 64, 4, "bf16", sb_dtype=sb_dtype)
            assert p.workspace_bytes(4) == q.workspace_bytes(4)
        else:
            assert p.workspace_bytes(4) == 0


def test_f32_output_flag():
    """QMM_FLAG_F32_OUT is the one defined flag; the fused gate/up entry point
    (bf16 output by definition) rejects such plans before any HIP call."""
    L = b.lib()
    h = ctypes.c_void_p()
    d = b.QmmDesc(3, 64, 5120, 10240, 16, b.QMM_BF16, b.QMM_BF16, 2)
    assert L.qmm_create(ctypes.byref(d), ctypes.byref(h)) == b.QMM_ERR_INVALID_ARG
    assert h.value is None
    p = b.Plan(3, 5120, 10240, 16, "bf16", f32_out=True)
    fake = ctypes.c_void_p(1 << 20)
    assert L.qmm_run_gate_up(p.handle, fake, fake, fake, fake, fake, fake, 4, 0,
                             None) == b.QMM_ERR_UNSUPPORTED
    assert b"F32_OUT" in L.qmm_last_error()
    # the same validation as any plan otherwise
    assert L.qmm_run(p.handle, fake, fake, fake, fake, 0, None, 0, None) == b.QMM_ERR_INVALID_ARG


def test_noalloc_refuses_oversized_calls_without_gpu():
    """qmm_run_noalloc checks the workspace a call needs against its array
    (QMM_NOALLOC_MAX_WORKSPACE, 8 MiB) before any HIP call."""
    L = b.lib()
    fake = ctypes.c_void_p(1 << 20)
    assert L.qmm_run_noalloc(None, fake, fake, fake, fake, 1, None) == b.QMM_ERR_INVALID_ARG
    p = b.Plan(3, 5120, 65536, 64, "bf16")
    assert L.qmm_workspace_bytes_ex(p.handle, 0, 0, 0, 0, 64) > 8 << 20
    assert L.qmm_run_noalloc(p.handle, fake, fake, fake, fake, 64, None) == b.QMM_ERR_WORKSPACE
    assert b"qmm_run_noalloc holds" in L.qmm_last_error()
    q = b.Plan(3, 5120, 10240, 64, "bf16")
    assert 0 < L.qmm_workspace_bytes_ex(q.handle, 0, 0, 0, 0, 64) <= 8 << 20


def test_group_sum_entry_points_validate_without_gpu():
    """qmm_sum_group names the group width of the sums qmm_run_sums takes (64
    on the native layout, groups of 128 included; the group size otherwise);
    qmm_run_sums and qmm_residual_rms_norm_ex reject bad sums arguments before
    any HIP call."""
    L = b.lib()
    assert b.Plan(3, 5120, 10240, 16, "bf16").sum_group() == 64
    assert b.Plan(4, 5120, 10240, 16, "bf16", group_size=128).sum_group() == 64
    assert b.Plan(2, 5120, 10240, 16, "bf16", group_size=32).sum_group() == 32
    assert b.Plan(8, 5120, 10240, 16, "bf16", group_size=128).sum_group() == 128
    assert L.qmm_sum_group(None) == 0
    p = b.Plan(3, 5120, 10240, 16, "bf16")
    fake = ctypes.c_void_p(1 << 20)
    run = lambda sums, ld, rows: L.qmm_run_sums(p.handle, fake, sums, ld, fake, fake, fake, rows,
                                                None, 0, None)
    assert run(None, 16, 4) == b.QMM_ERR_INVALID_ARG
    assert b"x_sums is NULL" in L.qmm_last_error()
    assert run(fake, 8, 4) == b.QMM_ERR_INVALID_ARG       # not a multiple of 16
    assert run(fake, 16, 17) == b.QMM_ERR_INVALID_ARG     # below rows rounded up to 16
    assert run(ctypes.c_void_p((1 << 20) + 4), 16, 4) == b.QMM_ERR_INVALID_ARG  # misaligned
    norm = lambda sums, gs, ld, D: L.qmm_residual_rms_norm_ex(fake, fake, fake, fake, fake, sums,
                                                             gs, ld, 4, D, 1e-5, b.QMM_BF16, None)
    assert norm(fake, 48, 16, 512) == b.QMM_ERR_INVALID_ARG   # not an MLX group size
    assert norm(fake, 64, 16, 96) == b.QMM_ERR_INVALID_ARG    # D not a multiple of 64
    assert norm(fake, 64, 2, 512) == b.QMM_ERR_INVALID_ARG    # sums_ld below rows


def test_group_sum_shapes_checked_by_the_binding():
    """The binding rejects sums buffers with fewer groups than the
    projection's K (or the norm's D) needs, before any library call."""
    import torch
    p = b.Plan(3, 1024, 64, 4, "bf16")
    x = torch.zeros(4, 1024, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="groups"):
        p.run_sums(x, torch.zeros(1024 // 64 - 1, 16), None, None)
    w = torch.zeros(1024, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="groups"):
        b.residual_rms_norm(x, x, w, 1e-5, group_sums=torch.zeros(1024 // 32 - 1, 16),
                            group_size=32)


def test_attention_workspace_sizes():
    # none for one block; else the partial outputs [H, G, D] and the
    # (max, sum) pairs [H, G, 2] of G = ceil(N / 256) blocks
    L = b.lib()
    assert L.qmm_attention_workspace_bytes(16, 256, 256) == 0
    assert L.qmm_attention_workspace_bytes(16, 1, 128) == 0
    assert L.qmm_attention_workspace_bytes(16, 8192, 256) == 16 * 32 * 258 * 4
    assert L.qmm_attention_workspace_bytes(65, 257, 128) == 65 * 2 * 130 * 4
    assert L.qmm_attention_workspace_bytes(0, 8192, 256) == 0
