"""qmm_run_noalloc (the split-K workspace from the library's own device
array) against qmm_run with a caller workspace, through the C ABI."""
import numpy as np
import pytest

from bit_quantized_matmul_affine_amd import binding as b
from bit_quantized_matmul_affine_amd import synth
from tests.gpu_util import Runner, check_against_oracle, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    b.lib()


def _both(r, rows, **kw):
    """(workspace the automatic choice needs, stats, qmm_run's y, qmm_run_noalloc's y)."""
    import torch
    plan = r.lin.plan
    need = b.lib().qmm_workspace_bytes_ex(plan.handle, 0, 0, 0, 0, rows)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    y_run = plan.run(r.x[:rows], r.lin.codes, r.lin.sb, workspace=ws, **kw)
    y_na = plan.run_noalloc(r.x[:rows], r.lin.codes, r.lin.sb)
    torch.cuda.synchronize()
    return need, plan.stats(), b.to_numpy_bits(y_run), b.to_numpy_bits(y_na)


def test_noalloc_matches_qmm_run_two_calls_in_a_row():
    """3-bit 5120 -> 10240: 64 rows (the split slab kernel, 5.3 MB of
    workspace), then 40 rows (48-row blocks: a smaller workspace); the
    second call reuses the array the first left behind.  Each equals
    qmm_run's output bit for bit and passes the oracle check."""
    (p,) = synth.workload(2, M=64)
    r = Runner(p, max_rows=64)
    for rows in (64, 40):
        say("noalloc rows", rows)
        need, st, y_run, y_na = _both(r, rows)
        assert need > 0 and st["last_splitk"] == 2, (need, st)
        assert np.array_equal(y_na, y_run), "rows %d differ from qmm_run" % rows
        check_against_oracle(p.rows(rows), y_na, rows=rows, sample=(3000, rows),
                             label="noalloc rows %d" % rows)


def test_noalloc_step_layout_plan():
    """A plan of another format (8-bit weights, groups of 32: the step layout
    on the streaming and resident kernels, no workspace) through
    qmm_run_noalloc equals qmm_run."""
    p = synth.small(56, bits=8, K=2048, N=512, M=16, group_size=32)
    r = Runner(p, max_rows=16)
    for rows in (16, 1):
        say("noalloc step layout rows", rows)
        need, st, y_run, y_na = _both(r, rows)
        assert need == 0 and st["last_variant"] in ("stream", "resident"), (need, st)
        assert np.array_equal(y_na, y_run)
        check_against_oracle(p.rows(rows), y_na, rows=rows, label="noalloc 8-bit g32 rows %d" % rows)


def test_noalloc_smaller_plan_after_larger_and_no_workspace_case():
    """A different, smaller projection after the large one (its ticket words
    sit at the same place in the array), then a call that needs no workspace
    at all, and f32 outputs."""
    p = synth.small(55, bits=4, K=5120, N=208, M=40)
    r = Runner(p, max_rows=40)
    for rows in (40, 33, 1):
        say("noalloc small plan rows", rows)
        need, st, y_run, y_na = _both(r, rows)
        assert (need > 0) == (rows > 32), (rows, need)
        assert np.array_equal(y_na, y_run)
        check_against_oracle(p.rows(rows), y_na, rows=rows, label="noalloc small rows %d" % rows)
    q = synth.small(56, bits=3, K=8192, N=96, M=48)
    rq = Runner(q, max_rows=48, f32_out=True)
    need, st, y_run, y_na = _both(rq, 48)
    assert need > 0 and np.array_equal(y_na, y_run)
    check_against_oracle(q, y_na, label="noalloc f32 out", out_dtype="f32")


def test_noalloc_rejects_calls_beyond_its_array():
    """65536 outputs at 64 rows need more than the array holds: the call is
    refused before any launch (the buffers are full-size and zero, so
    nothing would be out of bounds even if it ran)."""
    import torch
    plan = b.Plan(3, 5120, 65536, 64, "bf16")
    assert b.lib().qmm_workspace_bytes_ex(plan.handle, 0, 0, 0, 0, 64) > 8 << 20
    cb, sbb = plan.packed_bytes()
    codes = torch.zeros(cb // 4, dtype=torch.int32, device="cuda")
    sb = torch.zeros(sbb // 2, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(64, 5120, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(b.QmmError) as ei:
        plan.run_noalloc(x, codes, sb)
    assert ei.value.status == b.QMM_ERR_WORKSPACE
    y = plan.run_noalloc(x[:8], codes, sb)       # 8 rows need none: runs
    torch.cuda.synchronize()
    assert torch.count_nonzero(y.float()) == 0
