"""HIP-graph capture and replay of every entry point: each kernel family of
the projection (the split-K ticket protocol of the 64-row kernel included:
its tickets must be re-armed by every replay), the fused gate/up, residual
add + RMS norm and decode attention with a block merge.  Everything is
captured once, then replayed several times with eager calls of the same
work and synchronizations between the replays; the graph outputs are
poisoned before each replay, and every replay must equal the eager results
bit for bit (same kernels, fixed reduction orders)."""
import pytest

from bit_quantized_matmul_affine_amd import binding as b, synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

# (family, split K, bits, K, N, rows, group size, scale dtype); every family
# is the default for its shape except the wide one, forced at this small N;
# the 2- and 8-bit cases run on the step layout (streaming and resident
# kernels) and, with f32 scales, on MLX's layout (vector-ALU kernel)
PROJECTIONS = [
    ("stream", 1, 3, 5120, 160, 1, 64, "bf16"),
    ("resident", 1, 3, 5120, 160, 9, 64, "bf16"),
    ("slab", 1, 3, 5120, 208, 32, 64, "bf16"),
    ("slab", 2, 3, 5120, 208, 64, 64, "bf16"),
    ("wide", 1, 4, 2048, 256, 100, 64, "bf16"),
    ("stream", 1, 2, 1024, 64, 2, 64, "bf16"),
    ("resident", 1, 8, 1024, 64, 9, 32, "bf16"),
    ("generic", 1, 2, 1024, 64, 2, 64, "f32"),
]
FORCED = {"wide"}


def _work():
    """Callables run(outs) that enqueue one call each on the current stream,
    and the output tensors each one needs."""
    import torch
    calls = []
    for i, (fam, split, bits, K, N, M, gs, sbd) in enumerate(PROJECTIONS):
        p = synth.small(700 + i, bits=bits, K=K, N=N, M=M, group_size=gs, sb_dtype=sbd)
        lin = b.QuantizedLinear(p, max_rows=M)
        x = b.to_device(p.x)
        v = fam if fam in FORCED else "auto"
        ws = lin.plan.workspace(lin.plan.workspace_bytes(M), x.device)
        lin(x, workspace=ws, variant=v)
        torch.cuda.synchronize()
        st = lin.plan.stats()
        assert st["last_variant"] == fam and st["last_splitk"] == split, (fam, split, st)

        def run(out, lin=lin, x=x, ws=ws, v=v):
            lin(x, out=out, workspace=ws, variant=v)
        calls.append(("%s S=%d M=%d" % (fam, split, M), run,
                      lambda N=N, M=M: torch.empty(M, N, dtype=torch.bfloat16, device="cuda")))

    g = synth.small(801, bits=4, K=1024, N=400, M=5)
    u = synth.small(802, bits=4, K=1024, N=400, M=5)
    lg, lu = b.QuantizedLinear(g, max_rows=5), b.QuantizedLinear(u, max_rows=5)
    xg = b.to_device(g.x)

    def run_gu(out):
        lg.plan.run_gate_up(xg, lg.codes, lg.sb, lu.codes, lu.sb, out=out)
    calls.append(("gate/up", run_gu,
                  lambda: torch.empty(5, 400, dtype=torch.bfloat16, device="cuda")))

    xn, un, wn = (b.to_device(a) for a in synth.norm_inputs(803, 4, 3840))
    res = torch.empty_like(xn)

    def run_norm(out):
        b.residual_rms_norm(xn, un, wn, 1e-5, residual=res, normalized=out)
    calls.append(("norm", run_norm, lambda: torch.empty_like(xn)))

    q, k, v = synth.attention_inputs(804, H=8, KV=2, N=700, D=128, bits=4, group_size=64)
    qd = b.to_device(q)
    kd, vd = tuple(b.to_device(a) for a in k), tuple(b.to_device(a) for a in v)
    need = b.lib().qmm_attention_workspace_bytes(8, 700, 128)
    assert need > 0  # three blocks: the merge kernel runs
    wsa = torch.empty(need, dtype=torch.uint8, device="cuda")

    def run_attn(out):
        b.decode_attention(qd, kd, vd, 4, 64, out=out, workspace=wsa)
    calls.append(("attention", run_attn, lambda: torch.empty_like(qd)))
    return calls


def test_graph_replays_match_eager():
    import torch
    calls = _work()
    ref = []
    for name, run, make in calls:
        say("eager", name)
        o = make()
        run(o)
        ref.append(o)
    torch.cuda.synchronize()

    outs = [make() for _, _, make in calls]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for (_, run, _), o in zip(calls, outs):
            run(o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for (_, run, _), o in zip(calls, outs):
            run(o)
    torch.cuda.synchronize()

    scratch = [make() for _, _, make in calls]
    for rep in range(3):
        say("replay", rep)
        for o in outs:
            o.fill_(float("nan"))
        for (_, run, _), o in zip(calls, scratch):  # eager work between replays
            run(o)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (name, _, _), o, r in zip(calls, outs, ref):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16)), \
                "%s: replay %d differs from the eager result" % (name, rep)
        for (name, _, _), o, r in zip(calls, scratch, ref):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16)), \
                "%s: eager call between replays %d differs" % (name, rep)
