"""Every entry point captured in a HIP graph and replayed: each replay, with eager
work and synchronisations between the replays, must reproduce the eager result
bitwise.  Covers the calls with device-side state that must be back at rest after
each call (the arrival counters of the sliced streaming launches and of the tiled
launches' split last round) and the small reduction kernels a decode step captures."""
import pytest
import torch

import tensor_mlp_shard_amd as tpm
from tensor_mlp_shard_amd import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
REPLAYS = 4


def say(*a):
    print(*a, flush=True)


def check_graph(name, run, outs):
    """run() writes `outs` on torch's current stream."""
    say("graph replay:", name)
    run()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(REPLAYS):
        for o in outs:
            if o.dtype.is_floating_point:
                o.fill_(float("nan"))
            else:
                o.fill_(0x55)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), (name, i)
        run()  # eager work between replays
        torch.cuda.synchronize()
    del g


def test_reduction_kernels_in_graphs():
    g = torch.Generator().manual_seed(5)
    parts = [torch.randn(32, 8192, generator=g).to(DEV) for _ in range(8)]
    z = torch.empty(32, 8192, device=DEV)
    check_graph("tp_partials_reduce", lambda: tpm.tp_partials_reduce(parts, z), [z])

    res = torch.randn(32, 8192, generator=g).to(torch.bfloat16).to(DEV)
    gamma = (1.0 + 0.1 * torch.randn(8192, generator=g)).to(torch.bfloat16).to(DEV)
    y = torch.empty(32, 8192, dtype=torch.bfloat16, device=DEV)
    ro = torch.empty_like(res)
    check_graph("tp_partials_reduce_add_rmsnorm",
                lambda: tpm.tp_partials_reduce_add_rmsnorm(parts, res, gamma, 1e-5, y, ro), [y, ro])

    qs = [torch.empty(32, 8192, dtype=torch.uint8, device=DEV) for _ in parts]
    ss = [torch.empty(32, device=DEV) for _ in parts]
    z8 = torch.empty(32, 8192, device=DEV)

    def fp8():
        for p, q, s in zip(parts, qs, ss):
            tpm.tp_partials_quantize_fp8(p, q, s)
        tpm.tp_partials_reduce_fp8(qs, ss, z8)
    check_graph("fp8 quantize + reduce", fp8, qs + ss + [z8])

    vals, maxs, sums = synth.attn_partials(2048, 128, 8)
    vals = [v.to(DEV) for v in vals]
    maxs = [m.to(DEV) for m in maxs]
    sums = [s.to(DEV) for s in sums]
    out = torch.empty(2048, 128, device=DEV)
    mo = torch.empty(2048, device=DEV)
    eo = torch.empty(2048, device=DEV)
    check_graph("tp_attn_partials_merge",
                lambda: tpm.tp_attn_partials_merge(vals, maxs, sums, out, mo, eo), [out, mo, eo])


def test_sliced_streaming_launches_in_graphs():
    """Narrow shards slice the contraction; the last slice to arrive resets the unit's
    arrival counter, which every replay relies on."""
    spec = synth.ModelSpec(d_model=8192, ffn=2048, pieces=8)
    a, b = spec.shard(5, 8)  # per-rank F = 256: 16 gate/up column blocks
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=32, path="stream")
    x = synth.tokens(32).to(DEV)
    p = torch.empty(32, 8192, device=DEV)
    try:
        check_graph("sliced MLP shard", lambda: sh.forward(x, out=p), [p])
    finally:
        sh.close()
    wqkv, _ = synth.AttentionSpec().shard(2, 8)  # [8192 x 1280]: 40 column blocks, sliced
    pr = tpm.Projection(wqkv.to(DEV), max_tokens=32, out_dtype=torch.bfloat16)
    yq = torch.empty(32, 1280, dtype=torch.bfloat16, device=DEV)
    try:
        check_graph("sliced QKV projection", lambda: pr.forward(x, out=yq), [yq])
    finally:
        pr.close()


def test_tiled_split_round_and_grouped_experts_in_graphs():
    """The tiled path's split last round (contraction halves meeting through an
    arrival counter) and the grouped expert launches (device-side counts)."""
    spec = synth.ModelSpec(d_model=1024, ffn=4096, pieces=8)
    a, b = spec.shard(0, 2)  # F = 2048: 32 gate/up tiles at M = 512, all split
    sh = tpm.Shard(a.to(DEV), b.to(DEV), "silu_gate", max_tokens=512, path="tiled")
    x = synth.tokens(512, 1024).to(DEV)
    p = torch.empty(512, 1024, device=DEV)
    try:
        check_graph("tiled shard with split round", lambda: sh.forward(x, out=p), [p])
    finally:
        sh.close()
    es = synth.ExpertSpec(d_model=1024, ffn_expert=512, n_experts=4)
    w1, w2 = es.weights()
    counts = torch.tensor([100, 0, 257, 43], dtype=torch.int32, device=DEV)
    xe = synth.tokens(400, 1024).to(DEV)
    ye = torch.empty(400, 1024, device=DEV)
    for path in ("stream", "tiled"):  # both grouped kernels (AUTO streams at this size)
        ge = tpm.GroupedExperts(w1.to(DEV), w2.to(DEV), max_tokens=400, path=path)
        try:
            check_graph("grouped experts, " + path, lambda: ge.forward(xe, counts, out=ye), [ye])
        finally:
            ge.close()
