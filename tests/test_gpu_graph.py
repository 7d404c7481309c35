"""The entry points on several streams and under HIP graph capture.  Calls on two
streams at once give what each gives alone.  Each captured graph
(torch.cuda.CUDAGraph on the capturing stream) is replayed several times, with
eager work of the program between the replays (other calls of the same entry
point, which reuse the library's scratch array, torch kernels and device
synchronisations), and every replay must give exactly the eager result on the
same inputs.  The library records kernel launches only: no memset, copy or
allocation."""
import pytest
import torch

from sub_quadratic_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_sequence_amd import gla

    gla.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def _capture(fn):
    """fn() run once more on a side stream (lazy set-up), then captured."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _eager_noise(dev, gla, other):
    """Unrelated eager work between replays: torch kernels, and a call of the
    same entry point on other inputs (which overwrites the library's scratch)."""
    a = torch.randn(512, 512, device=dev)
    (a @ a).sum().item()
    if other is not None:
        other()
    torch.cuda.synchronize()


def test_noalloc_split_forward_replays(dev):
    from sub_quadratic_sequence_amd import gla

    w = I.ChunkWorkload("graph_split", B=1, H=4, T=2048, dk=128, dv=128, dtype="bf16", seed=61)
    say("graph of gla_chunk_fwd_noalloc (sequence split): B=1 H=4 T=2048 d=128, initial state")
    d = I.chunk_inputs(w, s0=True)
    q, k, v, g, s0 = (d[n].to(dev) for n in ("q", "k", "v", "g", "s0"))
    assert gla.workspace_size(q, v) > 0   # this shape splits, so the scratch array is used
    o_e, sf_e = gla.gla_chunk_fwd_noalloc(q, k, v, g, initial_state=s0, output_final_state=True)
    w2 = I.ChunkWorkload("graph_split_other", B=1, H=2, T=3000, dk=128, dv=128, dtype="bf16", seed=62)
    d2 = I.chunk_inputs(w2, s0=True)
    q2, k2, v2, g2, s02 = (d2[n].to(dev) for n in ("q", "k", "v", "g", "s0"))
    other = lambda: gla.gla_chunk_fwd_noalloc(q2, k2, v2, g2, initial_state=s02, output_final_state=True)
    o_g = torch.empty_like(o_e)
    sf_g = torch.empty_like(sf_e)
    graph = _capture(lambda: gla.gla_chunk_fwd_noalloc(q, k, v, g, initial_state=s0, out=o_g,
                                                        final_state=sf_g))
    for rep in range(REPLAYS):
        o_g.fill_(float("nan"))
        sf_g.fill_(float("nan"))
        _eager_noise(dev, gla, other)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), rep
        assert torch.equal(sf_g, sf_e), rep


@pytest.mark.parametrize("dv_slice", [64, 128])
def test_sliced_forward_replays(dev, dv_slice):
    from sub_quadratic_sequence_amd import gla

    w = I.ChunkWorkload("graph_fwd", B=2, H=3, T=190, dk=128, dv=256, dtype="bf16", seed=63)
    say(f"graph of gla_chunk_fwd_sliced (dv_slice={dv_slice}): B=2 H=3 T=190 dk=128 dv=256")
    d = I.chunk_inputs(w, s0=True, gate="strong")
    q, k, v, g, s0 = (d[n].to(dev) for n in ("q", "k", "v", "g", "s0"))
    o_e, sf_e = gla.gla_chunk_fwd(q, k, v, g, initial_state=s0, output_final_state=True,
                                  dv_slice=dv_slice)
    o_g = torch.empty_like(o_e)
    sf_g = torch.empty_like(sf_e)
    graph = _capture(lambda: gla.gla_chunk_fwd(q, k, v, g, initial_state=s0, out=o_g,
                                               final_state=sf_g, dv_slice=dv_slice))
    for rep in range(REPLAYS):
        o_g.zero_()
        sf_g.zero_()
        _eager_noise(dev, gla, None)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(sf_g, sf_e), rep


def test_decode_step_replays_advance_the_state(dev):
    """One captured decode step updates the state in place: each replay is the
    next step, equal to the eager steps on a copy of the same state."""
    from sub_quadratic_sequence_amd import gla

    wd = I.DecodeWorkload("graph_decode", N=8, H=2, dk=128, dv=128, steps=1, seed=64, dtype="bf16")
    say("graph of gla_recurrent_step: N=8 H=2 d=128, state updated in place")
    d = I.decode_inputs(wd)
    q, k, v, g = (d[n][0].to(dev) for n in "qkvg")
    st_g = d["s0"].to(dev).clone()
    st_e = st_g.clone()
    o_g = torch.empty(8, 2, 128, dtype=torch.bfloat16, device=dev)
    graph = _capture(lambda: gla.gla_recurrent_step(q, k, v, g, st_g, out=o_g))
    # the warm-up and the capture-time run each advanced st_g by one step (the
    # capture itself launches nothing); bring the eager copy level with it
    st_e.copy_(st_g)
    for rep in range(REPLAYS):
        _eager_noise(dev, gla, None)
        o_e = gla.gla_recurrent_step(q, k, v, g, st_e)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(st_g, st_e), rep


def test_split_backward_replays(dev):
    from sub_quadratic_sequence_amd import gla

    w = I.ChunkWorkload("graph_bwd", B=1, H=2, T=2048, dk=128, dv=128, dtype="bf16", seed=65,
                        k_scaled=True, s0=True)
    say("graph of gla_chunk_bwd (sequence split): B=1 H=2 T=2048 d=128, initial state, dS_T")
    d = I.chunk_inputs(w)
    d.update(I.upstream_grads(w, d, final=True))
    q, k, v, g, do = (d[n].to(dev) for n in ("q", "k", "v", "g", "do"))
    s0, dsT = d["s0"].to(dev), d["dsT"].to(dev)
    need = gla.bwd_workspace_size(q, v)
    ws = torch.zeros(need + 256, dtype=torch.uint8, device=dev)
    ref = gla.gla_chunk_bwd(q, k, v, g, do, initial_state=s0, d_final_state=dsT, workspace=ws)
    outs = tuple(torch.empty_like(x) for x in ref[:4])
    res = {}

    def call():
        res["r"] = gla.gla_chunk_bwd(q, k, v, g, do, initial_state=s0, d_final_state=dsT,
                                     workspace=ws, out=outs)

    graph = _capture(call)
    for rep in range(REPLAYS):
        for x in outs:
            x.zero_()
        ws.fill_(0xAB)   # the workspace holds nothing the next replay relies on
        _eager_noise(dev, gla, None)
        graph.replay()
        torch.cuda.synchronize()
        got = res["r"]
        for name, a, b in zip(("dq", "dk", "dv", "dg", "ds0"), got, ref):
            assert torch.equal(a, b), (rep, name)


def test_calls_on_two_streams_are_independent(dev):
    """Forward, backward and decode calls on two streams at once (different inputs,
    no ordering between the streams) give exactly what each gives alone: the
    entry points other than the scratch-array one share no device state."""
    from sub_quadratic_sequence_amd import gla

    say("two streams: forward (both slice widths), backward and decode, interleaved")

    def make(seed):
        w = I.ChunkWorkload("streams", B=2, H=4, T=700, dk=128, dv=128, dtype="bf16", seed=seed,
                            k_scaled=True, s0=True)
        d = I.chunk_inputs(w)
        d.update(I.upstream_grads(w, d, final=True))
        t = {n: d[n].to(dev) for n in ("q", "k", "v", "g", "do", "s0", "dsT")}
        wd = I.DecodeWorkload("streams_dec", N=16, H=2, dk=128, dv=128, steps=1, seed=seed, dtype="bf16")
        dd = I.decode_inputs(wd)
        t.update({"dq_" + n: dd[n][0].to(dev) for n in "qkvg"})
        t["state"] = dd["s0"].to(dev)
        return t

    def run(t, state):
        f1 = gla.gla_chunk_fwd(t["q"], t["k"], t["v"], t["g"], initial_state=t["s0"],
                               output_final_state=True, dv_slice=64)
        f2 = gla.gla_chunk_fwd(t["q"], t["k"], t["v"], t["g"], initial_state=t["s0"],
                               output_final_state=True, dv_slice=128)
        b = gla.gla_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["do"], initial_state=t["s0"],
                              d_final_state=t["dsT"])
        o = gla.gla_recurrent_step(t["dq_q"], t["dq_k"], t["dq_v"], t["dq_g"], state)
        return [*f1, *f2, *b, o, state]

    ta, tb = make(71), make(72)
    sa, sb = ta["state"].clone(), tb["state"].clone()
    ref_a, ref_b = run(ta, sa), run(tb, sb)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    sa2, sb2 = ta["state"].clone(), tb["state"].clone()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        got_a = run(ta, sa2)
    with torch.cuda.stream(s2):
        got_b = run(tb, sb2)
    torch.cuda.synchronize()
    for ref, got in ((ref_a, got_a), (ref_b, got_b)):
        for i, (x, y) in enumerate(zip(ref, got)):
            assert (x is None and y is None) or torch.equal(x, y), i
