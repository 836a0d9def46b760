"""Stream capture: the training step (fa_fwd + fa_bwd) and decode (fa_decode and
fa_decode_noalloc) captured into a HIP graph and replayed.  Between replays the test
overwrites the inputs with other values, clobbers the outputs and the workspace (so a
replay that skipped staging its work plan, or any kernel, shows), and runs unrelated
eager work with synchronisations; every replay must reproduce the eager call on the
same inputs bit for bit (the deterministic passes), or within rounding (atomic dQ)."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import workloads as wl
from harness import config_of, device_inputs, say

pytestmark = pytest.mark.gpu


def _capture(fn):
    """Capture fn() into a graph after one warm-up call on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _unrelated_eager_work(dev):
    a = torch.randn(512, 512, device=dev)
    (a @ a).sum().item()
    torch.cuda.synchronize()


def _other_values(tensors, seed):
    gen = torch.Generator().manual_seed(seed)
    return {k: torch.randn(t.shape, generator=gen).to(t.dtype).to(t.device) for k, t in tensors.items()}


def _replay_and_check(g, dynamic, sets, outputs, workspaces, dev, exact, tol=0.0):
    """sets: [(input values, eager outputs)]; replays the graph once per set."""
    for n, (values, want) in enumerate(sets):
        for k, t in values.items():
            dynamic[k].copy_(t)
        for t in outputs:
            t.fill_(float("nan"))
        for w in workspaces:
            w.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        _unrelated_eager_work(dev)
        for i, (got, ref) in enumerate(zip(outputs, want)):
            if exact:
                assert torch.equal(got, ref), f"replay {n}, output {i} differs from the eager call"
            else:
                r = ref.double()
                err = float((got.double() - r).norm() / r.norm())
                assert err <= tol, f"replay {n}, output {i}: relL2 {err:.2e}"
        say(f"replay {n} matches the eager call")


@pytest.mark.parametrize("variant", ["deterministic", "atomic_dq", "bnsd"])
def test_training_step_graph_replays_match_eager(variant):
    dev = torch.device("cuda")
    if variant == "bnsd":
        # fixed-length layout: gathers into the workspace and scatters back inside the graph
        case = wl.make_case("graph_bnsd", [256, 256, 256], head_num=4, kv_heads=2, head_dim=128,
                            dtype=torch.bfloat16, sparse_mode=3, sink=True, seed=43)
    else:
        case = wl.make_case("graph_step", [300, 77, 513, 1000], head_num=8, kv_heads=2, head_dim=128,
                            dtype=torch.bfloat16, sparse_mode=3, keep_prob=0.9,
                            alibi=variant == "deterministic", sink=True, seed=41)
    x = device_inputs(case)
    det = variant != "atomic_dq"
    cfg = config_of(case, det)
    if variant == "bnsd":
        b, s = case.batch, int(case.lens_q[0])
        to_bnsd = lambda t: t.reshape(b, s, t.shape[1], t.shape[2]).permute(0, 2, 1, 3).contiguous()
        for k in ("q", "k", "v", "dy"):
            x[k] = to_bnsd(x[k])
        cfg = fa.Config(case.cu_seqlens_q, case.cu_seqlens_kv, case.head_num, case.kv_heads, case.head_dim,
                        case.dtype, case.scale, case.keep_prob, case.sparse_mode, case.pre_tokens,
                        case.next_tokens, True, layout="BNSD")
    tq, nq = int(case.cu_seqlens_q[-1]), case.head_num
    out = torch.empty_like(x["q"])
    m = torch.empty((tq, nq), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
    dsink = torch.empty((nq,), dtype=torch.float32, device=dev)
    ws_f = torch.empty(fa.fa_fwd_workspace_size(cfg), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(fa.fa_bwd_workspace_size(cfg), dtype=torch.uint8, device=dev)
    outputs = (out, m, l, dq, dk, dv, dsink)

    def step():
        fa.fa_fwd(cfg, x["q"], x["k"], x["v"], x["drop"], x["slopes"], x["sink"], out, m, l, workspace=ws_f)
        fa.fa_bwd(cfg, x["q"], x["k"], x["v"], x["dy"], out, m, l, x["drop"], x["slopes"], x["sink"], dq, dk, dv,
                  dsink, workspace=ws_b)

    dyn = {k: x[k] for k in ("q", "k", "v", "dy")}
    first = {k: t.clone() for k, t in dyn.items()}
    second = _other_values(dyn, 7)
    sets = []
    for values in (first, second):
        for k, t in values.items():
            dyn[k].copy_(t)
        step()
        torch.cuda.synchronize()
        sets.append((values, [t.clone() for t in outputs]))
    say(f"training step ({variant}): capture")
    g = _capture(step)
    _replay_and_check(g, dyn, sets + [sets[0]], outputs, (ws_f, ws_b), dev, exact=det, tol=1e-2)


def test_decode_graph_replays_match_eager():
    dev = torch.device("cuda")
    # a 1000-key sequence is split over two work items, so the staged plan holds partial slots
    dc = wl.make_decode_case("graph decode", [5, 300, 0, 1000], 1024, num_heads=8, num_kv_heads=2, head_dim=128,
                             dtype=torch.bfloat16, layout="BSND", seed=42)
    dcfg = fa.DecodeConfig(dc.batch, dc.max_seq_len, dc.num_heads, dc.num_kv_heads, dc.head_dim, dc.dtype,
                           dc.scale, dc.layout, dc.lens)
    q = dc.q.to(dev)
    k, v = dc.padded_cache("k", dev), dc.padded_cache("v", dev)
    out_ws, out_na = torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_decode_workspace_size(dcfg), dtype=torch.uint8, device=dev)

    def step():
        fa.fa_decode(dcfg, q, k, v, out_ws, workspace=ws)
        fa.fa_decode_noalloc(dcfg, q, k, v, out_na)

    dyn = {"q": q, "k": k, "v": v}
    first = {kk: t.clone() for kk, t in dyn.items()}
    second = _other_values(dyn, 8)
    sets = []
    for values in (first, second):
        for kk, t in values.items():
            dyn[kk].copy_(t)
        step()
        torch.cuda.synchronize()
        assert torch.equal(out_ws, out_na)
        sets.append((values, [out_ws.clone(), out_na.clone()]))
    say("decode: capture")
    g = _capture(step)
    _replay_and_check(g, dyn, sets + [sets[0]], (out_ws, out_na), (ws,), dev, exact=True)
