"""HIP-graph capture of the verifier.  A per-request batch call (its row
passes fork onto the library's side streams and join back to the captured
stream) and a single-setting call are captured on a torch stream and
replayed several times, with other eager calls and synchronisations between
the replays.  The draws are counter-based (seed, request, position, token),
so every replay must reproduce the eager result bit for bit."""

import os

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_rejection_amd as sv
    sv.load_library()
    return sv


def _capture_and_replay(call, keys):
    eager = {k: v.clone() for k, v in call(42).items() if k in keys}
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(42)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        res = call(42)
    for rep in range(3):
        other = call(1000 + rep)  # eager work between the replays
        torch.cuda.synchronize()
        for k in keys:
            res[k].fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {rep}", flush=True)
        for k in keys:
            assert torch.equal(res[k], eager[k]), (rep, k)
        assert other["out_tokens"].shape == res["out_tokens"].shape


def test_batch_call_in_graph(sv):
    wl = workloads.BATCH_WORKLOADS["batch_mixed_f32_b256_g7_v151936"].scaled(B=24, V=20011)
    inp = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in workloads.generate(wl).items()}
    mk = max(k for _, k, _ in wl.mix)
    ws = {}

    def call(seed):
        r = sv.verify_batch(inp["target_logits"], inp["draft_tokens"], inp["draft_logits"],
                            temperature=inp["temperature"], top_k=inp["top_k"], top_p=inp["top_p"], max_top_k=mk,
                            seed=seed, beta=True, workspace=ws.get(seed == 42))
        ws.setdefault(seed == 42, r["workspace"])
        return r

    print(f"[graph] batch B={wl.B} V={wl.V} kinds={sorted(set(inp['top_k'].tolist()))}", flush=True)
    _capture_and_replay(call, ("out_tokens", "num_accepted", "p_draft", "q_draft", "beta"))


def test_single_setting_call_in_graph(sv):
    wl = workloads.WORKLOADS["prob_topk64_bf16_b1024_g8_v256000"].scaled(B=16, V=30001)
    inp = workloads.generate(wl)
    lt, x, ld = inp["target_logits"].to(DEV), inp["draft_tokens"].to(DEV), inp["draft_logits"].to(DEV)
    ws = {}

    def call(seed):
        r = sv.verify("prob", lt, x, ld, temperature=wl.temperature, top_k=wl.top_k, seed=seed,
                      workspace=ws.get(seed == 42))
        ws.setdefault(seed == 42, r["workspace"])
        return r

    print(f"[graph] prob B={wl.B} V={wl.V} top_k={wl.top_k}", flush=True)
    _capture_and_replay(call, ("out_tokens", "num_accepted", "p_draft", "q_draft"))


def test_match_tree_call_in_graph_shared_workspace(sv):
    """A sampler-match tree batch (per-row races, the tree walk) captured and
    replayed, with the eager calls between the replays made on the captured
    call's own workspace: a replay depends on nothing that earlier calls
    left there."""
    wl = workloads.MATCH_WORKLOADS["match_tree_bf16_b256_g7_v151936"].scaled(B=16, V=9001, data_seed=4)
    inp = workloads.generate(wl)
    lt, x = inp["target_logits"].to(DEV), inp["draft_tokens"].to(DEV)
    t, k, p = inp["temperature"].to(DEV), inp["top_k"].to(DEV), inp["top_p"].to(DEV)
    par = inp["parents"].to(DEV).contiguous()
    ws = {}

    def call(seed):
        r = sv.verify_batch(lt, x, None, draft_kind=sv.SV_DRAFT_MATCH, parents=par, temperature=t, top_k=k,
                            top_p=p, max_top_k=int(inp["top_k"].max()), seed=seed, workspace=ws.get(0))
        ws.setdefault(0, r["workspace"])
        return r

    print(f"[graph] match tree B={wl.B} V={wl.V}", flush=True)
    _capture_and_replay(call, ("out_tokens", "num_accepted", "p_draft", "q_draft", "path_nodes"))


def test_first_batch_call_under_capture():
    """A process whose first batch call is captured: the library does not
    create its side streams during the capture (the row passes then run on
    the captured stream), the capture succeeds, and its replays equal an
    eager call made afterwards (which creates the streams).  Runs in a child
    process so that no earlier call has created the streams."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = r'''
import sys, torch
sys.path.insert(0, sys.argv[1])
import speculative_decoding_rejection_amd as sv, workloads
sv.load_library()
dev = torch.device("cuda:0")
wl = workloads.BATCH_WORKLOADS["batch_mixed_f32_b256_g7_v151936"].scaled(B=16, V=20011)
inp = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in workloads.generate(wl).items()}
mk = max(k for _, k, _ in wl.mix)
nbytes = sv.sv_workspace_bytes_batch(sv.make_params(16, wl.G, wl.V, torch.float32, 1.0, 0, 3),
                                     sv.make_sampling(inp["temperature"], inp["top_k"], inp["top_p"], mk))
ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
def call(w):
    return sv.verify_batch(inp["target_logits"], inp["draft_tokens"], inp["draft_logits"],
                           temperature=inp["temperature"], top_k=inp["top_k"], top_p=inp["top_p"],
                           max_top_k=mk, seed=3, beta=True, workspace=w)
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):
    res = call(ws)
eager = call(torch.empty_like(ws))
torch.cuda.synchronize()
for rep in range(3):
    g.replay()
    torch.cuda.synchronize()
    for k in ("out_tokens", "num_accepted", "p_draft", "q_draft", "beta"):
        assert torch.equal(res[k], eager[k]), (rep, k)
print("first-capture ok", flush=True)
'''
    r = subprocess.run([sys.executable, "-c", code, root], capture_output=True, text=True, timeout=240)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "first-capture ok" in r.stdout
