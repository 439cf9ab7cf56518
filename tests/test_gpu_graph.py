"""HIP-graph capture of the verifier.  A per-request batch call (its row
passes fork onto the library's side streams and join back to the captured
stream) and a single-setting call are captured on a torch stream and
replayed several times, with other eager calls and synchronisations between
the replays.  The draws are counter-based (seed, request, position, token),
so every replay must reproduce the eager result bit for bit."""

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
