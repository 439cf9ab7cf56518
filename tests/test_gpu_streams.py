"""Batch calls fork their row passes onto the library's side streams and join
them back.  Four host threads call spec_verify_batch at once, each on its
own stream with its own workspace (the C call releases the interpreter
lock), and one call runs on the legacy NULL stream: every result must equal
the single-threaded result bit for bit (draws are counter-based)."""

import threading

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
KEYS = ("out_tokens", "num_accepted", "p_draft", "q_draft", "beta")


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import speculative_decoding_rejection_amd as sv
    sv.load_library()
    return sv


@pytest.fixture(scope="module")
def inp():
    wl = workloads.BATCH_WORKLOADS["batch_mixed_f32_b256_g7_v151936"].scaled(B=32, V=20011)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in workloads.generate(wl).items()}
    d["mk"] = max(k for _, k, _ in wl.mix)
    return d


def call(sv, inp, stream, seed=5):
    return sv.verify_batch(inp["target_logits"], inp["draft_tokens"], inp["draft_logits"],
                           temperature=inp["temperature"], top_k=inp["top_k"], top_p=inp["top_p"],
                           max_top_k=inp["mk"], seed=seed, beta=True, stream=stream)


def test_concurrent_host_threads(sv, inp):
    ref = {k: v.clone() for k, v in call(sv, inp, None).items() if k in KEYS}
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    results = [[] for _ in streams]
    errors = []

    def worker(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(6):
                    r = call(sv, inp, streams[i])
                    results[i].append({k: v for k, v in r.items() if k in KEYS})
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(streams))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    print(f"[streams] {sum(len(r) for r in results)} calls from {len(streams)} threads", flush=True)
    for rs in results:
        for r in rs:
            for k in KEYS:
                assert torch.equal(r[k], ref[k]), k


def test_null_stream(sv, inp):
    ref = {k: v.clone() for k, v in call(sv, inp, None).items() if k in KEYS}
    torch.cuda.synchronize()
    got = call(sv, inp, 0)
    torch.cuda.synchronize()
    for k in KEYS:
        assert torch.equal(got[k], ref[k]), k


def test_stream_read_hook(sv):
    """The read-ceiling measurement hook streams a buffer and writes its sink
    only through a data-dependent test (never for an all-zero buffer)."""
    buf = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda:0")
    for _ in range(3):
        sv.sv_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0
