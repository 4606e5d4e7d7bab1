"""Calls from several host threads at once, each on its own stream, with their
own outputs and workspaces: results equal one thread's, bit for bit (the library
keeps no per-call state outside its arguments).
"""

import threading

import pytest
import torch

from gated_delta_rule_10_amd import inputs, kda
from tests import gpu_common as gc

pytestmark = pytest.mark.gpu


def test_prefill_and_decode_from_concurrent_threads(monkeypatch):
    monkeypatch.setenv("KDA_SEG_CHUNKS", "2")
    cases = [gc.to_device(inputs.prefill_inputs(80 + i, [300, 77, 500], 4, 128, 128, "bf16", 0.1, "random"))
             for i in range(3)]
    dec = inputs.device_decode_inputs(83, 4, 8, 4, 128, 128)
    N, H, K, V = 3, 4, 128, 128

    def buffers(d):
        T = d["q"].shape[0]
        return dict(o=torch.empty((T, H, V), dtype=torch.bfloat16, device="cuda"),
                    fin=torch.empty((N, H, K, V), dtype=torch.float32, device="cuda"),
                    ws=torch.empty(kda.kda_chunk_fwd_workspace_size(N, T, H, K, V, torch.bfloat16),
                                   dtype=torch.uint8, device="cuda"))

    def work(bufs, state, outs, stream):
        for rep in range(3):
            for d, b in zip(cases, bufs):
                kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"],
                                  initial_state=d["initial_state"], final_state=b["fin"], o=b["o"],
                                  workspace=b["ws"], stream=stream)
            for s in range(dec["q"].shape[0]):
                kda.kda_decode_step(dec["q"][s], dec["k"][s], dec["v"][s], dec["log_alpha"][s], dec["beta"][s],
                                    state, o=outs[s], stream=stream)

    # one thread, for reference: the decode state after 3 x 4 steps from the same start
    ref_bufs = [buffers(d) for d in cases]
    ref_state = dec["state"].clone()
    ref_outs = torch.empty((4, 8, H, V), dtype=torch.bfloat16, device="cuda")
    work(ref_bufs, ref_state, ref_outs, torch.cuda.current_stream())
    torch.cuda.synchronize()

    nthreads = 4
    bufs = [[buffers(d) for d in cases] for _ in range(nthreads)]
    states = [dec["state"].clone() for _ in range(nthreads)]
    outs = [torch.empty((4, 8, H, V), dtype=torch.bfloat16, device="cuda") for _ in range(nthreads)]
    streams = [torch.cuda.Stream() for _ in range(nthreads)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    errors = []

    def run(i):
        try:
            with torch.cuda.stream(streams[i]):
                work(bufs[i], states[i], outs[i], streams[i])
        except Exception as e:  # reported below, on the test's thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(nthreads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(nthreads):
        for b, r in zip(bufs[i], ref_bufs):
            assert torch.equal(b["o"], r["o"]) and torch.equal(b["fin"], r["fin"]), f"thread {i}: prefill differs"
        assert torch.equal(states[i], ref_state) and torch.equal(outs[i], ref_outs), f"thread {i}: decode differs"


def test_capture_in_one_thread_while_another_runs_eagerly(monkeypatch):
    """One thread captures a multi-segment prefill into a HIP graph on its stream
    while another thread runs prefills eagerly on its own stream. The library
    shares nothing between calls, so neither the capture nor the eager calls see
    the other: the replayed graph and the eager calls give the single-thread
    results bit for bit."""
    monkeypatch.setenv("KDA_SEG_CHUNKS", "2")
    N, H, K, V = 3, 4, 128, 128
    cases = [gc.to_device(inputs.prefill_inputs(90 + i, [300, 77, 500], H, K, V, "bf16", 0.1, "random"))
             for i in range(2)]
    T = cases[0]["q"].shape[0]

    def buffers():
        return dict(o=torch.empty((T, H, V), dtype=torch.bfloat16, device="cuda"),
                    fin=torch.empty((N, H, K, V), dtype=torch.float32, device="cuda"),
                    ws=torch.empty(kda.kda_chunk_fwd_workspace_size(N, T, H, K, V, torch.bfloat16),
                                   dtype=torch.uint8, device="cuda"))

    def call(d, b, stream):
        kda.kda_chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"],
                          initial_state=d["initial_state"], final_state=b["fin"], o=b["o"], workspace=b["ws"],
                          stream=stream)

    refs = [buffers() for _ in cases]
    for d, b in zip(cases, refs):
        call(d, b, torch.cuda.current_stream())
    torch.cuda.synchronize()

    bufs = [buffers() for _ in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(streams[0]):  # warm the capture stream, as torch graph capture expects
        call(cases[0], bufs[0], streams[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    started = threading.Barrier(2)
    errors = []

    def capture():
        try:
            with torch.cuda.graph(graph, stream=streams[0], capture_error_mode="thread_local"):
                started.wait()
                call(cases[0], bufs[0], streams[0])
        except Exception as e:  # reported below, on the test's thread
            errors.append(e)

    def eager():
        try:
            with torch.cuda.stream(streams[1]):
                started.wait()
                for _ in range(4):
                    call(cases[1], bufs[1], streams[1])
            streams[1].synchronize()
        except Exception as e:
            errors.append(e)

    threads = [threading.Thread(target=capture), threading.Thread(target=eager)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for b in (bufs[0]["o"], bufs[0]["fin"]):
        b.zero_()
    for _ in range(2):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[0]["o"], refs[0]["o"]) and torch.equal(bufs[0]["fin"], refs[0]["fin"])
    assert torch.equal(bufs[1]["o"], refs[1]["o"]) and torch.equal(bufs[1]["fin"], refs[1]["fin"])
