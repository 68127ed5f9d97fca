"""HIP-graph replay of a whole step equals the eager step, bit for bit.

bench.py times the calls as replays of captured HIP graphs; this checks that
a captured step (rope + cache write, prefill, decode) gives exactly the eager
results on every replay, with eager work and synchronizations in between.
"""
import numpy as np
import pytest
import torch

from paged_gqa_attention_neox_amd import runner
from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_bitwise():
    require_gpu()
    b = W.small_case(310, "bf16", 28, 4, 128, context_lens=[300, 77, 1500, 2049],
                     query_lens=[300, 20, 1, 1], num_prefill=2, keep_logical=False)
    say("graph: eager step")
    eager = runner.DeviceStep(b)
    eager.step()
    ref = eager.results()

    dev = runner.DeviceStep(b)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dev.step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dev.step()
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"graph: replay {rep}")
        dev.out.fill_(float("nan"))           # eager work between replays
        dev.q_out.zero_()
        torch.cuda.synchronize()
        g.replay()
        got = dev.results()
        for key in ("q_out", "k_cache", "v_cache", "out"):
            assert np.array_equal(got[key].view(np.uint16), ref[key].view(np.uint16)), (rep, key)


def test_overlapped_step_matches_serial_bitwise():
    """The mixed step with prefill and decode on two streams (forked after the
    cache write, joined after both) gives the serial step's results bit for
    bit, eagerly and as a captured graph replayed several times."""
    require_gpu()
    b = W.mixed_tp2()
    say("overlap: serial step")
    ser = runner.DeviceStep(b)
    ser.step()
    ref = ser.results()
    dev = runner.DeviceStep(b)
    say("overlap: eager overlapped step")
    dev.step_overlapped()
    got = dev.results()
    for key in ("q_out", "k_cache", "v_cache", "out"):
        assert np.array_equal(got[key].view(np.uint16), ref[key].view(np.uint16)), key
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dev.step_overlapped()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dev.step_overlapped()
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"overlap: graph replay {rep}")
        dev.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        got = dev.results()
        assert np.array_equal(got["out"].view(np.uint16), ref["out"].view(np.uint16)), rep
