"""paged_attn_decode_noalloc under HIP graph capture: the call allocates
nothing and enqueues only kernel launches, so it can be recorded into a
graph.  The graph is replayed several times, with the program's own eager
work and synchronisations between the replays and new query rows copied into
the captured input buffer before each, and every replay is compared bit for
bit with an eager call of paged_attn_decode on the same inputs."""
import sys

import numpy as np
import pytest
import torch

import paged_gqa_attention_02_amd as pa
from paged_gqa_attention_02_amd import inputs as I
from tests._gpu import DEV

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_decode_replays_from_a_graph():
    rng = np.random.default_rng(71)
    lens = rng.integers(1, 2000, size=12)
    case = I.make_decode("graph", lens, 32, 8, 128, 16, 71, lens_rng=rng)
    t = I.decode_tensors(case, DEV)
    pl = pa.decode_plan(t["q"], t["k_pool"], t["block_table"], case.max_kv_len)
    say(f"[graph] {pl.describe()}")
    q = t["q"].clone()
    out = torch.empty_like(q)
    args = lambda qq, o: (pl, qq, t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"],
                          case.scale)
    # first call outside the capture (looks the scratch array up once)
    pa.decode_noalloc(*args(q, out), out=out)
    torch.cuda.synchronize()

    # (the host-side contract check copies metadata to the host: not while
    # capturing; it ran on the call above)
    checks = pa.set_input_checks(False)
    try:
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            pa.decode_noalloc(*args(q, out), out=out)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
    finally:
        pa.set_input_checks(checks)

    for rep in range(4):
        fresh = I._dev(I.bf16_bits(rng.standard_normal(q.shape, dtype=np.float32)), DEV,
                       torch.bfloat16)
        q.copy_(fresh)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = pa.decode(*args(fresh, None))
        # eager work between replays
        _ = (fresh.float() * 2).sum().item()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {rep}"
        say(f"[graph] replay {rep} matches")
