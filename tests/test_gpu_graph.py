"""HIP-graph capture of the prepared calls: every replay, with eager work and
synchronisations in between, must give the eager result bit for bit (the
kernels record no memset: the decode workspace is zeroed once, at
allocation, and every call, replays included, leaves its counter area
zero)."""

import sys

import pytest
import torch

import grouped_query_attention_fwd_amd as gqa
import workloads
from tests.parity import to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def replay_matches(op, reps=4):
    torch.cuda.synchronize()
    eager = op().clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        op(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            op(side)
    torch.cuda.synchronize()
    for r in range(reps):
        op.out.fill_(float("nan"))                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(op.out, eager), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("B,H,H_kv,M", [
    (4, 32, 8, 4096),   # key splits merged by the last split
    (2, 64, 1, 3000),   # 64 heads per KV head: the splits merge in the prefill kernel
])
def test_graph_decode(B, H, H_kv, M):
    say(f"graph decode B={B} H={H} H_kv={H_kv} M={M}")
    q, k, v, _ = workloads.random_case(60, B, H, H_kv, 1, M, 128, torch.bfloat16)
    ws = torch.zeros(gqa.decode_workspace_size(B, H, H_kv, M, 128), dtype=torch.uint8,
                     device="cuda")
    replay_matches(gqa.decode_op(*to_dev(q, k, v), workspace=ws))
    assert ws[:gqa.DECODE_COUNTER_BYTES].count_nonzero().item() == 0


def test_graph_decode_paged():
    say("graph paged decode")
    q, kp, vp, table, lens = workloads.random_paged_case(61, 4, 32, 8, 128, 16, 3000,
                                                         torch.bfloat16)
    dev = [t.cuda() for t in (q, kp, vp, table, lens)]
    need = gqa.decode_paged_workspace_size(4, 32, 8, table.shape[1], 16, 128)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    replay_matches(gqa.decode_paged_op(*dev, workspace=ws))
    assert ws[:gqa.DECODE_COUNTER_BYTES].count_nonzero().item() == 0


def test_graph_prefill_and_band():
    say("graph prefill")
    q, k, v, _ = workloads.random_case(62, 1, 8, 2, 300, 300, 128, torch.bfloat16)
    qd, kd, vd = to_dev(q, k, v)
    replay_matches(gqa.prefill_op(qd, kd, vd, causal=True))
    replay_matches(gqa.prefill_band_op(qd, kd, vd, None, 0, 63, 0))
