"""gqa_decode_noalloc (no workspace, no allocation in the library) against
gqa_decode on the same inputs, through the C ABI: bit-identical outputs on
calls in a row that share the fixed per-GPU scratch area, the second call
smaller than the first."""

import sys

import pytest
import torch

import grouped_query_attention_fwd_amd as gqa
import workloads
from tests.parity import TOL, compare, oracle_out

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(seed, B, H, H_kv, M, D, dtype, mask_kind=None):
    q, k, v, mask = workloads.random_case(seed, B, H, H_kv, 1, M, D, dtype, mask_kind)
    if mask is not None:
        mask = mask[:, :1, :].contiguous()
    return q, k, v, mask


# (seed, B, H, H_kv, M, D, dtype, mask) per call; each sequence runs in a row
# in one process, so later calls find the scratch left by earlier ones
SEQUENCES = [
    # the Mistral-7B-shaped decode (two key splits per unit), then a smaller one
    [(1, 16, 32, 8, 4096, 128, torch.bfloat16, None), (2, 4, 32, 8, 1000, 128, torch.bfloat16, None)],
    # many splits of one unit (65536 keys), then a masked fp32 call, then g = 64
    # through the large-group path, then a small fp16 call
    [(3, 1, 16, 4, 65536, 128, torch.bfloat16, None), (4, 2, 8, 2, 3000, 64, torch.float32, "padding"),
     (5, 2, 64, 1, 3000, 128, torch.bfloat16, None), (6, 1, 8, 2, 300, 128, torch.float16, None)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_decode(seq):
    for case in SEQUENCES[seq]:
        seed, B, H, H_kv, M, D, dtype, mk = case
        say(f"noalloc case seed={seed} B={B} H={H} H_kv={H_kv} M={M} D={D} {dtype} mask={mk}")
        q, k, v, mask = _inputs(seed, B, H, H_kv, M, D, dtype, mk)
        dev = [None if t is None else t.cuda() for t in (q, k, v, mask)]
        want = gqa.decode(*dev)
        got = gqa.decode_noalloc(*dev)
        again = gqa.decode_noalloc(*dev)
        torch.cuda.synchronize()
        assert torch.equal(got, want), case
        assert torch.equal(again, want), case
        compare(got, oracle_out(q, k, v, mask), TOL[dtype], f"noalloc seed={seed}")


def test_noalloc_rejects_too_large():
    """A problem whose workspace exceeds the scratch area is rejected before
    any work is enqueued (one KV head, 256 query heads, 16384 keys of D 256:
    the large-group path's partials need about 68 MB)."""
    B, H, H_kv, M, D = 1, 256, 1, 16384, 256
    assert gqa.decode_workspace_size(B, H, H_kv, M, D) > gqa.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, H, 1, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, H_kv, M, D, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="status 10"):
        gqa.decode_noalloc(q, k, k.clone())
