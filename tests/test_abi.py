"""C ABI on the CPU: the library loads, exports every entry point the header
declares (and nothing else), and rejects every invalid call before any HIP
call is made (so these run without a GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

import grouped_query_attention_fwd_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")

OK, NULL, SHAPE, GROUP, DTYPE, ALIGN, UNSUP, WS, HIP, ALIAS, SCRATCH = range(11)
F32, BF16, F16 = 0, 1, 2

# fake, 16-byte aligned, non-overlapping "device" addresses: never dereferenced
# because every call below fails validation first
Q, K, V, O, W, MK, BT, KL = (0x10000000 * (i + 1) for i in range(8))


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(gqa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    # GQA_TEST_LIBRARY: run these checks against another build of the same
    # library (the host-sanitized one, see test_sanitize_cpu.py)
    return gqa.load_library(os.environ.get("GQA_TEST_LIBRARY") or None)


def test_exports_match_header(lib):
    names = declared_functions()
    assert names == ["gqa_decode", "gqa_decode_noalloc", "gqa_decode_paged",
                     "gqa_decode_paged_workspace_size",
                     "gqa_decode_workspace_size", "gqa_prefill", "gqa_prefill_band",
                     "gqa_status_string"]
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", gqa.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines()
                      if " T " in line)
    assert exported == names


def test_status_strings(lib):
    for code in range(11):
        s = gqa.status_string(code)
        assert s and s != "unknown status"
    assert gqa.status_string(123) == "unknown status"


def dec(lib, q=Q, k=K, v=V, mask=None, out=O, B=2, H=8, H_kv=2, M=300, D=128,
        tin=BF16, tout=BF16, ws=W, wsb=1 << 30):
    return lib.gqa_decode(q, k, v, mask, out, B, H, H_kv, M, D, tin, tout, ws, wsb, None)


def pre(lib, q=Q, k=K, v=V, mask=None, causal=0, out=O, B=2, H=8, H_kv=2, N=7, M=9,
        D=128, tin=BF16, tout=BF16):
    return lib.gqa_prefill(q, k, v, mask, causal, out, B, H, H_kv, N, M, D, tin, tout, None)


def band(lib, q=Q, k=K, v=V, mask=None, out=O, B=2, H=8, H_kv=2, N=7, M=9, D=128,
         tin=BF16, tout=BF16, q_offset=2, wl=3, wr=0):
    return lib.gqa_prefill_band(q, k, v, mask, out, B, H, H_kv, N, M, D, q_offset, wl, wr,
                                tin, tout, None)


def paged(lib, q=Q, k=K, v=V, bt=BT, kl=KL, out=O, B=2, H=8, H_kv=2, M=None, D=128,
          tin=BF16, tout=BF16, ws=W, wsb=1 << 30, max_blocks=None, block_size=32,
          num_blocks=64):
    # M, when given, is split into max_blocks blocks of block_size keys
    if max_blocks is None:
        max_blocks = 10 if M is None else (M if M < 1 else max(1, M // block_size))
    return lib.gqa_decode_paged(q, k, v, bt, kl, out, B, H, H_kv, max_blocks, block_size,
                                num_blocks, D, tin, tout, ws, wsb, None)


@pytest.mark.parametrize("fn", [dec, pre, paged, band])
def test_rejections_common(lib, fn):
    assert fn(lib, q=None) == NULL
    assert fn(lib, k=None) == NULL
    assert fn(lib, v=None) == NULL
    assert fn(lib, out=None) == NULL
    assert fn(lib, B=0) == SHAPE
    assert fn(lib, H=0) == SHAPE
    assert fn(lib, H_kv=0) == SHAPE
    assert fn(lib, M=0) == SHAPE
    assert fn(lib, D=0) == SHAPE
    assert fn(lib, B=-3) == SHAPE
    assert fn(lib, H=6, H_kv=4) == GROUP
    assert fn(lib, tin=7) == DTYPE
    assert fn(lib, tout=9) == DTYPE
    assert fn(lib, tin=F32, tout=BF16, D=128) == DTYPE   # fp32 in, bf16 out
    assert fn(lib, tin=F16, tout=BF16) == DTYPE           # fp16 in, bf16 out
    assert fn(lib, tin=BF16, tout=F16) == DTYPE
    assert fn(lib, tin=F16, tout=F16, D=12) == UNSUP      # fp16 needs D % 8 == 0
    assert fn(lib, tin=F32, tout=F16, D=128) == DTYPE
    assert fn(lib, D=264) == UNSUP
    assert fn(lib, D=12) == UNSUP                         # bf16 needs D % 8 == 0
    assert fn(lib, tin=F32, tout=F32, D=6) == UNSUP       # fp32 needs D % 4 == 0
    assert fn(lib, q=Q + 8) == ALIGN
    assert fn(lib, k=K + 2) == ALIGN
    assert fn(lib, out=O + 4) == ALIGN
    assert fn(lib, out=Q) == ALIAS
    assert fn(lib, out=K + 16) == ALIAS
    assert fn(lib, B=1 << 20, H=1 << 12, H_kv=1 << 12) == SHAPE  # rows >= 2^31


def test_rejections_prefill(lib):
    assert pre(lib, N=0) == SHAPE
    assert pre(lib, mask=O) == ALIAS
    assert band(lib, N=0) == SHAPE
    assert band(lib, mask=O) == ALIAS


def test_rejections_decode_workspace(lib):
    need = lib.gqa_decode_workspace_size(2, 8, 2, 300, 128)
    assert need > 0
    assert dec(lib, ws=None, wsb=0) == WS
    assert dec(lib, wsb=need - 1) == WS
    assert dec(lib, ws=W + 8, wsb=need) == ALIGN
    assert dec(lib, out=W, wsb=need) == ALIAS


def test_rejections_paged(lib):
    assert paged(lib, bt=None) == NULL
    assert paged(lib, kl=None) == NULL
    assert paged(lib, max_blocks=0) == SHAPE
    assert paged(lib, block_size=0) == SHAPE
    assert paged(lib, num_blocks=0) == SHAPE
    assert paged(lib, num_blocks=-1) == SHAPE
    assert paged(lib, block_size=24) == UNSUP             # not a multiple of 16
    assert paged(lib, block_size=8) == UNSUP
    assert paged(lib, max_blocks=1 << 20, block_size=1 << 12) == SHAPE  # M >= 2^31
    assert paged(lib, bt=BT + 2) == ALIGN
    assert paged(lib, kl=KL + 1) == ALIGN
    assert paged(lib, out=BT) == ALIAS
    assert paged(lib, out=KL) == ALIAS
    need = lib.gqa_decode_paged_workspace_size(2, 8, 2, 10, 32, 128)
    assert need > 0
    assert paged(lib, ws=None, wsb=0) == WS
    assert paged(lib, wsb=need - 1) == WS
    assert lib.gqa_decode_paged_workspace_size(2, 8, 2, 0, 32, 128) == 0
    assert lib.gqa_decode_paged_workspace_size(2, 8, 2, 1 << 20, 1 << 12, 128) == 0


def test_workspace_size_rules(lib):
    f = lib.gqa_decode_workspace_size
    assert f(0, 8, 2, 64, 128) == 0
    assert f(1, 6, 4, 64, 128) == 0          # bad group
    # many units: one split per unit, no workspace
    assert f(512, 8, 8, 256, 128) == 0
    # few (batch row, KV head) pairs and a long cache: key splits, workspace
    s2 = f(1, 8, 1, 65536, 128)
    assert s2 > 0 and s2 % 4 == 0
    # a pure function of the sizes
    assert f(1, 8, 1, 65536, 128) == s2
    # layout: the counter area, then [units][splits][16][D + 4] fp32 partials
    # (one unit of 8 heads, 256 splits of 256 keys)
    assert s2 == gqa.DECODE_COUNTER_BYTES + 1 * 256 * 16 * (128 + 4) * 4
    # the large-group path (64 heads on one KV head) keeps the counter area
    # in front of its [B*H][splits][D + 4] partials (47 splits of 64 keys)
    assert f(1, 64, 1, 3000, 64) == gqa.DECODE_COUNTER_BYTES + 64 * 47 * (64 + 4) * 4


def test_paged_workspace_layout(lib):
    """Paged workspace: the counter area, then one [16][D + 4] fp32 partial
    per piece of the length-balanced plan.  The plan launches 512 pieces
    for fewer than 512 (batch row, KV head, head chunk) units, else two per
    unit rounded up to a multiple of 8; caches of at most 256 key slots are
    not split (no workspace)."""
    f = lib.gqa_decode_paged_workspace_size
    part = 16 * (128 + 4) * 4
    nc = gqa.DECODE_COUNTER_BYTES
    assert f(16, 32, 8, 256, 16, 128) == nc + 512 * part       # 128 units
    assert f(64, 32, 8, 256, 16, 128) == nc + 1024 * part      # 512 units
    assert f(31, 8, 1, 64, 16, 128) == nc + 512 * part         # 31 units
    assert f(129, 6, 2, 64, 16, 128) == nc + 512 * part        # 258 units
    assert f(260, 6, 2, 64, 16, 128) == nc + 1040 * part       # 520 units -> 2 * 520
    assert f(16, 32, 8, 16, 16, 128) == 0                      # 256 key slots: no split
    assert f(4096, 8, 1, 64, 16, 128) == 0                     # 4096 units: static plan


def test_counter_area_constant_matches_header():
    import re
    with open(os.path.join(ROOT, "include", "gqa.h")) as fh:
        src = fh.read()
    m = re.search(r"#define GQA_DECODE_COUNTER_BYTES (\d+)", src)
    assert m and int(m.group(1)) == gqa.DECODE_COUNTER_BYTES
    m = re.search(r"#define GQA_DECODE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == gqa.DECODE_NOALLOC_SCRATCH_BYTES


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gqa.decode(q, q[:, :2], q[:, :2])
    with pytest.raises(ValueError):
        gqa.prefill(q, q[:, :2], q[:, :2])
    bt = torch.zeros(1, 1, dtype=torch.int32)
    with pytest.raises(ValueError):
        gqa.decode_paged(q, q[:, :2], q[:, :2], bt, bt[0])


def noalloc(lib, q=Q, k=K, v=V, mask=None, out=O, B=2, H=8, H_kv=2, M=300, D=128,
            tin=BF16, tout=BF16):
    return lib.gqa_decode_noalloc(q, k, v, mask, out, B, H, H_kv, M, D, tin, tout, None)


def test_noalloc_validation(lib):
    """gqa_decode_noalloc checks like gqa_decode, and rejects a problem whose
    workspace would exceed the fixed scratch area, all before any HIP call."""
    assert noalloc(lib, q=None) == NULL
    assert noalloc(lib, B=0) == SHAPE
    assert noalloc(lib, H=9, H_kv=2) == GROUP
    assert noalloc(lib, tin=BF16, tout=F16) == DTYPE
    assert noalloc(lib, D=100) == UNSUP
    assert noalloc(lib, q=Q + 8) == ALIGN
    assert noalloc(lib, out=Q) == ALIAS
    big = (1, 256, 1, 16384, 256)
    assert gqa.decode_workspace_size(*big) > gqa.DECODE_NOALLOC_SCRATCH_BYTES
    assert noalloc(lib, B=big[0], H=big[1], H_kv=big[2], M=big[3], D=big[4]) == SCRATCH
    # a problem that fits needs a GPU (it would launch): not called here
    assert 0 < gqa.decode_workspace_size(16, 32, 8, 4096, 128) <= gqa.DECODE_NOALLOC_SCRATCH_BYTES
