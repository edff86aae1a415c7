"""attn_fwd_balanced: the shortest query blocks handed out through a counter
give the same bits as attn_fwd_ex's fixed order.

Shapes with at least 32 query blocks of 256 rows per head take the shared
tail: q_cut = nqb/4 blocks of every head, claimed by 2*B*H*q_cut workgroups.
Each claiming workgroup adds one to the counter, so the counter ends at that
number. At 128 blocks or more with B*H a multiple of 8, the fixed part is
in the head-major order per XCD; otherwise it is in the query-block-major
order. Shorter problems leave the counter alone. The
counter's contents on entry do not matter: the call clears it first. The
parity of these outputs with the oracle is the subject of the full-size
tests, which call through flash_attn_func and so through this entry point.
"""
import math

import pytest
import torch

import causal_prefill_attention_attn_amd as pkg

from gpu_util import DEV

pytestmark = pytest.mark.gpu

BF16, FP8 = 0, 1


def _inputs(B, S, H, dqk, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    t = [torch.randn((B, S, H, d), generator=g, device=DEV) for d in (dqk, dqk, 128)]
    if dtype == BF16:
        return [x.to(torch.bfloat16) for x in t]
    return [x.to(torch.float8_e4m3fn).view(torch.uint8) for x in t]


def _run(fn, q, k, v, B, S, H, dqk, dtype, flags, counter=None):
    o = torch.empty((B, S, H, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, S, H,
            dqk, 128, 1.0 / math.sqrt(dqk), 1, dtype, 1.0, 1.0, 1.0, flags]
    st = torch.cuda.current_stream().cuda_stream
    if fn == "ex":
        rc = pkg.attn_fwd_ex(*args, st)
    else:
        rc = pkg.attn_fwd_balanced(*args, counter, st)
    assert rc == 0, pkg.attn_status_string(rc)
    return o, lse


def _same(a, b):
    return torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and \
        torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("B,S,H,dqk,dtype,flags", [
    (1, 32768, 8, 128, FP8, 0),
    (1, 32768, 8, 128, FP8, 2),          # exact probabilities
    (1, 32768, 8, 128, FP8, 1),          # O rotated back in the epilogue
    (2, 32768 + 100, 4, 192, FP8, 0),    # 129 blocks per head, ragged last block
    (1, 32768, 8, 128, BF16, 0),
    (1, 32768, 8, 192, BF16, 0),
    (1, 32768, 4, 128, FP8, 0),          # B*H = 4: query-block-major order
    (3, 33000, 3, 128, FP8, 0),          # B*H = 9, ragged
    (1, 16384, 32, 128, FP8, 0),         # 64 blocks per head
    (2, 8192, 4, 192, BF16, 0),          # 32 blocks per head, the smallest shared case
])
def test_shared_tail_gives_the_fixed_order_bits(B, S, H, dqk, dtype, flags):
    q, k, v = _inputs(B, S, H, dqk, dtype, seed=S + H + dqk + flags)
    print("case B %d S %d H %d dqk %d dtype %d flags %d" % (B, S, H, dqk, dtype, flags), flush=True)
    ref = _run("ex", q, k, v, B, S, H, dqk, dtype, flags)
    nqb = (S + 255) // 256
    q_cut = nqb // 4
    counter = torch.full((1,), -12345, dtype=torch.int32, device=DEV)
    for _ in range(2):  # the second call finds the first call's count and clears it
        got = _run("bal", q, k, v, B, S, H, dqk, dtype, flags, counter.data_ptr())
        torch.cuda.synchronize()
        assert _same(got, ref)
        assert int(counter.item()) == 2 * B * H * q_cut
    got = _run("bal", q, k, v, B, S, H, dqk, dtype, flags, None)
    assert _same(got, ref)


@pytest.mark.parametrize("B,S,H", [(1, 4096, 8), (2, 7936, 4), (1, 300, 3)])
def test_other_shapes_leave_the_counter_alone(B, S, H):
    """Fewer than 32 blocks per head: the fixed order, the counter
    untouched."""
    q, k, v = _inputs(B, S, H, 128, FP8, seed=7 * S + H)
    ref = _run("ex", q, k, v, B, S, H, 128, FP8, 0)
    counter = torch.full((1,), 777, dtype=torch.int32, device=DEV)
    got = _run("bal", q, k, v, B, S, H, 128, FP8, 0, counter.data_ptr())
    torch.cuda.synchronize()
    assert _same(got, ref)
    assert int(counter.item()) == 777


def test_flash_attn_func_balanced_and_fixed_agree():
    q, k, v = _inputs(1, 32768, 8, 128, FP8, seed=11)
    q, k, v = (x.view(torch.float8_e4m3fn) for x in (q, k, v))
    a = pkg.flash_attn_func(q, k, v)
    b = pkg.flash_attn_func(q, k, v, balanced=False)
    torch.cuda.synchronize()
    assert _same(a, b)


def test_shared_tail_replays_in_a_graph():
    """The counter clear is a kernel, so a captured flash_attn_func on the
    shared-tail path replays correctly. At 8192 tokens (32 blocks per head)
    each replay must claim its blocks again, and every output is poisoned
    before the replay."""
    q, k, v = (x.view(torch.float8_e4m3fn) for x in _inputs(1, 8192, 2, 128, FP8, seed=21))
    o = torch.empty((1, 8192, 2, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, 2, 8192), dtype=torch.float32, device=DEV)
    ref = pkg.flash_attn_func(q, k, v, balanced=False)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pkg.flash_attn_func(q, k, v, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same((o, lse), ref), rep
        pkg.flash_attn_func(k, q, v)  # unrelated eager work between replays
        torch.cuda.synchronize()
