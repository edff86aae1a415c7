"""The binding rejects caller-supplied output buffers that do not match what
the C functions write (wrong shape, dtype, device or layout) before any
launch: the C side cannot see buffer sizes, so such a buffer would otherwise
be written out of bounds.  Each rejected buffer is filled with a sentinel
first and must come back untouched."""
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg

from gpu_util import DEV

pytestmark = pytest.mark.gpu

B, S, H, D = 1, 64, 2, 128


def _qkv(dtype=torch.bfloat16, shape=(B, S, H, D)):
    g = torch.Generator(device="cpu").manual_seed(5)
    return [torch.randn(shape, generator=g).to(dtype).to(DEV) for _ in range(3)]


def _sentinel(shape, dtype, device=DEV):
    t = torch.empty(shape, dtype=dtype, device=device)
    t.view(torch.uint8).fill_(0xA5)
    return t


def _untouched(t):
    torch.cuda.synchronize()
    return bool((t.contiguous().view(torch.uint8) == 0xA5).all())


BAD_OUT = [
    ("float32", dict(shape=(B, S, H, D), dtype=torch.float32)),
    ("too small", dict(shape=(B, S - 1, H, D), dtype=torch.bfloat16)),
    ("on the host", dict(shape=(B, S, H, D), dtype=torch.bfloat16, device="cpu")),
]


@pytest.mark.parametrize("name,kw", BAD_OUT, ids=[n for n, _ in BAD_OUT])
def test_prefill_bad_out(name, kw):
    q, k, v = _qkv()
    out = _sentinel(**kw)
    with pytest.raises(ValueError):
        pkg.flash_attn_func(q, k, v, out=out)
    if out.is_cuda:
        assert _untouched(out)


def test_prefill_non_contiguous_out():
    q, k, v = _qkv()
    base = _sentinel((B, S, D, H), torch.bfloat16)
    with pytest.raises(ValueError):
        pkg.flash_attn_func(q, k, v, out=base.transpose(2, 3))
    assert _untouched(base)


@pytest.mark.parametrize("shape,dtype", [((B, S, H), torch.float32), ((B, H, S), torch.float16),
                                         ((B, H, S - 1), torch.float32)])
def test_prefill_bad_lse(shape, dtype):
    q, k, v = _qkv()
    lse = _sentinel(shape, dtype)
    out = _sentinel((B, S, H, D), torch.bfloat16)
    with pytest.raises(ValueError):
        pkg.flash_attn_func(q, k, v, out=out, lse=lse)
    assert _untouched(lse) and _untouched(out)


def test_varlen_bad_buffers():
    total = 100
    q, k, v = _qkv(shape=(total, H, D))
    cu = torch.tensor([0, 40, 100], dtype=torch.int32, device=DEV)
    lse_t = _sentinel((total, H), torch.float32)       # transposed LSE layout
    with pytest.raises(ValueError):
        pkg.flash_attn_varlen_func(q, k, v, cu, 60, lse=lse_t)
    assert _untouched(lse_t)
    out = _sentinel((total - 1, H, D), torch.bfloat16)
    with pytest.raises(ValueError):
        pkg.flash_attn_varlen_func(q, k, v, cu, 60, out=out)
    assert _untouched(out)


def test_decode_bad_buffers():
    Bd, Hq, Hkv, ps, pages = 2, 4, 2, 16, 8
    g = torch.Generator(device="cpu").manual_seed(6)
    q = torch.randn((Bd, Hq, D), generator=g).to(torch.bfloat16).to(DEV)
    kc = torch.randn((pages, ps, Hkv, D), generator=g).to(torch.bfloat16).to(DEV)
    vc = torch.randn((pages, ps, Hkv, D), generator=g).to(torch.bfloat16).to(DEV)
    table = torch.arange(Bd * 4, dtype=torch.int32, device=DEV).view(Bd, 4)
    lens = torch.tensor([30, 64], dtype=torch.int32, device=DEV)
    need = pkg.attn_decode_workspace_bytes(Bd, Hq, Hkv, 64, D)
    cases = [
        dict(out=_sentinel((Bd, Hq, D - 1), torch.bfloat16)),
        dict(lse=_sentinel((Hq, Bd), torch.float32)),
        dict(workspace=_sentinel((need - 1,), torch.uint8)),
        dict(workspace=_sentinel(((need + 3) // 4,), torch.float32)),
    ]
    for kw in cases:
        with pytest.raises(ValueError):
            pkg.flash_attn_decode_paged(q, kc, vc, table, lens, 64, **kw)
        (t,) = kw.values()
        assert _untouched(t), kw.keys()
    with pytest.raises(ValueError):
        pkg.flash_attn_decode_paged(q, kc, vc, table, lens, 64,
                                    workspace=torch.empty((need,), dtype=torch.uint8))


def test_good_buffers_still_accepted():
    q, k, v = _qkv()
    out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)
    o2, l2 = pkg.flash_attn_func(q, k, v, out=out, lse=lse)
    torch.cuda.synchronize()
    assert o2.data_ptr() == out.data_ptr() and l2.data_ptr() == lse.data_ptr()
    assert torch.isfinite(out.float()).all()
