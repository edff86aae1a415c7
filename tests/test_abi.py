"""The C-ABI library builds, loads and exports what include/attn.h declares,
and rejects bad arguments on the host before any HIP call.

Every call here fails validation, so no kernel is launched and no GPU is
needed; the pointers are made-up aligned addresses that are never touched.
"""
import ctypes
import os
import re

import pytest

import causal_prefill_attention_attn_amd as pkg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkg.lib_path()):
        from causal_prefill_attention_attn_amd import _build
        _build.build()
    return pkg.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == sorted(["attn_version", "attn_status_string", "attn_fwd", "attn_fwd_ex",
                            "attn_fwd_balanced", "attn_fwd_varlen",
                            "attn_amax_f32", "attn_quantize_fp8",
                            "attn_quantize_e4m3", "attn_hadamard_f32", "attn_hadamard_bf16",
                            "attn_hadamard_amax_f32", "attn_hadamard_quantize_e4m3",
                            "attn_decode_paged", "attn_decode_paged_noalloc",
                            "attn_decode_workspace_bytes"]), names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert pkg.attn_version() >= 200
    for code in range(0, -11, -1):
        s = pkg.attn_status_string(code)
        assert s and s != "unknown status"
    assert pkg.attn_status_string(-100) == "unknown status"


# made-up, 256-byte aligned, far apart addresses (never dereferenced)
Q, K, V, O, L = (0x10000000 * (i + 1) for i in range(5))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, S=256, H=2, d_qk=128, d_v=128, softmax_scale=0.088,
            causal=1, dtype=0, q_descale=1.0, k_descale=1.0, v_descale=1.0, stream=None)


def _call(**over):
    a = dict(GOOD)
    a.update(over)
    return pkg.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["S"], a["H"],
                        a["d_qk"], a["d_v"], a["softmax_scale"], a["causal"], a["dtype"],
                        a["q_descale"], a["k_descale"], a["v_descale"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(B=0), -2), (dict(S=0), -2), (dict(H=-1), -2), (dict(S=2 ** 31), -2),
    (dict(B=2 ** 20, H=2 ** 12), -2),
    (dict(dtype=2), -3), (dict(dtype=-1), -3),
    (dict(d_qk=64), -4), (dict(d_v=192), -4), (dict(d_qk=192, d_v=192), -4), (dict(causal=2), -4),
    (dict(softmax_scale=0.0), -5), (dict(softmax_scale=float("inf")), -5),
    (dict(softmax_scale=float("nan")), -5), (dict(softmax_scale=-1.0), -5),
    (dict(dtype=1, q_descale=0.0), -5), (dict(dtype=1, v_descale=float("nan")), -5),
    (dict(q=Q + 8), -6), (dict(o=O + 2), -6), (dict(lse=L + 2), -6),
    (dict(o=Q), -7), (dict(o=K + 256), -7), (dict(lse=V + 64), -7), (dict(lse=O + 1024), -7),
])
def test_attn_fwd_rejects(lib, over, code):
    assert _call(**over) == code


def test_balanced_entry_point_checks_its_counter(lib):
    """attn_fwd_balanced runs attn_fwd's checks, plus: the counter (when
    given) must be 4-byte aligned and must not overlap any tensor.  Only
    rejected calls are made here (no GPU)."""
    C = 0x70000000

    def call(counter, **over):
        a = dict(GOOD)
        a.update(over)
        return pkg.attn_fwd_balanced(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["S"],
                                     a["H"], a["d_qk"], a["d_v"], a["softmax_scale"],
                                     a["causal"], a["dtype"], a["q_descale"], a["k_descale"],
                                     a["v_descale"], 0, counter, a["stream"])
    assert call(C + 2) == -6
    assert call(O) == -7 and call(Q + 64) == -7 and call(L) == -7 and call(V + 4) == -7
    assert call(C, q=None) == -1 and call(C, S=0) == -2 and call(C, dtype=2) == -3
    assert call(C, d_qk=64) == -4 and call(C, softmax_scale=0.0) == -5
    assert call(None, o=O + 2) == -6


def test_bf16_ignores_descales_fp8_checks_them(lib):
    # a BF16 call with invalid descales is still rejected only for its real fault
    assert _call(q_descale=float("nan"), d_qk=64) == -4


def test_quant_entry_points_reject(lib):
    assert pkg.attn_amax_f32(None, 10, O) == -1
    assert pkg.attn_amax_f32(Q, 0, O) == -2
    assert pkg.attn_amax_f32(Q, 10, Q + 4) == -7
    assert pkg.attn_quantize_e4m3(Q, 10, 0.0, O) == -5
    assert pkg.attn_quantize_e4m3(Q, 10, 1.0, None) == -1
    assert pkg.attn_quantize_e4m3(Q, 0, 1.0, O) == -2
    assert pkg.attn_quantize_e4m3(Q, 16, 1.0, Q + 8) == -7


def test_quantize_fp8_rejects(lib):
    D = 0x68000000   # descale slot
    f = pkg.attn_quantize_fp8
    assert f(None, 4, 128, 0, O, D) == -1
    assert f(Q, 4, 128, 0, None, D) == -1
    assert f(Q, 4, 128, 0, O, None) == -1
    assert f(Q, 0, 128, 0, O, D) == -2
    assert f(Q, 4, 0, 0, O, D) == -2
    assert f(Q, 1 << 60, 128, 0, O, D) == -2
    assert f(Q, 4, 128, 2, O, D) == -4            # rotate is 0 or 1
    assert f(Q, 4, 100, 1, O, D) == -4            # rotation needs rows of 128 or 192
    assert f(Q + 2, 4, 128, 0, O, D) == -6
    assert f(Q, 4, 128, 0, O, D + 2) == -6
    assert f(Q, 4, 128, 0, Q + 100, D) == -7      # codes inside x
    assert f(Q, 4, 128, 0, O, Q + 64) == -7       # descale inside x
    assert f(Q, 4, 128, 0, O, O + 8) == -7        # descale inside the codes


def test_hadamard_entry_points_reject(lib):
    for fn, esz in ((pkg.attn_hadamard_f32, 4), (pkg.attn_hadamard_bf16, 2)):
        assert fn(None, 4, 128, O) == -1
        assert fn(Q, 4, 128, None) == -1
        assert fn(Q, 0, 128, O) == -2
        assert fn(Q, 1 << 60, 128, O) == -2
        assert fn(Q, 4, 64, O) == -4
        assert fn(Q, 4, 256, O) == -4
        assert fn(Q + 1, 4, 128, O) == -6
        assert fn(Q, 4, 128, Q + 2 * esz) == -7     # partial overlap
    assert pkg.attn_hadamard_amax_f32(None, 4, 128, O) == -1
    assert pkg.attn_hadamard_amax_f32(Q, 0, 128, O) == -2
    assert pkg.attn_hadamard_amax_f32(Q, 4, 64, O) == -4
    assert pkg.attn_hadamard_amax_f32(Q, 4, 128, Q + 8) == -7
    assert pkg.attn_hadamard_quantize_e4m3(Q, 4, 128, 1.0, None) == -1
    assert pkg.attn_hadamard_quantize_e4m3(Q, 4, 192, 0.0, O) == -5
    assert pkg.attn_hadamard_quantize_e4m3(Q, 4, 100, 1.0, O) == -4
    assert pkg.attn_hadamard_quantize_e4m3(Q + 2, 4, 128, 1.0, O) == -6
    assert pkg.attn_hadamard_quantize_e4m3(Q, 4, 128, 1.0, Q + 100) == -7


def test_varlen_entry_point_rejects(lib):
    C = 0x60000000   # cu_seqlens

    def call(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, cu_seqlens=C, n_seqs=3, total=1000, max_seqlen=500,
                 H=4, d_qk=128, d_v=128, softmax_scale=0.1, causal=1, dtype=1, q_descale=1.0,
                 k_descale=1.0, v_descale=1.0)
        a.update(kw)
        return pkg.attn_fwd_varlen(*a.values())
    assert call(cu_seqlens=None) == -1
    assert call(q=None) == -1
    assert call(n_seqs=0) == -2
    assert call(total=0) == -2
    assert call(max_seqlen=0) == -2
    assert call(max_seqlen=1 << 31) == -2
    assert call(d_qk=64) == -4
    assert call(dtype=5) == -3
    assert call(softmax_scale=-1.0) == -5
    assert call(cu_seqlens=C + 2) == -6
    assert call(cu_seqlens=O + 16) == -7          # cu_seqlens inside o
    assert call(lse=Q + 64) == -7


def test_decode_workspace_bytes(lib):
    # B*H_q partial rows of (128 + 1) floats per key split
    n = pkg.attn_decode_workspace_bytes(4, 32, 8, 8192, 128)
    assert n > 0 and n % (4 * 32 * 129 * 4) == 0
    splits = n // (4 * 32 * 129 * 4)
    assert 1 <= splits <= 8192 // 256
    assert pkg.attn_decode_workspace_bytes(1, 8, 8, 100, 128) == 8 * 129 * 4   # one split
    assert pkg.attn_decode_workspace_bytes(0, 8, 8, 100, 128) == -2
    assert pkg.attn_decode_workspace_bytes(1, 12, 8, 100, 128) == -2           # H_q % H_kv
    assert pkg.attn_decode_workspace_bytes(1, 24, 8, 100, 128) == -4           # G = 3
    assert pkg.attn_decode_workspace_bytes(1, 8, 8, 100, 64) == -4
    assert pkg.attn_decode_workspace_bytes(1, 8, 8, 1 << 30, 128) == -2


def test_decode_entry_point_rejects(lib):
    T, N, W = 0x70000000, 0x78000000, 0x80000000   # block table, seq_lens, workspace

    def call(**kw):
        a = dict(q=Q, k_cache=K, v_cache=V, block_table=T, seq_lens=N, o=O, lse=L, workspace=W,
                 workspace_bytes=1 << 30, B=4, H_q=8, H_kv=2, d_qk=128, d_v=128, num_pages=64,
                 page_size=64, max_pages_per_seq=16, max_seqlen=1000, softmax_scale=0.1,
                 dtype=0, q_descale=1.0, k_descale=1.0, v_descale=1.0)
        a.update(kw)
        return pkg.attn_decode_paged(*a.values())
    assert call(block_table=None) == -1
    assert call(seq_lens=None) == -1
    assert call(workspace=None) == -1
    assert call(B=0) == -2
    assert call(H_q=7) == -2                      # not a multiple of H_kv
    assert call(H_q=48, H_kv=2) == -4            # 24 query heads per key/value head
    assert call(page_size=48) == -2               # not a power of two
    assert call(page_size=8) == -2
    assert call(max_seqlen=16 * 64 + 1) == -2     # beyond the block table's pages
    assert call(d_qk=64) == -4
    assert call(d_v=192) == -4
    assert call(dtype=3) == -3
    assert call(softmax_scale=0.0) == -5
    assert call(dtype=1, v_descale=float("inf")) == -5
    assert call(q=Q + 8) == -6
    assert call(block_table=T + 2) == -6
    assert call(workspace=W + 4) == -6
    need = pkg.attn_decode_workspace_bytes(4, 8, 2, 1000, 128)
    assert call(workspace_bytes=need - 1) == -9
    assert call(o=K + 64) == -7                   # o inside the key cache
    assert call(workspace=T) == -7                # workspace over the block table
    assert call(lse=O + 16) == -7                 # lse inside o


def test_decode_noalloc_rejects_on_the_host(lib):
    """Host checks of the allocation-free decode: the same argument checks as
    attn_decode_paged, and steps needing more scratch than the library holds
    rejected before any HIP call (no GPU needed)."""
    T, N = 0x70000000, 0x78000000

    def call(**kw):
        a = dict(q=Q, k_cache=K, v_cache=V, block_table=T, seq_lens=N, o=O, lse=L, B=4, H_q=8,
                 H_kv=2, d_qk=128, d_v=128, num_pages=64, page_size=64, max_pages_per_seq=16,
                 max_seqlen=1000, softmax_scale=0.1, dtype=0, q_descale=1.0, k_descale=1.0,
                 v_descale=1.0)
        a.update(kw)
        return pkg.attn_decode_paged_noalloc(*a.values())
    assert call(q=None) == -1
    assert call(block_table=None) == -1
    assert call(B=0) == -2
    assert call(H_q=48) == -4
    assert call(d_qk=64) == -4
    assert call(dtype=3) == -3
    assert call(softmax_scale=float("nan")) == -5
    assert call(q=Q + 8) == -6
    assert call(o=K + 64) == -7
    assert call(lse=O + 16) == -7
    # 512 sequences of up to 2^20 keys on 64 query heads: the split partials
    # need far more than the static scratch
    big = dict(B=512, H_q=64, H_kv=8, max_seqlen=1 << 20, max_pages_per_seq=1 << 14, num_pages=1 << 20)
    need = pkg.attn_decode_workspace_bytes(512, 64, 8, 1 << 20, 128)
    assert need > pkg.ATTN_DECODE_SCRATCH_BYTES
    assert call(**big) == -10
    assert "scratch" in pkg.attn_status_string(-10)


def test_fwd_ex_flags(lib):
    def call(**kw):
        a = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, S=256, H=2, d_qk=128, d_v=128,
                 softmax_scale=0.1, causal=1, dtype=1, q_descale=1.0, k_descale=1.0,
                 v_descale=1.0, flags=0)
        a.update(kw)
        return pkg.attn_fwd_ex(*a.values())
    assert call(flags=4) == -4                   # unknown flag bit
    assert call(flags=1, dtype=0) == -4          # the O rotation is FP8 only
    assert call(flags=2, dtype=0) == -4          # so is exact P
    assert call(flags=3, dtype=0) == -4
    assert call(flags=1, q=None) == -1
    assert call(flags=1, B=0) == -2
    assert call(flags=1, o=Q + 64) == -7

