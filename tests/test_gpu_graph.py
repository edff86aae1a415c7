"""The attention and decode entry points inside a captured HIP graph.

With outputs (and the decode workspace) allocated beforehand, the calls
allocate nothing and issue no memset, so a graph captured around them
replays the same kernels.  Each replay is checked bitwise against the eager
result, with unrelated eager work and synchronizations between replays."""
import numpy as np
import pytest
import torch

import causal_prefill_attention_attn_amd as pkg
from decode_util import scatter
from gpu_util import DEV, u8_to_device

pytestmark = pytest.mark.gpu


def _fp8(oracle, rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    d = oracle.descale_amax(x)
    return u8_to_device(oracle.quantize_e4m3(x, d)), d


def test_prefill_and_decode_replay_in_a_graph(oracle):
    rng = np.random.default_rng(99)
    B, S, H = 1, 1000, 4
    (q, dq), (k, dk), (v, dv) = (_fp8(oracle, rng, (B, S, H, 128)) for _ in range(3))
    o = torch.empty((B, S, H, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=DEV)

    lens = [700, 33, 1500]
    kc = rng.standard_normal((3, 1500, 2, 128)).astype(np.float32)
    vc = rng.standard_normal((3, 1500, 2, 128)).astype(np.float32)
    dkc, dvc = oracle.descale_amax(kc), oracle.descale_amax(vc)
    kp, vp, table = scatter(rng, oracle.quantize_e4m3(kc, dkc), oracle.quantize_e4m3(vc, dvc),
                            lens, 64)
    dq2 = 0.01
    qd = u8_to_device(rng.integers(0, 0x70, (3, 8, 128), dtype=np.uint8))
    dec_in = (qd, u8_to_device(kp), u8_to_device(vp), torch.from_numpy(table).to(DEV),
              torch.tensor(lens, dtype=torch.int32, device=DEV))
    od = torch.empty((3, 8, 128), dtype=torch.bfloat16, device=DEV)
    ld = torch.empty((3, 8), dtype=torch.float32, device=DEV)
    ws = torch.empty((pkg.attn_decode_workspace_bytes(3, 8, 2, 1500, 128),), dtype=torch.uint8,
                     device=DEV)

    def work():
        pkg.flash_attn_func(q, k, v, q_descale=dq, k_descale=dk, v_descale=dv, out=o, lse=lse,
                            hadamard_o=True)
        pkg.flash_attn_decode_paged(*dec_in, 1500, q_descale=dq2, k_descale=dkc, v_descale=dvc,
                                    out=od, lse=ld, workspace=ws)

    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, od, ld)]

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    other = torch.empty((B, S, H, 128), dtype=torch.bfloat16, device=DEV)
    for rep in range(4):
        for t in (o, lse, od, ld):
            t.fill_(float("nan"))          # the replay must rewrite every output
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in zip((o, lse, od, ld), ref, ("o", "lse", "decode o", "decode lse")):
            assert torch.equal(a.view(torch.int8), b.view(torch.int8)), "replay %d: %s" % (rep,
                                                                                          name)
        # unrelated eager work between replays
        pkg.flash_attn_func(k, q, v, q_descale=dk, k_descale=dq, v_descale=dv, out=other,
                            return_lse=False)
        torch.cuda.synchronize()
    print("4 replays bitwise equal to the eager results")
