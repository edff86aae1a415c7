"""Paged KV cache layout for the decode tests: contiguous per-sequence rows
scattered into a pool of pages taken in random order.  Input layout only;
no attention arithmetic."""
import numpy as np


def scatter(rng, kc, vc, lens, ps, extra_pages=3):
    """Contiguous per-sequence rows kc[b][:L_b], vc[b][:L_b] ([B, Lmax, H, d]
    encodings) stored in pools of pages taken in random order, one block table
    for both; every slot no sequence owns holds inf (bf16) or NaN (e4m3), so
    a read of it shows in the result.  Returns (k_pool, v_pool, table)."""
    B = kc.shape[0]
    need = [(n + ps - 1) // ps for n in lens]
    total = sum(need) + extra_pages
    order = iter(rng.permutation(total))
    bad = 0x7F80 if kc.dtype == np.uint16 else 0x7F
    kp = np.full((total, ps) + kc.shape[2:], bad, kc.dtype)
    vp = np.full((total, ps) + vc.shape[2:], bad, vc.dtype)
    table = np.zeros((B, max(max(need), 1)), np.int32)
    for b, n in enumerate(lens):
        for p in range(need[b]):
            table[b, p] = next(order)
        for j in range(n):
            kp[table[b, j // ps], j % ps] = kc[b, j]
            vp[table[b, j // ps], j % ps] = vc[b, j]
    return kp, vp, table
