"""Selection when pooled scores tie exactly: key blocks are duplicated in
groups, so every query block scores a group's blocks equally and the Top-k /
Top-p boundary falls inside a group.  The oracle ranks ties by lower block
index; the kernel must keep the same first ties (bit-exact sets).  Also a row
of all-equal scores.  Calls prism_select directly on a hand-made layout of
64-token blocks."""
import math

import numpy as np
import pytest
import torch

from oracle import prism_oracle as orc

pytestmark = pytest.mark.gpu

NB, D, HEADS = 64, 64, 2


def _run(Q, K, k, p):
    from dynamic_block_sparse_amd import prism as P
    N = NB * 64
    q = torch.from_numpy(Q).to(torch.bfloat16).cuda()
    kk = torch.from_numpy(K).to(torch.bfloat16).cuda()
    offs = torch.arange(0, N + 1, 64, dtype=torch.int32, device="cuda")
    cap = NB * NB
    so = torch.empty((HEADS, NB + 1), dtype=torch.int32, device="cuda")
    si = torch.empty((HEADS, cap), dtype=torch.int32, device="cuda")
    tot = torch.empty(HEADS, dtype=torch.int64, device="cuda")
    ws = torch.empty(P.prism_workspace_size(P.OP_SELECT, N, HEADS, D, NB, cap), dtype=torch.uint8, device="cuda")
    sc = float(np.float32(1.0 / math.sqrt(D)))
    P.prism_select(q, kk, N, HEADS, D, q.stride(0), q.stride(1), offs, NB, k, p, sc, so, si, cap, tot, ws)
    torch.cuda.synchronize()
    Qn, Kn = q.float().cpu().numpy(), kk.float().cpu().numpy()
    off_np = np.arange(NB + 1) * 64
    checked = 0
    for h in range(HEADS):
        L = orc.block_logits(orc.pool_blocks(Qn, off_np, h), orc.pool_blocks(Kn, off_np, h), sc)
        og = so[h].cpu().numpy()
        ig = si[h, :og[-1]].cpu().numpy()
        for i in range(NB):
            want, flag = orc.select_row(L[i], k, p)
            if flag:
                continue
            np.testing.assert_array_equal(ig[og[i]:og[i + 1]], want, err_msg=f"head {h} row {i} (k={k}, p={p})")
            checked += 1
    assert checked >= HEADS * NB // 2
    return checked


@pytest.mark.parametrize("k,p", [(5, 0.0), (3, 0.5), (16, 0.9), (0, 0.37), (64, 0.5), (1, 0.75)])
def test_selection_with_tied_groups(k, p):
    rng = np.random.default_rng(97)
    Kb = rng.standard_normal((NB // 4, 64, HEADS, D)).astype(np.float32)
    K = np.repeat(Kb, 4, axis=0).reshape(NB * 64, HEADS, D)          # blocks 4g..4g+3 identical
    Q = (2.0 * rng.standard_normal((NB * 64, HEADS, D))).astype(np.float32)
    _run(Q, K, k, p)


@pytest.mark.parametrize("k,p", [(0, 0.37), (5, 0.2), (10, 0.9)])
def test_selection_with_all_scores_equal(k, p):
    rng = np.random.default_rng(98)
    Kb = rng.standard_normal((1, 64, HEADS, D)).astype(np.float32)
    K = np.repeat(Kb, NB, axis=0).reshape(NB * 64, HEADS, D)           # every key block identical
    Q = rng.standard_normal((NB * 64, HEADS, D)).astype(np.float32)
    _run(Q, K, k, p)
