"""The no-allocation entry point against the existing one (GPU).

csa2_index_full_noalloc runs the kernels of csa2_index_full with their
workspace in the library's fixed per-GPU scratch; its top-k, pool and pool
counts must equal csa2_index_full's bit for bit.  Two calls in a row, the
second smaller, show that nothing left in the scratch by the first call
reaches the second's results.
"""
import numpy as np
import pytest
import torch

import compressed_sparse_attention_mxfp4_amd as csa2
from compressed_sparse_attention_mxfp4_amd import synth

pytestmark = pytest.mark.gpu


def _case(n_entries, T, HI, seed):
    n = np.asarray(n_entries, np.int32)
    B = len(n)
    pg = synth.paging(n, seed=seed)
    kidx = np.zeros((pg.n_pages, 64, 128), np.uint8)
    kidx.reshape(-1, 128)[pg.all_slots()] = synth.fp8_normal((int(n.sum()), 128), seed + 1)
    L = synth.layer_inputs("full", B, T, HI, 16, seed + 2)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return (d(L.q_idx), d(L.w), d(kidx), d(pg.page_table), d(n)), int(n.max())


def test_noalloc_matches_index_full_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.load()
    for label, n_entries, T, HI, topk in (("first, larger", [262144, 40000, 3001, 9], 1, 64, 2048),
                                          ("second, smaller", [1000, 17], 2, 16, 256)):
        print(f"[gpu-case] no-alloc {label}: n={n_entries} T={T} HI={HI} topk={topk}", flush=True)
        args, max_n = _case(n_entries, T, HI, 31 + T)
        ref = csa2.index_full(*args, max_n, topk, 2048)
        got = csa2.index_full_noalloc(*args, max_n, topk, 2048)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        # a request beyond the fixed scratch is refused on the host
    big, _ = _case([8], 2, 64, 5)
    with pytest.raises(csa2.Csa2Error) as e:
        q = torch.zeros((32, 2, 64, 128), dtype=torch.uint8, device="cuda")
        w = torch.zeros((32, 2, 64), dtype=torch.float32, device="cuda")
        pt = torch.zeros((32, 4096), dtype=torch.int32, device="cuda")
        ne = torch.zeros((32,), dtype=torch.int32, device="cuda")
        csa2.index_full_noalloc(q, w, big[2], pt, ne, 262144, 2048, 2048)
    assert e.value.status == csa2.ERR_SCRATCH
