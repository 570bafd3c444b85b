"""GPU check of the allocation-free varlen entry against the workspace entry.

chunk_attn_varlen_noalloc runs the mixed prefill + decode batch on the
library's static per-device scratch instead of a caller workspace.  Two calls
in a row, the second on a smaller batch (so the scratch still holds the first
call's offsets and partials), must give outputs and LSE bitwise equal to
chunk_attn_varlen on the same batch, and within the parity bar of the fp64
oracle.
"""
import math

import numpy as np
import pytest
import torch

from chunked_prefill_causal_amd import _lib as L

from gpu_common import BF16_TOL, LSE_TOL, build_batch, log, max_err, oracle_chunk, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    require_gpu()


def run_both(q_lens, kv_lens, hq, hkv, d, dv, seed):
    pool, tables, cu, q_all, seqs = build_batch(q_lens, kv_lens, hq, hkv, d, dv, seed)
    scale = 1.0 / math.sqrt(d)
    q = q_all.cuda()
    ref_out, ref_lse = L.chunk_attn_varlen(q, pool.k, pool.v, tables, cu, kv_lens, scale, return_lse=True)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    cu_dev = torch.tensor(cu, dtype=torch.int32, device="cuda")
    kv_dev = torch.tensor(kv_lens, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    L.chunk_attn_varlen_noalloc(q, pool.k, pool.v, tables, cu, kv_lens, scale, out=out, lse=lse,
                                cu_seqlens_q_dev=cu_dev, kv_lens_dev=kv_dev)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "output differs from chunk_attn_varlen"
    assert torch.equal(lse, ref_lse), "LSE differs from chunk_attn_varlen"
    worst, worst_lse = 0.0, 0.0
    for s, (qh, k, v) in enumerate(seqs):
        ref, ref_l = oracle_chunk(qh, k, v, kv_lens[s] - q_lens[s], scale)
        worst = max(worst, max_err(out[cu[s]: cu[s + 1]], ref))
        worst_lse = max(worst_lse, max_err(lse[:, cu[s]: cu[s + 1]], ref_l))
    log(f"no-alloc varlen, {len(q_lens)} sequences, {cu[-1]} rows: bitwise equal to the workspace entry; "
        f"oracle max err {worst:.3e}, lse {worst_lse:.2e}")
    assert worst <= BF16_TOL and worst_lse <= LSE_TOL


def test_noalloc_matches_workspace_entry_on_two_calls():
    rng = np.random.default_rng(71)
    dec = rng.integers(50, 5000, size=40).tolist()
    run_both([300] + [1] * 40 + [3, 3], [2300] + dec + [700, 4100], 32, 8, 128, 128, 7100)
    dec = rng.integers(10, 900, size=10).tolist()
    run_both([70] + [1] * 10, [700] + dec, 32, 8, 128, 128, 7200)
