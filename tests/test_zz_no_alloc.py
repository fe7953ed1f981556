"""The allocation-free selection (sparse_attn_select_noalloc) against the selection
with a caller's workspace: identical block lists, on two calls in a row that share
the library's static scratch, the second on a smaller input."""
import numpy as np
import pytest
import torch

from block_sparse_attention_row_amd import binding as B
from block_sparse_attention_row_amd.synth import make_inputs, small_workload

from . import parity as P

pytestmark = pytest.mark.gpu


def _lists(rp, ci):
    rp_h = rp.cpu().numpy().astype(np.int64)
    return rp_h, ci[:int(rp_h[-1])].cpu().numpy()


def test_noalloc_selection_matches_the_workspace_selection():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    cases = [
        # larger first, then smaller: the second call finds the first one's contents
        small_workload("noalloc_big", 3, 128, (6, 12, 20), "bf16", threshold=0.8, window=(1, 1, 1),
                       head_threshold_range=(0.6, 0.9), seed=31),
        small_workload("noalloc_small", 2, 64, (2, 3, 5), "bf16", threshold=0.7, seed=32),
    ]
    for wl in cases:
        q, k, _, thr = make_inputs(wl, "A")
        qd, kd = P.to_device(q, k)
        shape = P.shape_for(wl)
        assert 0 < B.sparse_attn_select_noalloc_bytes(shape) <= B.SPARSE_ATTN_SCRATCH_BYTES
        head_thr = None if wl.head_threshold_range is None else [float(x) for x in thr]
        kw = dict(threshold=float(np.float32(wl.threshold)), head_thresholds=head_thr, window=wl.window)
        ref_rp, ref_ci = _lists(*B.sparse_attn_select(shape, qd, kd, **kw))
        bufs = B.alloc_buffers(shape)
        rp, ci = B.sparse_attn_select_noalloc(shape, qd, kd, bufs.row_ptr, bufs.col_idx, **kw)
        torch.cuda.synchronize()
        got_rp, got_ci = _lists(rp, ci)
        print(f"[case] {wl.name}: nnz {int(ref_rp[-1])} (noalloc {int(got_rp[-1])})", flush=True)
        assert np.array_equal(got_rp, ref_rp) and np.array_equal(got_ci, ref_ci)
