"""The allocation-free forward (dspine_draft_forward_noalloc) against the
forward with a caller workspace (dspine_draft_forward): the same kernels on
the library's static scratch, so the outputs are bit-identical.  Two calls
in a row, the second with a smaller input (fewer requests, narrower block),
then a call whose plan exceeds the scratch, refused before any launch."""
import numpy as np
import pytest

import synth
from tests.gpu_cases import Case, Run, rel_err, tol_for, to_np64

pytestmark = pytest.mark.gpu

G_N = synth.Geometry(hidden=512, n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024,
                     n_feat_layers=2, code_dim=128, msg_dim=64, vocab=1000, windows=(40, 0))


@pytest.fixture(autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_drafter_amd as bd
    bd.lib()


def test_noalloc_forward_matches_workspace_forward():
    import torch
    import block_drafter_amd as bd
    print("[noalloc] B=2 W=16, then B=1 W=7, then B=8 W=16 refused", flush=True)
    run = Run(Case(G_N, 99, 2, 16, [45, 130]))
    ws = run.model.workspace(2, 16, 256)
    # first call: two requests, full width
    a = to_np64(run.model.forward(run.ctxs, run.anchors, 16, workspace=ws))
    b = to_np64(run.model.forward_noalloc(run.ctxs, run.anchors, 16))
    assert np.array_equal(a, b)
    orc = run.oracle_forward()
    for r in range(2):
        assert rel_err(b[r], orc[r]) <= tol_for(G_N)
    # second call, smaller: one request, W = 7 (the scratch keeps the first
    # call's contents; only the tile counters must be zero, and are)
    a2 = to_np64(run.model.forward(run.ctxs[1:], run.anchors[1:], 7, workspace=ws))
    b2 = to_np64(run.model.forward_noalloc(run.ctxs[1:], run.anchors[1:], 7))
    assert np.array_equal(a2, b2)
    assert not np.array_equal(b2, b[1:, :7])      # a different block width is a different forward
    # a plan larger than the scratch is refused before any launch
    big = [run.model.new_context(full_capacity=256) for _ in range(8)]
    with pytest.raises(bd.DSpineError) as e:
        run.model.forward_noalloc(big, [1] * 8, 16)
    assert e.value.code == bd.E_WORKSPACE
    torch.cuda.synchronize()
    # the earlier result is unchanged by the refused call
    b3 = to_np64(run.model.forward_noalloc(run.ctxs, run.anchors, 16))
    assert np.array_equal(b3, b)
