"""The allocation-free routed projection (iqk_moe_auto_noalloc, called
through the C ABI by the binding) against iqk_moe_auto with a caller's
workspace: the same path and the same bits, on calls in a row that reuse
the library's device scratch (the second smaller than the first), and the
refusal of a call whose scratch would not fit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import dequant_iqk_moe_amd as q
from gpu_common import TOL_BF16, TOL_GEMV, announce, bf16_round, rel_err_per_vector, to_dev

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_call_on_consecutive_calls():
    fmt, E, out, n = q.IQ2_K, 16, 96, 4096
    wire = synth.wire(fmt, E * out, n, 1600)
    w = q.Weights.from_wire(fmt, E, out, n, wire)
    s = oracle.pack(fmt, wire, E * out, n)
    values = synth.values_table(1601)
    # pairs per expert 40*6/16 = 15 (fused prefill), then 3*6/16 = 1.1
    # (grouped matvec), then 1*6/16 (per-pair matvec): each call smaller
    for T, seed, want in ((40, 1602, "fused_prefill"), (3, 1603, "grouped_gemv"), (1, 1604, "gemv")):
        ids = synth.topk_ids(T, 6, E, seed)
        if T == 40:
            ids[5, 2] = -1  # an invalid id: a NaN row on every path
        x = bf16_round(synth.normal((T, 1, n), seed + 1))
        xd, idd = to_dev(x, torch.bfloat16), to_dev(ids)
        announce(f"no-alloc auto T={T}")
        y_na = torch.full((T, 6, out), 3.0, dtype=torch.float32, device="cuda")
        path = q.moe_auto_noalloc(w, xd, idd, y_na, values)
        y_ws, path_ws = q.moe_auto(w, xd, idd, values)
        torch.cuda.synchronize()
        assert path == path_ws == want
        a, b = y_na.cpu().numpy(), y_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        valid = ids >= 0
        ref = oracle.moe(fmt, s, E, out, n, x, np.where(valid, ids, 0), values)
        tol = TOL_BF16 if path == "fused_prefill" else TOL_GEMV
        assert np.all(rel_err_per_vector(a[valid], ref[valid]) <= tol)
        assert np.all(np.isnan(a[~valid]))


def test_noalloc_refuses_calls_beyond_its_scratch():
    fmt, E, out, n = q.IQ2_K, 16, 16, 512
    w = q.Weights.from_wire(fmt, E, out, n, synth.wire(fmt, E * out, n, 1610))
    T, k = 50_000, 6  # 300 000 pairs: the permutation alone needs 1.2 MB
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    x = torch.zeros((T, 1, n), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, k, out), dtype=torch.float32, device="cuda")
    announce("no-alloc auto: scratch limit")
    with pytest.raises(q.IqkValueError) as ei:
        q.moe_auto_noalloc(w, x, ids, y, synth.values_table(1611))
    assert ei.value.code == -6
