"""GPU: a layer whose send and output buffers exceed 2 GiB, through the C ABI.

16384 tokens, hidden 8704, 64 experts, top-8, capacity 4096 rows per expert (nothing dropped): rows_max = 131072,
so send_buf and out_buf hold 2.1 GiB each and the rows from 123362 on start past the 2 GiB mark. 31-bit buffer offsets cannot address them, so the grouped GEMM takes its
register-staged path with 64-bit pointers (no buffer loads) and the dispatch and combine index past 2^31 bytes.
The layout arrays are checked in full; send rows, expert-MLP rows and combined tokens on samples that include
the rows past the 2 GiB mark.
"""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from tests._hip_runner import LazyExperts, check_close, combine_abs_sum, run_layer, sum_bound_ratio, to_np

pytestmark = pytest.mark.gpu


def test_send_and_output_buffers_above_2_gib():
    T, H, E, k, F, R, C = 16384, 8704, 64, 8, 256, 1, 4096
    cfg = W.small_config(W.workload("dsv3-prefill-ep8-share"), seed=800, name="large_buffers", T=T, H=H, E=E, k=k,
                         F=F, R=R, dtype="bf16", routing="uniform")
    print(f"\n[gpu] large buffers: T={T} H={H} E={E} k={k} F={F} R={R} C={C} bf16 uniform", flush=True)
    inp = W.make_inputs(cfg, device="cuda")
    inp["C"] = C
    out = run_layer(inp, k, R)
    L = out["layout"]
    assert L.rows_max * H * 2 >= 2 ** 31
    x = to_np(inp["x"])
    ids = to_np(out["ids"])
    # layout in full: the oracle's dispatch without materialising its 2 GiB send buffer
    counts = np.bincount(ids.ravel(), minlength=E)
    assert np.array_equal(to_np(L.expert_count), counts)
    lay, _ = oracle.dispatch(np.zeros((T, 8), np.uint16), "bf16", ids, E, C, R)
    for nm in ("expert_count", "expert_kept", "expert_overflow", "expert_offset", "pair_row"):
        assert np.array_equal(to_np(getattr(L, nm)), getattr(lay, nm)), nm
    n = lay.total
    assert n * H * 2 > 2 ** 31, "the kept rows must reach past 2 GiB"
    assert np.array_equal(to_np(L.row_token)[:n], lay.row_token)
    rng = np.random.default_rng(0)
    past = np.nonzero(np.arange(n) * H * 2 >= 2 ** 31)[0]
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 24, replace=False), rng.choice(past, 24, replace=False)]))
    idx = torch.as_tensor(rows, device="cuda", dtype=torch.int64)
    assert np.array_equal(to_np(out["send_buf"][idx]), x[lay.row_token[rows]])
    rex = oracle.row_experts(lay.expert_offset, E)
    ref = oracle.expert_mlp(to_np(out["send_buf"][idx]), "bf16", rex[rows], E // R, LazyExperts(inp["w_gate_up"]),
                            LazyExperts(inp["w_down"]), F)
    check_close(oracle.to_f64(to_np(out["out_buf"][idx]), "bf16"), oracle.to_f64(ref, "bf16"), "bf16", "MLP", 2e-2)
    # combine on tokens whose rows lie past 2 GiB
    tok = np.unique(lay.row_token[rows])
    pr = lay.pair_row[tok]
    used = np.unique(pr[pr >= 0])
    remap = np.full(L.rows_max, -1, dtype=np.int64)
    remap[used] = np.arange(len(used))
    ob = to_np(out["out_buf"][torch.as_tensor(used, device="cuda", dtype=torch.int64)])
    pr_l = np.where(pr >= 0, remap[np.maximum(pr, 0)], -1)
    ref_y = oracle.combine(ob, "bf16", pr_l, to_np(out["w"])[tok])
    got_y, ref_y = oracle.to_f64(to_np(out["y"])[tok], "bf16"), oracle.to_f64(ref_y, "bf16")
    ratio = sum_bound_ratio(got_y, ref_y, combine_abs_sum(oracle.to_f64(ob, "bf16"), pr_l, to_np(out["w"])[tok]),
                            L.k, "bf16")
    check_close(got_y, ref_y, "bf16", "combine", 2e-2, ratio=ratio)
    print(f"[gpu] large buffers: {n} rows ({n * H * 2 / 2**30:.2f} GiB), {len(rows)} rows and {len(tok)} tokens checked")
