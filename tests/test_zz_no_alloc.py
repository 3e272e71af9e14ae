"""gdn_forward_no_alloc (the forward call whose workspace is the library's static
scratch array) against gdn_forward with a caller workspace, through the C ABI.

Both run the same kernels, so the outputs and final states must agree bit for
bit, which meets the FP16 tolerances (output max-abs 2e-2, final-state relative
L2 1e-3) with room to spare. Two CHUNK-plan calls in a row, the second smaller,
share the one scratch array; a call too large for it is refused before anything
is enqueued.
"""
from __future__ import annotations

import numpy as np
import pytest

from gdn_workloads import make_inputs
from gpu_helpers import device_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gateddeltanet_recurrence_amd as gdn          # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.lib()


def _case(msg):
    print(f"[gpu case] {msg}", flush=True)


def _call(inp, no_alloc, plan):
    d = device_inputs(inp, torch)
    N, Hv, Dv = inp["v"].shape
    R = len(inp["cu_seqlens"]) - 1
    out = torch.full((N, Hv, Dv), float("nan"), dtype=d["v"].dtype, device="cuda")
    fin = torch.full((R, Hv, Dv, inp["Dk"]), float("nan"), dtype=torch.float32, device="cuda")
    args = (d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["cu_seqlens"], out)
    kw = dict(initial_state=d["initial_state"], final_state=fin, cu_seqlens_host=inp["cu_seqlens"], plan=plan)
    if no_alloc:
        gdn.gdn_forward_no_alloc(*args, **kw)
    else:
        nws = gdn.gdn_forward_workspace_bytes(N, R, inp["Hk"], Hv, inp["Dk"], Dv, gdn.GDN_F16, plan=plan,
                                              cu_seqlens_host=inp["cu_seqlens"])
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
        gdn.gdn_forward(*args, workspace=ws, **kw)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), fin.cpu().numpy()


def _same(a, b):
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_no_alloc_matches_workspace_call_twice_second_smaller():
    first = make_inputs([300, 64, 129, 1, 0], 2, 4, 128, 128, "f16", seed=71)
    second = make_inputs([65, 7], 1, 2, 128, 128, "f16", seed=72)
    _case("no-alloc CHUNK call 1: lengths [300, 64, 129, 1, 0], Hv=4")
    _same(_call(first, True, gdn.PLAN_CHUNK), _call(first, False, gdn.PLAN_CHUNK))
    _case("no-alloc CHUNK call 2 (smaller): lengths [65, 7], Hv=2")
    _same(_call(second, True, gdn.PLAN_CHUNK), _call(second, False, gdn.PLAN_CHUNK))
    # the first shape again, after the smaller call left its contents in the array
    _case("no-alloc CHUNK call 3: the first shape again")
    _same(_call(first, True, gdn.PLAN_CHUNK), _call(first, False, gdn.PLAN_CHUNK))


def test_no_alloc_recurrent_plan():
    inp = make_inputs([1] * 8, 2, 4, 128, 128, "f16", seed=73)
    _case("no-alloc RECURRENT decode 8 x 1")
    _same(_call(inp, True, gdn.PLAN_RECURRENT), _call(inp, False, gdn.PLAN_RECURRENT))


def test_no_alloc_refuses_a_call_beyond_the_scratch():
    # forced CHUNK plan without a host mirror: the workspace bound for 8192
    # one-token requests at Hv = 16 is far above 128 MiB; nothing may be written
    R, Hk, Hv, D = 8192, 16, 16, 128
    N = R
    need = gdn.gdn_forward_workspace_bytes(N, R, Hk, Hv, D, D, gdn.GDN_F16, plan=gdn.PLAN_CHUNK)
    assert need > gdn.NO_ALLOC_SCRATCH_BYTES
    _case(f"no-alloc refusal: workspace {need} bytes")
    q = torch.zeros((N, Hk, D), dtype=torch.float16, device="cuda")
    v = torch.zeros((N, Hv, D), dtype=torch.float16, device="cuda")
    a = torch.zeros((N, Hv), dtype=torch.float32, device="cuda")
    A_log = torch.zeros(Hv, dtype=torch.float32, device="cuda")
    cu = torch.arange(R + 1, dtype=torch.int32, device="cuda")
    out = torch.full((N, Hv, D), 3.0, dtype=torch.float16, device="cuda")
    st = gdn.gdn_forward_no_alloc(q, q, v, a, a, A_log, A_log, cu, out, plan=gdn.PLAN_CHUNK, check=False)
    torch.cuda.synchronize()
    assert st == gdn.GDN_ERR_SCRATCH
    assert bool(torch.all(out == 3.0))
