"""CPU checks of the test helpers that the GPU parity tests rely on."""
from __future__ import annotations

import numpy as np

from gdn_workloads import make_inputs
from gpu_helpers import oracle_forward_all_heads
from oracle import gdn_oracle as O


def test_all_heads_oracle_in_workers_equals_one_call():
    # head groups run in separate processes and are put back in head order; the
    # grouped-key expansion must give exactly the single-call oracle
    inp = make_inputs([5, 0, 9, 3], 2, 6, 8, 4, "f16", seed=61)
    out, fin = oracle_forward_all_heads(inp, heads_per_task=4, workers=2)
    ref_o, ref_s, _ = O.gdn_forward(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                                    inp["dt_bias"], inp["cu_seqlens"], inp["initial_state"])
    assert np.array_equal(out, ref_o) and np.array_equal(fin, ref_s)
