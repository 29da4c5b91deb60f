"""The allocation-free entry point (sparsepr_attention_noalloc), through the
C ABI: two calls in a row, the second with a smaller input, each equal bit
for bit (output and statistics) to sparsepr_attention on the same inputs.
Both run the same kernels; the fixed scratch keeps the first call's contents
when the second runs."""

import pytest
import torch

import free_block_sparse_amd as sp
from parity_cases import case, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("first,second", [("bf16_d64", "tiny_n"), ("c2_two_heads", "bf16_d64")])
def test_noalloc_equals_the_workspace_call_twice_in_a_row(first, second):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert sp.noalloc_scratch_bytes() == 128 << 20
    for name in (first, second):
        c = case(name)
        print(f"[noalloc] case={name} N={c.n} H={c.heads} d={c.d}", flush=True)
        x = inputs(name)
        q, k, v = (x[t].cuda() for t in ("q", "k", "v"))
        cfg = sp.make_config(c.n, c.d, **c.lib_cfg_kwargs())
        ref, st_ref = sp.sparsepr_attention(q, k, v, cfg, workspace=sp.Workspace(), with_stats=True)
        got, st = sp.sparsepr_attention_noalloc(q, k, v, cfg, with_stats=True)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(st, st_ref)
