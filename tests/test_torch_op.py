"""The sparsepr::attention operator: fake shapes (CPU), layouts, batches and
HIP-graph capture (GPU, through the C ABI)."""

import pytest
import torch

import free_block_sparse_amd as sp
import free_block_sparse_amd.torch_op  # noqa: F401  (registers torch.ops.sparsepr.attention)
from synth import make_video_qkv


def test_fake_implementation_propagates_shapes():
    from torch._subclasses.fake_tensor import FakeTensorMode

    with FakeTensorMode():
        q = torch.empty(2, 3, 128, 64, dtype=torch.bfloat16)
        o = torch.ops.sparsepr.attention(q, q, q, density=0.3)
        assert o.shape == q.shape and o.dtype == q.dtype
        qn = torch.empty(2, 128, 3, 64, dtype=torch.bfloat16)
        assert torch.ops.sparsepr.attention(qn, qn, qn, layout="bnhd").shape == qn.shape


def _qkv(heads, seed=21):
    x = make_video_qkv(4, 10, 25, heads, 64, "bf16", seed, [0.06] * heads)
    return tuple(x[t].cuda() for t in ("q", "k", "v"))


KW = dict(density=0.3, n_kv_groups=12, n_q_groups=10, probe_rows=32, residual_rank=8)


@pytest.mark.gpu
def test_token_major_layout_matches_head_major():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q, k, v = _qkv(2)
    ref = torch.ops.sparsepr.attention(q, k, v, **KW)
    qn, kn, vn = (t.permute(0, 2, 1, 3).contiguous() for t in (q, k, v))  # [B, N, H, d]
    got = torch.ops.sparsepr.attention(qn, kn, vn, layout="bnhd", **KW)
    torch.cuda.synchronize()
    assert got.shape == qn.shape
    assert torch.equal(got.permute(0, 2, 1, 3), ref)


@pytest.mark.gpu
def test_batch_is_heads_of_one_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q, k, v = _qkv(4)
    flat = torch.ops.sparsepr.attention(q, k, v, **KW)  # [1, 4, N, d]
    qb, kb, vb = (t.reshape(2, 2, *t.shape[2:]) for t in (q, k, v))  # [2, 2, N, d]: (b, h) -> b*H + h
    got = torch.ops.sparsepr.attention(qb, kb, vb, **KW)
    torch.cuda.synchronize()
    assert torch.equal(got.reshape(flat.shape), flat)


@pytest.mark.gpu
def test_hip_graph_capture_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q, k, v = _qkv(2)
    eager = torch.ops.sparsepr.attention(q, k, v, **KW)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static_out = torch.ops.sparsepr.attention(q, k, v, **KW)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(static_out, eager)
        # eager work between replays, on the same workspace
        again = torch.ops.sparsepr.attention(q, k, v, **KW)
        torch.cuda.synchronize()
        assert torch.equal(again, eager)


@pytest.mark.gpu
def test_opcheck_schema_and_fake():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q, k, v = _qkv(1)
    torch.library.opcheck(torch.ops.sparsepr.attention.default, (q, k, v), KW,
                          test_utils=("test_schema", "test_faketensor"))


@pytest.mark.gpu
def test_operator_token_major_batch_of_two_matches_the_oracle():
    """torch.ops.sparsepr.attention on [B, N, H, d] inputs with B = 2 against
    the oracle's call on the same tensors: every (b, h) slice is its own
    problem, seeded by its index b H + h on both sides."""
    import numpy as np

    from oracle import OracleConfig, sparsepr_call

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q, k, v = _qkv(4, seed=23)
    qb, kb, vb = (t.reshape(2, 2, *t.shape[2:]).permute(0, 2, 1, 3).contiguous() for t in (q, k, v))
    got = torch.ops.sparsepr.attention(qb, kb, vb, layout="bnhd", **KW)
    torch.cuda.synchronize()
    ref = sparsepr_call(*(t.permute(0, 2, 1, 3).cpu() for t in (qb, kb, vb)),
                        OracleConfig(density=0.3, n_kv_groups=12, n_q_groups=10, probe_rows=32, residual_rank=8))
    out = got.permute(0, 2, 1, 3).double().cpu().numpy()
    for b in range(2):
        for h in range(2):
            a, r = out[b, h], ref[b, h]
            ma = float(np.abs(a - r).max())
            rf = float(np.linalg.norm(a - r) / np.linalg.norm(r))
            print(f"  (b={b}, h={h}): max-abs {ma:.2e} rel-Frobenius {rf:.2e}")
            assert ma <= 2e-2 and rf <= 5e-3


@pytest.mark.gpu
def test_first_call_ever_on_a_stream_under_capture():
    """A capture stream that no call has used: the call runs on the capture
    stream and its workspace is that stream's own buffer (allocated in the capture's
    pool).  Replays, with eager calls on the default stream between them,
    match the eager result."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import free_block_sparse_amd as sp

    q, k, v = _qkv(2)  # B = 1, H = 2
    B, H, N, d = q.shape
    cfg = sp.make_config(N, d, density=0.25, probe_rows=32, residual_rank=8)
    ws = sp.Workspace()
    eager = sp.sparsepr_attention(q, k, v, cfg, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        static_out = sp.sparsepr_attention(q, k, v, cfg, workspace=ws)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(static_out, eager)
        again = sp.sparsepr_attention(q, k, v, cfg, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(again, eager)
