"""radix_attn_decode_noalloc (the decode entry point that allocates nothing, using
the library's built-in per-GPU scratch array) against radix_attn_decode with a
caller workspace, through the C ABI.

Each case runs the same workload twice, once per entry point, and compares every
decode output: max-abs <= 2e-2 (bf16 I/O) / 1e-4 (fp32), LSE <= 1e-3 / 1e-5 (the
in-kernel merge may fold partials in another order from run to run, so the two are
equal up to rounding, not bit for bit). The no-allocation outputs are also checked
against the oracle. Cases go from a larger workload to a smaller one, so later
calls find the scratch array holding an earlier, larger call's contents.
"""
import numpy as np
import pytest

from conftest import gpu_available
from workloads import config, few_shot, gqa128_shape, mla_groups

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-4, 1e-5), "bf16": (2e-2, 1e-3)}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def _decode_outputs(w, **kw):
    import torch
    from prefix_shared_kv_radix_amd.runner import Engine
    outs = {}

    def on_decode(rnd, step, out, lse):
        for b, a in enumerate(rnd.admissions):
            outs[(a.rid, step)] = (out[b].float().cpu().numpy(), lse[b].cpu().numpy())

    Engine(w, device="cuda", on_decode=on_decode, **kw).run()
    torch.cuda.synchronize()
    return outs


def _compare(w, **kw):
    from test_gpu_parity import Checker, _run
    print(f"[no-alloc case] {w.name} {kw}", flush=True)
    ref = _decode_outputs(w, **kw)
    got = _decode_outputs(w, noalloc=True, **kw)
    assert ref.keys() == got.keys() and ref
    tol_o, tol_l = TOL[w.shape.q_dtype]
    for k in ref:
        assert np.abs(ref[k][0] - got[k][0]).max() <= tol_o, k
        assert np.abs(ref[k][1] - got[k][1]).max() <= tol_l, k
    _run(w, Checker(w), noalloc=True, **kw)


def test_noalloc_matches_workspace_decode_large_then_small():
    # fused shared-segment decode (plan), 96 requests
    _compare(few_shot(41, gqa128_shape(), 500, 96, 40, 3, q_rows=4096))
    # private-tail work queue without a plan, forced splits, fewer requests
    _compare(few_shot(42, gqa128_shape(), 300, 40, 25, 3, q_rows=4096), use_plan=False,
             num_splits=9)
    # smallest: one request group, one chunk each
    _compare(few_shot(43, gqa128_shape(), 100, 6, 10, 2, q_rows=512))


def test_noalloc_fp32_and_mla_paths():
    _compare(config(1))                                   # fp32 segments + tail + combine
    _compare(mla_groups(44, "bf16", 2, 300, 3, 200, 2, q_rows=256), num_splits=3)


def test_noalloc_rejects_calls_above_its_scratch():
    """A call whose workspace would exceed the built-in array is refused on the host
    (E_INVAL, nothing launched)."""
    import torch
    from prefix_shared_kv_radix_amd import _lib
    from prefix_shared_kv_radix_amd.runner import DeviceState
    w = few_shot(12, gqa128_shape(), 40, 2, 8, 1, q_rows=64)
    d = DeviceState(w, "cuda", 2, 64)
    B, S = 2048, 64
    need = _lib.decode_workspace_size(d.shape, B, 64, None, S)
    assert need > _lib.decode_noalloc_max_bytes()
    s = w.shape
    # every buffer sized for the whole batch (slot lists of slot 0), so the call would
    # stay in bounds even if it were launched
    q = torch.zeros((B, s.num_q_heads, s.head_dim_qk), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, s.num_q_heads, s.head_dim_v), dtype=torch.bfloat16, device="cuda")
    rtt = torch.zeros((B, 64), dtype=torch.int32, device="cuda")
    seq = torch.full((B,), 5, dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.RadixError, match="scratch"):
        _lib.attn_decode_noalloc(d.shape, d.kv, q, None, None, None, None, rtt, None, seq, B, 64,
                                 None, S, out, None)
    torch.cuda.synchronize()
