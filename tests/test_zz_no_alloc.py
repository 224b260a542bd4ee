"""ttt_chunk_bwd_noalloc (scratch in a fixed device array) against ttt_chunk_bwd (caller
workspace) through the C ABI: two calls in a row, the second on a smaller problem, each
compared with the workspace entry point's output on the same inputs."""
import numpy as np
import pytest

from chunkwise_weight_recurrence_amd import binding as B
from chunkwise_weight_recurrence_amd import workloads as wl
from tests.parity_utils import compare, small_cfg

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dbeta", "dlog_a", "dgamma", "dw0")


def _run_both(cfg, saved):
    import torch
    from chunkwise_weight_recurrence_amd.layer import TTTLayerBuffers, to_f64
    inp = wl.make_ttt_inputs(cfg)
    bufs = TTTLayerBuffers(inp, saved=saved)
    assert B.ttt_workspace_size(bufs.desc, B.ENTRY_BWD) <= B.ttt_noalloc_scratch_bytes()
    bufs.forward()
    bufs.backward()
    torch.cuda.synchronize()
    ref = {g: to_f64(getattr(bufs, g)) for g in GRADS if getattr(bufs, g, None) is not None}
    for g in ref:  # poison the outputs so a call that writes nothing cannot pass
        getattr(bufs, g).fill_(float("nan"))
    B.ttt_chunk_bwd_noalloc(bufs.desc, bufs.q, bufs.k, bufs.v, bufs.beta, bufs.gamma, bufs.log_a, bufs.w0,
                            bufs.w_ckpt, bufs.saved, bufs.d_o, None, bufs.dq, bufs.dk, bufs.dv, bufs.dbeta,
                            bufs.dgamma, bufs.dlog_a, bufs.dw0)
    torch.cuda.synchronize()
    got = {g: to_f64(getattr(bufs, g)) for g in ref}
    return got, ref


@pytest.mark.parametrize("decay,saved", [("vector", True), ("scalar", False)])
def test_noalloc_matches_workspace_entry_two_calls(decay, saved):
    large = small_cfg("bf16", "ip", "silu", decay, B=2, H=4, T=1000, dk=128, dv=128, C=256, b=-4.0)
    small = small_cfg("bf16", "ip", "silu", decay, B=1, H=2, T=300, dk=128, dv=128, C=256, b=-4.0)
    for cfg in (large, small):
        got, ref = _run_both(cfg, saved)
        errs, bad = compare(got, ref, "bf16")
        print(f"[noalloc] {decay} saved={saved} T={cfg['T']}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()),
              flush=True)
        assert not bad, bad
        for g in got:  # the same kernels on the same inputs: identical results
            assert np.array_equal(got[g], ref[g]), g


def test_noalloc_rejects_a_problem_above_the_scratch():
    desc = B.make_desc(64, 16, 8192, 128, 128, 256, "bf16", "ip", "silu", "vector")
    assert B.ttt_workspace_size(desc, B.ENTRY_BWD) > B.ttt_noalloc_scratch_bytes()
    with pytest.raises(B.TTTError) as e:
        B.ttt_chunk_bwd_noalloc(desc, *([1 << 20] * 18))
    assert e.value.status == B.Status.WORKSPACE
