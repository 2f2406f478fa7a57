"""time_attn_bwd_noalloc (the backward whose workspace is the library's static
device scratch) against time_attn_bwd with a caller-allocated workspace,
through the C ABI: two calls in a row, the second with a smaller input, both
needing the scratch (more than 320 frames: the Delta workspace is used), a
shape whose split last round puts its partials there, plus a shape that
needs none and one the scratch cannot hold.  Same kernels, so the
results must be bitwise equal; the first call is also checked against the
oracle.  A shape whose segment partials exceed the scratch takes the
two-kernel path instead and agrees to rounding."""
import numpy as np
import pytest

from block_causal_transformer_amd import configs as C
from block_causal_transformer_amd import gen, ops

import gpu_util as U

pytestmark = pytest.mark.gpu


def _needs_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(w, inp):
    import torch
    q, k, v, do = (U.to_dev(inp[n], w) for n in ("q", "k", "v", "dout"))
    kw = ops.workload_kwargs(w)
    o, lse = ops.attn_fwd("time", q, k, v, **kw)
    ref = ops.attn_bwd("time", q, k, v, o, lse, do, **kw)
    shape, mask = ops.make_shape(q, k), ops.make_mask("time", **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    rc = ops.time_attn_bwd_noalloc(shape, mask, q, k, v, o, lse, do, dq, dk, dv,
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == ops.BCA_OK, ops.bca_last_error()
    torch.cuda.synchronize()
    return ref, (dq, dk, dv)


def test_noalloc_matches_allocating_backward_twice():
    _needs_gpu()
    import torch
    big = C.Workload("time_T1024_W192", "time", 1, 1024, 3, 6, 2, 64, "bf16", 192, 0, 0, 1.0, 9301)
    small = C.Workload("time_T400_W0", "time", 1, 400, 1, 4, 1, 64, "bf16", 0, 0, 0, 1.0, 9302)
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_TIME, ops.BcaShape(1, 1024, 3, 6, 2, 64, 0)) > 0
    for i, w in enumerate((big, small)):
        print("case", w.name, flush=True)
        inp = gen.make_inputs(w)
        ref, got = _both(w, inp)
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), "%s differs from time_attn_bwd (call %d)" % (name, i)
        if i == 0:
            want = U.run_oracle(w, inp)
            print(U.assert_close(w, {"dq": U.to_np(got[0]), "dk": U.to_np(got[1]), "dv": U.to_np(got[2])},
                                 want, w.name + " noalloc"))


def test_noalloc_two_kernel_fallback():
    """Windowed time attention over 1024 frames with 80 problems: the
    segmented backward's fp32 partials (80 x 8 segments x 320 keys x 512
    bytes = 105 MB) do not fit the 64 MiB scratch, so the no-allocation call
    runs the two-kernel backward (Delta, 1 MB); the gradients are then those
    of time_attn_bwd up to rounding (both paths are checked against the
    oracle elsewhere), within the bf16 bars of the parity tests."""
    _needs_gpu()
    w = C.Workload("time_T1024_N40_W192", "time", 1, 1024, 40, 6, 2, 64, "bf16", 192, 0, 0, 1.0, 9304)
    print("case", w.name, flush=True)
    inp = gen.make_inputs(w)
    ref, got = _both(w, inp)
    same = []
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        a, b = U.to_np(a), U.to_np(b)
        excess = float(np.max(np.abs(a - b) - np.maximum(2e-2, 2 * U.half_ulp_bf16(a))))
        rel = float(np.linalg.norm(a - b) / np.linalg.norm(a))
        print(name, "excess %.3g rel %.3g" % (excess, rel))
        assert excess <= 0 and rel <= 5e-3, name
        same.append(np.array_equal(a, b))
    # (the other path: its sums in another order leave other roundings)
    assert not all(same), "expected the two-kernel path's rounding"


def test_noalloc_split_last_round():
    """A fused-path shape whose last round of problems is split (300 problems
    on 256 CUs): the halves' dK, dV partials go to the static scratch."""
    _needs_gpu()
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("sized for 256 CUs")
    w = C.Workload("time_T256_N100_split", "time", 1, 256, 100, 30, 3, 64, "bf16", 192, 0, 0, 1.0, 9303,
                   dout_scale=0.25)
    assert ops.bca_bwd_workspace_bytes(ops.BCA_OP_TIME, ops.BcaShape(1, 256, 100, 30, 3, 64, 0)) > 0
    inp = gen.make_inputs(w)
    ref, got = _both(w, inp)
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), "%s differs from time_attn_bwd" % name


def test_noalloc_without_workspace_and_oversize():
    _needs_gpu()
    import torch
    w = C.get("4").with_(N=2)
    inp = gen.make_inputs(w)
    ref, got = _both(w, inp)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    # 1024 frames x 1000 slots x 30 heads of Delta (123 MB) exceed the 64 MiB scratch:
    # refused on the host before any launch (fake pointers are never touched)
    shape = ops.BcaShape(1, 1024, 1000, 30, 3, 64, ops.BCA_BF16)
    rc = ops.time_attn_bwd_noalloc(shape, ops.make_mask("time", window=192), *([0x10000] * 9))
    assert rc == ops.BCA_ERR_INVALID_ARG and "static scratch" in ops.bca_last_error()
