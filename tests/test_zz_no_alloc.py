"""ttt_linear_fwd_noalloc (the entry point that allocates nothing: its
large-chunk workspace is the library's static device scratch array) against
ttt_linear_fwd with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so their outputs must agree bit
for bit; each is also within the bf16 tolerance (2e-3) of the fp64 oracle.
Two calls in a row, the second smaller than the first, check that a call does
not depend on what an earlier call left in the shared array.
"""
import numpy as np
import pytest

from weights_ttt_layer_amd import workloads as wlm

from gpu_helpers import TOL, gpu_linear, oracle_linear, rel_err, say

pytestmark = pytest.mark.gpu


def lc(B, H, N, b, eta, seed):
    wl = wlm.Workload(f"noalloc_{B}x{H}x{N}_b{b}_{eta}", "plain", "bf16", B, H, N, 128, b, eta, 0.01,
                      l2_rows=True)
    return wlm.generate(wl, seed)


def gpu_noalloc(inp):
    import torch
    from weights_ttt_layer_amd import linear_fwd_noalloc
    t = wlm.to_device(inp)
    wl = inp.wl
    z, w = linear_fwd_noalloc(t["q"], t["k"], t["v"], t["w0"], t["eta"], b=wl.b, kind=wl.kind,
                              eta_const=inp.eta_const, ln_gamma=t["gamma"], ln_beta=t["beta"], ln_eps=wl.ln_eps)
    torch.cuda.synchronize()
    return z.cpu().numpy(), w.cpu().numpy()


def compare(inp, check_oracle=True):
    z0, w0 = gpu_linear(inp)          # ttt_linear_fwd with a torch-allocated workspace
    z1, w1 = gpu_noalloc(inp)
    same = np.array_equal(z0, z1) and np.array_equal(w0, w1)
    say(f"  {inp.wl.name}: no-alloc output identical to the workspace entry point: {same}")
    assert same
    if check_oracle:
        zr, wr = oracle_linear(inp)
        ez, ew = rel_err(z1, zr), rel_err(w1, wr)
        say(f"  {inp.wl.name}: err Z {ez:.2e} W_end {ew:.2e} (tol 2e-03)")
        assert ez <= TOL["bf16"] and ew <= TOL["bf16"]


def test_noalloc_two_calls_large_then_small():
    """The large-chunk workload at full size (16 heads x 32768 tokens, b = 2048:
    49 MiB of the 64 MiB scratch), then a smaller call (2 heads x 1536 tokens,
    b = 512, per-token eta) in the same process."""
    big = wlm.workload_inputs(4)
    say(f"case {big.wl.name} (no-alloc, first call)")
    compare(big)
    small = lc(1, 2, 1536, 512, "sigmoid", seed=17)
    say(f"case {small.wl.name} (no-alloc, second call)")
    compare(small)


def test_noalloc_small_b_path_runs_as_linear_fwd():
    """The small-b path needs no workspace: the no-alloc entry point runs it as is."""
    wl = wlm.Workload("noalloc_ln_bf16", "ln", "bf16", 2, 3, 70, 64, 16, "sigmoid")
    inp = wlm.generate(wl, 5)
    say(f"case {wl.name}")
    compare(inp)


def test_noalloc_rejects_oversize_before_launch():
    """A problem whose workspace exceeds the scratch array is refused with
    TTT_ERR_WORKSPACE_TOO_SMALL and launches nothing."""
    import torch
    from weights_ttt_layer_amd import TTTError, binding, linear_fwd_noalloc
    B, H, N, d, b = 1, 21, 32768, 128, 2048
    lib = binding.load_library()
    assert lib.ttt_linear_fwd_workspace_bytes(0, 1, B, H, N, d, b) > (64 << 20)
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    w0 = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    z = torch.full((B, H, N, d), 7.0, device="cuda")
    with pytest.raises(TTTError) as ei:
        linear_fwd_noalloc(q, q, q, w0, None, b=b, eta_const=0.01, z=z)
    assert ei.value.status == binding.TTT_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert bool((z == 7.0).all())
