"""moe_permute_noalloc (the entry point for callers that cannot allocate)
against moe_permute through the C ABI: two calls in a row on one GPU, the
second with a smaller input, must each equal moe_permute's outputs bit for
bit (the scratch array keeps the first call's contents, which the second
must not depend on); sizes beyond the scratch are rejected."""
import numpy as np
import pytest

import moe_workloads as W
from gpu_util import dev_bf16, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_grouped_gemm_moe_amd as M


def _outputs(D, T, k, d, EL):
    cap = max(T * k, 1)
    return (torch.full((EL,), -7, dtype=torch.int32, device="cuda"),
            torch.full((EL + 1,), -7, dtype=torch.int32, device="cuda"),
            torch.full((cap,), -7, dtype=torch.int32, device="cuda"),
            torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
            torch.zeros((cap, d), dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("big,small", [((3000, 512, 8, 2, 0, 8), (700, 512, 8, 2, 0, 8)),
                                       ((2000, 256, 64, 6, 8, 40), (150, 256, 64, 6, 8, 40))])
def test_noalloc_permute_equals_permute_on_two_calls(big, small):
    for i, (T, d, E, k, e_lo, e_hi) in enumerate((big, small)):
        cfg = W.CONFIGS["tiny"].scaled(name=f"noalloc{i}", T=T, d=d, f=128, E=E, k=k, e_lo=e_lo,
                                       e_hi=e_hi, seed=40 + i)
        arrs = W.generate(cfg, with_weights=False)
        D = M.MoEDims.make(T, d, 128, E, k, e_lo, e_hi)
        x = dev_bf16(arrs["x"])
        ids, _, _ = M.moe_route(D, x, dev_bf16(arrs["w_router"]))
        say(f"moe_permute T={T} E={E} k={k} local=[{e_lo},{e_hi})")
        ref = M.moe_permute(D, x, ids)
        say(f"moe_permute_noalloc T={T} E={E} k={k} (call {i + 1})")
        got = M.moe_permute_noalloc(D, x, ids, *_outputs(D, T, k, d, e_hi - e_lo))
        torch.cuda.synchronize()
        N = int(ref[1][-1].item())
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
        assert torch.equal(got[2][:N], ref[2][:N]) and torch.equal(got[3], ref[3])
        assert torch.equal(got[4][:N].view(torch.int16), ref[4][:N].view(torch.int16))


def test_noalloc_permute_rejects_sizes_beyond_its_scratch():
    cap = M.load().moe_permute_noalloc_max_ints()
    assert cap == 1 << 18
    # 2 * ceil(T / 256) * E_loc ints are needed: E_loc = 1024 allows T <= 32768
    T, E = 32768 + 256, 1024
    D = M.MoEDims.make(T, 256, 128, E, 2)
    dummy = torch.empty(16, dtype=torch.int32, device="cuda")
    rc = M.load().moe_permute_noalloc(M.C.byref(D), dummy.data_ptr(), dummy.data_ptr(),
                                      dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(),
                                      dummy.data_ptr(), dummy.data_ptr(), None)
    assert rc == -2  # MOE_ERR_UNSUPPORTED, before any launch
