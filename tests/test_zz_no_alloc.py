"""fa_fwd_ws_static (the split launch on the library's static scratch array)
against fa_fwd_ws (the same launch on a caller workspace), through the C
ABI: bitwise equal outputs and lse on consecutive calls, the second with a
smaller input, then the first shape again (the arrival counters the calls
share must be back at zero), plus a shape outside the split that runs
fa_fwd; sampled rows against the oracle."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_04_amd as fa
from attention_fa_fwd_04_amd.workloads import WORKLOADS, make_inputs
from oracle import attention

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def test_static_scratch_matches_workspace_entry():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    fa.lib()
    dev = torch.device("cuda", 0)
    st = torch.cuda.current_stream(dev).cuda_stream
    for H, N in ((24, 4608), (18, 4096), (24, 4608), (2, 777)):
        w = WORKLOADS[2].with_shape(H=H, N=N)
        say(f"case static scratch B=1 H={H} N={N} D=128 bf16")
        inp = make_inputs(w)
        q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
        need = fa.fa_fwd_workspace_bytes(w.B, w.H, w.N, w.D, fa.FA_BF16)
        assert (need > 0) == (N != 777)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        o1, o2 = torch.empty_like(q), torch.full_like(q, float("nan"))
        l1 = torch.empty((1, H, N), dtype=torch.float32, device=dev)
        l2 = torch.full_like(l1, float("nan"))
        args = (w.B, w.H, w.N, w.D, w.scale, fa.FA_BF16)
        rc = fa.fa_fwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), l1.data_ptr(), None, *args,
                          ws.data_ptr(), ws.numel(), st)
        assert rc == fa.FA_OK
        rc = fa.fa_fwd_ws_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), None,
                                 *args, st)
        assert rc == fa.FA_OK, fa.fa_last_hip_error()
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        o_c, l_c = o2.cpu().double().numpy(), l2.cpu().double().numpy()
        worst = 0.0
        for h in range(0, H, 5):
            ids = np.array([0, 1 + 97 * h, N - 1 - 31 * h, N - 1])
            ro, rl = attention.rows(inp["q"][0, h, ids].double().numpy(), inp["k"][0, h].double().numpy(),
                                    inp["v"][0, h].double().numpy(), w.scale)
            worst = max(worst, float(np.abs(o_c[0, h, ids] - ro).max()))
            assert np.abs(l_c[0, h, ids] - rl).max() <= 1e-4
        say(f"  bitwise equal to fa_fwd_ws; sampled rows max|err| vs oracle {worst:.3e}")
        assert worst <= 1e-2
