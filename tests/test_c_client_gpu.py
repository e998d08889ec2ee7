"""The C ABI from plain C: ra_client (csrc/ra_client.c, C11 host code that
includes only include/ra.h and the HIP runtime header) runs one rank's
training step (double-buffered forward walk on its own compute and copy
streams, backward walk) on inputs written by this test.  Its outputs must
equal the Python binding's bit for bit on the same inputs, and the fp64
oracle's within the parity bounds."""

import math
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

import long_context_exact_step_amd as ra
import oracle
from parity import TOL_GRAD, TOL_LSE, TOL_O, assert_close, dev, f64, ring_tensors

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "long_context_exact_step_amd", "ra_client")


def test_c_client_training_step(tmp_path):
    B, H, Hk, P, C, d, rank, causal = 1, 4, 2, 3, 150, 128, 2, True
    scale = 1 / math.sqrt(d)
    print(f"ra_client B={B} H={H} H_kv={Hk} P={P} C={C} d={d} rank={rank}", flush=True)
    assert os.path.exists(CLIENT), "ra_client is not built"
    q, k, v, do = ring_tensors(113, B, H, P, C, d, with_do=True, ranks=[rank], H_kv=Hk)
    q, do = q[rank], do[rank]
    bits = lambda t: t.contiguous().view(torch.int16).numpy().tobytes()
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<8if", B, H, Hk, P, C, d, rank, int(causal), scale))
        for t in [q, *k, *v, do]:
            f.write(bits(t))
    r = subprocess.run([CLIENT, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    n_q, n_kv, rows = B * H * C * d, B * Hk * C * d, B * H * C
    got = np.fromfile(out, dtype=np.float32)
    assert got.size == 2 * n_q + rows + 2 * P * n_kv
    c_o = got[:n_q].reshape(B, H, C, d)
    c_lse = got[n_q:n_q + rows].reshape(B, H, C)
    c_dq = got[n_q + rows:2 * n_q + rows].reshape(B, H, C, d)
    kv = got[2 * n_q + rows:].reshape(2, P, B, Hk, C, d)

    # The same step through the Python binding.
    qd, dod = q.to(dev()), do.to(dev())
    kd = [t.to(dev()) for t in k]
    vd = [t.to(dev()) for t in v]
    o = torch.empty(B, H, C, d, device=dev())
    lse = torch.empty(B, H, C, device=dev())
    ra.ring_fwd(qd, kd, vd, o, lse, rank, causal, scale, ring_mode="double_buffer",
                copy_stream=torch.cuda.Stream())
    dq = torch.empty(B, H, C, d, device=dev())
    dk = [torch.zeros(B, Hk, C, d, device=dev()) for _ in range(P)]
    dv = [torch.zeros(B, Hk, C, d, device=dev()) for _ in range(P)]
    ra.ring_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, rank, causal, scale)
    torch.cuda.synchronize()
    for name, a, b in [("o", c_o, o), ("lse", c_lse, lse), ("dq", c_dq, dq)]:
        assert np.array_equal(a, b.cpu().numpy()), f"{name}: C client and binding differ"
    for j in range(P):
        assert np.array_equal(kv[0, j], dk[j].cpu().numpy()), f"dk chunk {j}: C client and binding differ"
        assert np.array_equal(kv[1, j], dv[j].cpu().numpy()), f"dv chunk {j}: C client and binding differ"

    # And the oracle.
    kf, vf = f64(torch.cat(k, 2)), f64(torch.cat(v, 2))
    pos = rank * C + np.arange(C)
    ro, rl = oracle.attention_fwd(f64(q), kf, vf, scale, causal, q_pos=pos)
    rq, rk, rv = oracle.attention_bwd(f64(q), kf, vf, f64(do), scale, causal, q_pos=pos)
    assert_close(c_o, ro, TOL_O, "o")
    assert_close(c_lse, rl, TOL_LSE, "lse", rel=None)
    assert_close(c_dq, rq, TOL_GRAD, "dq")
    for j in range(rank + 1):
        sl = slice(j * C, (j + 1) * C)
        assert_close(kv[0, j], rk[:, :, sl], TOL_GRAD, f"dk chunk {j}")
        assert_close(kv[1, j], rv[:, :, sl], TOL_GRAD, f"dv chunk {j}")
