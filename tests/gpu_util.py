"""Helpers shared by the GPU parity tests: host <-> device copies and the
oracle-side expected values. Uses the oracle and the binding side by side;
neither imports the other."""

import numpy as np

from block_quantized_qblk_amd import qblk
from oracle import qblk_oracle as o

# fp32 outputs: max|y - y_ref| / max|y_ref| per output matrix
REL_TOL = 1e-5


def torch():
    import torch as _t
    return _t


def dev(a):
    """numpy -> device tensor (same dtype)."""
    return torch().from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch().cuda.synchronize()
    return t.detach().cpu().numpy()


def dev_quantize(x_np):
    x = dev(x_np.astype(np.float32))
    return qblk.qblk_quantize_act(x)


def dev_pack(wtype, w_np):
    w = dev(w_np.astype(np.float32))
    return qblk.qblk_pack_weights(wtype, w)


def oracle_act(x_np):
    return o.quantize_act(x_np.astype(np.float32))


def oracle_weights(wtype, w_np):
    return o.encode_weights(wtype, w_np.astype(np.float32))


def expected(wtype, w_np, x_np):
    """Oracle y [M, N] (fp64) for float weights and activations."""
    _, enc = oracle_weights(wtype, w_np)
    act = oracle_act(x_np)
    return o.product(wtype, enc, act)[1]


def check_rel(y, yref, tol=REL_TOL):
    err = o.rel_err(y, yref)
    assert err <= tol, f"rel err {err:.3e} > {tol:.0e}"
    return err
