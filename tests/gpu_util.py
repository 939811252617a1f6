"""Helpers for GPU parity tests: move seeded inputs to the device, call the library through
its C ABI binding, compare with the fp64 oracle on the same bits."""
import sys

import numpy as np

TOL_F32 = 1e-4   # max|gpu - oracle| <= TOL * max|oracle|, fp32 inputs
TOL_BF16 = 2e-3  # bf16 inputs, fp32 state; the oracle consumes the identical bf16 values


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dev):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_channel_major(inp):
    """The (B,L,D) / (B,L,N) operands of a seeded input set as (B,D,L) / (B,N,L) arrays."""
    out = dict(inp)
    for k in ("x", "delta", "z", "B", "C"):
        if inp.get(k) is not None:
            out[k] = np.ascontiguousarray(inp[k].transpose(0, 2, 1))
    return out


def run_selective(inp, dev="cuda:0", return_last=True, fill=float("nan"), **options):
    """options: delta_bias (numpy), delta_softplus, exact_zoh, layout -- selective_scan_fwd_ex.
    With layout="bdl" the input arrays are channel-major and so is the returned y."""
    import torch
    import selective_state_space_20_amd as sss
    t = {k: to_dev(v, dev) for k, v in inp.items() if k != "io"}
    if options.get("layout", "bld") == "bdl":
        bt, dm, L = inp["x"].shape
        yshape = (bt, dm, L)
    else:
        bt, L, dm = inp["x"].shape
        yshape = (bt, L, dm)
    n = inp["A"].shape[1]
    y = torch.full(yshape, fill, dtype=torch.float32, device=dev)
    hl = torch.full((bt, dm, n), fill, dtype=torch.float32, device=dev) if return_last else None
    if options.get("delta_bias") is not None:
        options = dict(options, delta_bias=to_dev(options["delta_bias"], dev))
    sss.selective_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"], out=y,
                           out_last=hl, return_last=return_last, **options)
    torch.cuda.synchronize()
    return y.cpu().numpy(), (hl.cpu().numpy() if hl is not None else None)


def run_elementwise(inp, dev="cuda:0", return_last=True, fill=float("nan")):
    import torch
    import selective_state_space_20_amd as sss
    t = {k: to_dev(v, dev) for k, v in inp.items()}
    bt, L, dm = inp["x"].shape
    y = torch.full((bt, L, dm), fill, dtype=torch.float32, device=dev)
    hl = torch.full((bt, dm), fill, dtype=torch.float32, device=dev) if return_last else None
    sss.elementwise_scan(t["x"], t["A"], t["B"], t["C"], t["h0"], out=y, out_last=hl, return_last=return_last)
    torch.cuda.synchronize()
    return y.cpu().numpy(), (hl.cpu().numpy() if hl is not None else None)


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def run_update(x, delta, A, B, C, D, z, state, dev="cuda:0", fill=float("nan")):
    """One decode step on the GPU; returns (y, new state) as numpy float32."""
    import torch
    import selective_state_space_20_amd as sss
    st = to_dev(np.ascontiguousarray(state, dtype=np.float32), dev).clone()
    y = torch.full(x.shape, fill, dtype=torch.float32, device=dev)
    sss.selective_state_update(to_dev(x, dev), to_dev(delta, dev), to_dev(A, dev), to_dev(B, dev), to_dev(C, dev),
                               to_dev(D, dev), to_dev(z, dev), state=st, out=y)
    torch.cuda.synchronize()
    return y.cpu().numpy(), st.cpu().numpy()
