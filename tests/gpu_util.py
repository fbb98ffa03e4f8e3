"""Helpers for the GPU tests: move generator inputs to the device, run the
decode through the C ABI, compare with the oracle."""
import numpy as np
import torch

import paged_mla_decode_06_amd as mla

BF16_TOL = 1e-2   # max|gpu - oracle| <= tol * max|oracle|
FP8_TOL = 2e-2
LSE_TOL = 1e-3    # absolute, natural log


def to_device(inp, dev="cuda"):
    q = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(dev)
    if inp.kv_fp8:
        pool = torch.from_numpy(inp.pool).view(torch.float8_e4m3fn).to(dev)
    else:
        pool = torch.from_numpy(inp.pool.view(np.int16)).view(torch.bfloat16).to(dev)
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    return q, pool, bt, sl


def run(inp, num_splits=0, min_work_units=None, dev_inputs=None, max_seq_len=None, with_lse=True):
    """Decode on the GPU; returns (out float32 [B,q,H,512], lse float32 [B,q,H]) on the host."""
    q, pool, bt, sl = dev_inputs if dev_inputs is not None else to_device(inp)
    B, ql, H, _ = inp.q.shape
    out = torch.full((B, ql, H, 512), float("nan"), dtype=torch.bfloat16, device=q.device)
    lse = torch.full((B, ql, H), float("nan"), dtype=torch.float32, device=q.device) if with_lse else None
    mwu = inp.workload.min_work_units if min_work_units is None else min_work_units
    msl = inp.max_seq_len if max_seq_len is None else max_seq_len
    mla.mla_decode(q, pool, bt, sl, out, lse, max_seq_len=max(msl, 0), softmax_scale=inp.softmax_scale,
                   k_scale=inp.k_scale, num_splits=num_splits, min_work_units=mwu)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy() if with_lse else None
    return o, l


def compare(o, l, ref_o, ref_l, fp8=False, what=""):
    tol = FP8_TOL if fp8 else BF16_TOL
    ref_o = np.asarray(ref_o)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    scale = float(np.max(np.abs(ref_o))) if ref_o.size else 0.0
    err = float(np.max(np.abs(o - ref_o))) if ref_o.size else 0.0
    if not (err <= tol * max(scale, 1e-30) or (scale == 0 and err == 0)):
        raise AssertionError(f"{what}: max|gpu-oracle| = {err:.3e} > {tol} * {scale:.3e}\n" +
                             _mismatch_report(o, l, ref_o, ref_l, tol * max(scale, 1e-30)))
    if l is not None:
        ref_l = np.asarray(ref_l)
        inf = np.isneginf(ref_l)
        assert np.array_equal(np.isneginf(l), inf), f"{what}: -inf LSE pattern differs"
        if (~inf).any():
            lerr = float(np.max(np.abs(l[~inf] - ref_l[~inf])))
            assert lerr <= LSE_TOL, f"{what}: max|lse err| = {lerr:.3e}"
    return err / max(scale, 1e-30)


def lse_err(l, ref_l):
    """max |lse - ref| over the rows whose reference LSE is finite (0 if none)."""
    ref_l = np.asarray(ref_l)
    fin = ~np.isneginf(ref_l)
    return float(np.max(np.abs(np.asarray(l)[fin] - ref_l[fin]))) if fin.any() else 0.0


def _mismatch_report(o, l, ref_o, ref_l, bound):
    """Where the output is off: the leading indices (everything but the last,
    512-wide axis) of the rows over the bound, the span of dims involved, and
    the LSE error of those rows."""
    d = np.abs(np.asarray(o) - np.asarray(ref_o))
    rows_bad = (d > bound).any(axis=-1)
    idx = np.argwhere(rows_bad)
    lines = [f"  {idx.shape[0]} rows over the bound {bound:.3e}; max err {d.max():.3e} at {np.unravel_index(d.argmax(), d.shape)}"]
    for r in idx[:24]:
        r = tuple(int(x) for x in r)
        dims = np.nonzero(d[r] > bound)[0]
        lse_err = abs(float(np.asarray(l)[r]) - float(np.asarray(ref_l)[r])) if l is not None else float("nan")
        lines.append(f"  row {r}: dims [{dims.min()}, {dims.max()}] ({dims.size}), max err {d[r].max():.3e}, "
                     f"lse err {lse_err:.2e}")
    return "\n".join(lines)
