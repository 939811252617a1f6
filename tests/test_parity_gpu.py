"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on identical inputs.

Tolerances: max|gpu - oracle| <= 1e-4 * max|oracle| for fp32 inputs and 2e-3 * max|oracle|
for bf16 inputs with fp32 state, per output tensor (y and h_last separately).
Outputs are pre-filled with NaN so that an element the kernels never write fails.
"""
import os
import re
import zlib

import numpy as np
import pytest

from selective_state_space_20_amd import inputs as gen
from tests.gpu_util import (TOL_BF16, TOL_F32, note, rel_err, run_elementwise, run_selective, run_update, to_channel_major,
                            to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_forced_segments(monkeypatch):
    monkeypatch.delenv("SSS_FORCE_SEGMENTS", raising=False)
    monkeypatch.delenv("SSS_CHUNKED", raising=False)
    yield


def _check_sel(oracle_lib, inp, tag):
    note(f"[selective] {tag} x{inp['x'].shape} N={inp['A'].shape[1]} io={inp['io']}")
    y, hl = run_selective(inp)
    yr, hlr = oracle_lib.selective_scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                        inp["h0"])
    tol = TOL_BF16 if inp["io"] == "bf16" else TOL_F32
    ey, eh = rel_err(y, yr), rel_err(hl, hlr)
    note(f"    err y={ey:.3e} h_last={eh:.3e} (tol {tol:g})")
    assert ey <= tol and eh <= tol, (ey, eh)
    return ey, eh


SEL_CASES = [
    # (batch, seqlen, dim, dstate, io, z, D, h0)
    (1, 1, 1, 1, "f32", False, False, False),
    (1, 2, 3, 4, "f32", True, True, True),
    (2, 63, 4, 16, "f32", False, True, False),
    (1, 64, 64, 16, "bf16", True, True, True),
    (3, 65, 5, 8, "bf16", True, False, True),
    (2, 1000, 100, 16, "f32", True, True, True),
    (1, 1025, 8, 16, "bf16", True, True, True),
    (2, 2049, 12, 64, "f32", False, True, True),
    (1, 3000, 4, 2, "bf16", True, True, False),
    (2, 700, 33, 32, "bf16", False, False, True),
]


@pytest.mark.parametrize("case", SEL_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}N{c[3]}{c[4]}" for c in SEL_CASES])
def test_selective_random_shapes(oracle_lib, case):
    bt, L, dm, n, io, z, D, h0 = case
    inp = gen.selective_inputs(bt, L, dm, n, io=io, with_z=z, with_D=D, h0=h0, seed=zlib.crc32(repr(case).encode()) % 100000)
    _check_sel(oracle_lib, inp, "random")


@pytest.mark.parametrize("segments", [2, 3, 7])
def test_selective_two_pass_forced(oracle_lib, monkeypatch, segments):
    """The two-pass split (segment states, then outputs) forced on shapes that span
    several chunks, with a ragged last segment."""
    monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segments))
    inp = gen.selective_inputs(2, 5000, 8, 16, io="bf16", with_z=True, with_D=True, h0=True, seed=40 + segments)
    _check_sel(oracle_lib, inp, f"S={segments}")
    inp = gen.selective_inputs(1, 9000, 3, 4, io="f32", with_z=False, with_D=True, h0=True, seed=50 + segments)
    _check_sel(oracle_lib, inp, f"S={segments}")


ROW_CASES = [  # (batch, seqlen, dim, dstate, io, forced segments): B/C rows staged through LDS tiles
    (1, 4099, 70, 4, "bf16", 0),    # 64-step tiles, a ragged last tile, tiles past the sequence end
    (2, 517, 130, 16, "f32", 3),    # 16-step tiles; segments of 174 steps end inside a tile
    (1, 1601, 257, 8, "f32", 5),    # 32-step tiles, ragged channel group
    (3, 45, 64, 16, "bf16", 1),     # one segment: two whole tiles and 13 steps
    (1, 18, 5, 16, "bf16", 2),      # segments of 10 and 8 steps, inside one tile
]


@pytest.mark.parametrize("case", ROW_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}N{c[3]}{c[4]}S{c[5]}" for c in ROW_CASES])
def test_selective_row_tiles(oracle_lib, monkeypatch, case):
    """Time-major B/C rows through the per-wave LDS tiles (4, 8 and 16 states), with whole
    and partial tiles, segment ends inside a tile and tile loads past the end of the sequence."""
    bt, L, dm, n, io, S = case
    if S:
        monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(S))
    inp = gen.selective_inputs(bt, L, dm, n, io=io, with_z=True, with_D=True, h0=True,
                               seed=zlib.crc32(repr(case).encode()) % 100000)
    _check_sel(oracle_lib, inp, f"rows S={S}")


CHUNK_CASES = [  # (batch, seqlen, dim, dstate, io, z, D, h0): the single-pass workgroup pair scan
    (2, 1000, 100, 16, "bf16", True, True, True),   # ragged last chunk, ragged channel group
    (1, 32, 64, 16, "f32", False, True, False),     # exactly one chunk
    (3, 33, 70, 8, "bf16", True, False, True),      # one step past a chunk
    (1, 4097, 130, 4, "f32", True, True, True),
    (2, 5, 3, 16, "bf16", True, True, True),        # shorter than one wave's steps
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}N{c[3]}{c[4]}" for c in CHUNK_CASES])
def test_selective_workgroup_pair_scan(oracle_lib, monkeypatch, capfd, case):
    """The single-pass form (SSS_CHUNKED=1): waves of one workgroup take consecutive sub-chunks
    of the same channels, exchange their (decay product, state) pairs through LDS and scan
    them; the library logs that this path ran."""
    monkeypatch.setenv("SSS_CHUNKED", "1")
    monkeypatch.setenv("SSS_LOG", "1")
    bt, L, dm, n, io, z, D, h0 = case
    inp = gen.selective_inputs(bt, L, dm, n, io=io, with_z=z, with_D=D, h0=h0, seed=zlib.crc32(repr(case).encode()) % 100000)
    _check_sel(oracle_lib, inp, "pair scan")
    assert "workgroup pair scan" in capfd.readouterr().err


def test_selective_special_values(oracle_lib):
    """A = 0 (no decay: long carries), A = -inf (memoryless), z = 0 (gate closes)."""
    inp = gen.selective_inputs(2, 3000, 8, 16, io="f32", with_z=False, with_D=True, h0=True, seed=61)
    inp["A"][:, :4] = 0.0
    inp["A"][:, 4:8] = -np.inf
    _check_sel(oracle_lib, inp, "A=0/-inf")
    inp = gen.selective_inputs(1, 300, 8, 16, io="bf16", with_z=True, with_D=True, h0=True, seed=62)
    inp["z"][:] = 0
    y, hl = run_selective(inp)
    assert np.all(y == 0.0)


def test_selective_hand_worked_fixture(oracle_lib):
    """The hand-derived example of tests/golden (exact values) on the GPU."""
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked_selective.json")))
    f = lambda k: np.asarray(g[k], dtype=np.float32)
    inp = dict(x=f("x"), delta=f("delta"), A=f("A"), B=f("B"), C=f("C"), D=f("D"), z=None, h0=f("h0"), io="f32")
    y, hl = run_selective(inp)
    assert rel_err(y, np.asarray(g["y"])) < 1e-6 and rel_err(hl, np.asarray(g["h_last"])) < 1e-6


def test_selective_deterministic_and_no_h_last(oracle_lib):
    """Bitwise-identical repeat runs (no race in LDS/DPP); h_last may be omitted."""
    inp = gen.selective_inputs(2, 4100, 20, 16, io="bf16", with_z=True, with_D=True, h0=True, seed=63)
    y1, h1 = run_selective(inp)
    y2, h2 = run_selective(inp)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)
    y3, _ = run_selective(inp, return_last=False)
    assert np.array_equal(y1, y3)


def test_selective_guard_bands():
    """Writes stay inside y and h_last: canaries around both outputs survive."""
    import torch
    import selective_state_space_20_amd as sss
    from tests.gpu_util import to_dev
    inp = gen.selective_inputs(2, 777, 10, 16, io="bf16", with_z=True, with_D=True, h0=True, seed=64)
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    pad = 1024
    ybuf = torch.full((2 * 777 * 10 + 2 * pad,), 12345.0, device="cuda:0")
    hbuf = torch.full((2 * 10 * 16 + 2 * pad,), 12345.0, device="cuda:0")
    y = ybuf[pad:pad + 2 * 777 * 10].view(2, 777, 10)
    hl = hbuf[pad:pad + 2 * 10 * 16].view(2, 10, 16)
    sss.selective_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"], out=y, out_last=hl)
    torch.cuda.synchronize()
    for buf in (ybuf, hbuf):
        assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[-pad:] == 12345.0)


# ---------------------------------------------------------------- options: exact hold, delta front end
OPT_CASES = [  # (batch, seqlen, dim, dstate, io, exact_zoh, bias, softplus, forced segments)
    (2, 1000, 100, 16, "f32", True, False, False, 0),
    (1, 3000, 40, 16, "bf16", True, False, False, 3),
    (2, 777, 70, 8, "f32", False, True, True, 0),
    (3, 2100, 33, 16, "bf16", False, True, True, 5),
    (2, 500, 64, 4, "f32", False, True, False, 0),
    (2, 1500, 50, 32, "f32", True, True, True, 2),
    (1, 700, 20, 64, "bf16", True, True, True, 0),
]


@pytest.mark.parametrize("case", OPT_CASES, ids=[f"L{c[1]}D{c[2]}N{c[3]}{c[4]}z{int(c[5])}b{int(c[6])}s{int(c[7])}S{c[8]}"
                                                  for c in OPT_CASES])
def test_selective_options(oracle_lib, monkeypatch, case):
    """selective_scan_fwd_ex: exact zero-order hold and the delta front end (bias, softplus),
    alone and together, also across a forced two-pass split."""
    bt, L, dm, n, io, zoh, with_bias, sp, segs = case
    if segs:
        monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segs))
    seed = zlib.crc32(repr(case).encode()) % 100000
    inp = gen.selective_inputs(bt, L, dm, n, io=io, with_D=True, with_z=True, h0=True, seed=seed)
    rng = np.random.default_rng(seed + 1)
    if sp:  # raw step sizes before softplus: spread over both tails
        raw = rng.normal(-3.0, 2.5, size=inp["x"].shape).astype(np.float32)
        inp["delta"] = gen.f32_to_bf16_bits(raw) if io == "bf16" else raw
    bias = None
    if with_bias:  # without softplus the step must stay positive, or the state grows without bound
        bias = (0.5 * rng.standard_normal(dm) if sp else 0.01 * np.abs(rng.standard_normal(dm))).astype(np.float32)
    note(f"[options] {case}")
    y, hl = run_selective(inp, delta_bias=bias, delta_softplus=sp, exact_zoh=zoh)
    yr, hr = oracle_lib.selective_scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                       inp["h0"], exact_zoh=zoh, delta_bias=bias, delta_softplus=sp)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    ey, eh = rel_err(y, yr), rel_err(hl, hr)
    note(f"    err y={ey:.3e} h_last={eh:.3e}")
    assert ey <= tol and eh <= tol


ZOH_SPECIAL_CASES = [(16, "f32", 0), (8, "bf16", 0), (4, "f32", 3), (16, "bf16", 2)]


@pytest.mark.parametrize("case", ZOH_SPECIAL_CASES, ids=[f"N{c[0]}{c[1]}S{c[2]}" for c in ZOH_SPECIAL_CASES])
def test_selective_exact_zoh_special_values(oracle_lib, monkeypatch, case):
    """Exact hold where A = 0 (input term delta*B), A = -inf (no input term), |A| below 2^-64,
    and tiny delta*A (the series branch of expm1): small steps in whole channels, and in a
    few scattered steps of the other channels, so that both the steps that take the direct
    coefficient in every lane and those that need the series in some lanes occur."""
    n, io, segs = case
    if segs:
        monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segs))
    inp = gen.selective_inputs(2, 2000, 140, n, io="f32", with_D=True, with_z=False, h0=True, seed=95 + n)
    inp["A"][:4, :] = 0.0
    inp["A"][4:8, : n // 2] = -np.inf
    inp["A"][8:12, : n // 2] = -1e-30
    inp["delta"][:, :, 12:20] *= 1e-4
    rng = np.random.default_rng(96 + n)
    t_small = rng.choice(2000, size=40, replace=False)
    inp["delta"][:, t_small, 70:] *= 1e-3
    if io == "bf16":
        for k in ("x", "delta"):
            inp[k] = gen.f32_to_bf16_bits(inp[k])
        inp["io"] = "bf16"
    note(f"[exact hold special] N={n} {io} S={segs}")
    y, hl = run_selective(inp, exact_zoh=True)
    yr, hr = oracle_lib.selective_scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                       inp["h0"], exact_zoh=True)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    ey, eh = rel_err(y, yr), rel_err(hl, hr)
    note(f"    err y={ey:.3e} h_last={eh:.3e}")
    assert ey <= tol and eh <= tol


# ---------------------------------------------------------------- channel-major (B,D,L) layout
BDL_CASES = [  # (batch, seqlen, dim, dstate, io, z, D, h0, forced segments, options)
    (1, 1, 1, 1, "f32", False, False, False, 0, {}),
    (2, 64, 64, 16, "bf16", True, True, True, 0, {}),        # 16-byte row pieces
    (2, 200, 33, 16, "f32", True, True, True, 0, {}),        # 4-step pieces, ragged dim
    (1, 1003, 70, 16, "bf16", True, True, True, 0, {}),      # rows not 16-byte aligned: one step per access
    (3, 1000, 20, 8, "bf16", False, True, True, 5, {}),      # forced split, aligned
    (2, 777, 40, 4, "f32", True, False, True, 3, {}),        # forced split, unaligned
    (1, 2048, 130, 32, "bf16", True, True, True, 0, {"delta_softplus": True}),
    (2, 512, 24, 64, "f32", True, True, True, 2, {"exact_zoh": True}),
    (1, 3000, 16, 2, "bf16", True, True, False, 7, {"exact_zoh": True, "delta_softplus": True}),
    # rows a multiple of the 64-byte tile: staged through LDS (the "_rows" entry is the row
    # access the library must report choosing)
    (2, 4096, 100, 16, "bf16", True, True, True, 4, {"_rows": "tile"}),   # ragged last channel group
    (1, 2048, 70, 16, "f32", True, True, True, 2, {"_rows": "tile"}),     # fp32: half-line y pieces
    (2, 1024, 64, 8, "bf16", False, True, False, 0, {"_rows": "tile"}),   # no gate: two staged tensors
    (1, 2048, 96, 16, "bf16", True, True, True, 2, {"delta_softplus": True, "_rows": "tile"}),
    (1, 1024, 40, 4, "f32", True, False, True, 4, {"exact_zoh": True, "_rows": "tile"}),
    (1, 1024, 100, 8, "bf16", True, True, True, 3, {"exact_zoh": True, "delta_softplus": True, "_rows": "tile"}),
]


def _rows_logged(text):
    """(seg_len, row access) from the library's SSS_LOG line of a forward call."""
    m = re.search(r"\[sss\] selective_scan_fwd .* seg_len=(\d+) rows=(\S+)", text)
    assert m, f"no plan line in: {text!r}"
    return int(m.group(1)), m.group(2)


@pytest.mark.parametrize("case", BDL_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}N{c[3]}{c[4]}S{c[8]}" +
                                                 "".join(sorted(k for k in c[9] if not k.startswith("_")))
                                                 for c in BDL_CASES])
def test_selective_channel_major(oracle_lib, monkeypatch, capfd, case):
    """layout="bdl": x/delta/z/y (B,D,L), B/C (B,N,L), against the oracle's channel-major entry
    on the same arrays, over aligned and unaligned rows, splits and options; the row access the
    library reports follows its rule (LDS tiles for rows and segments that are whole 64-byte
    tiles at up to 16 states, else 16-byte pieces where they divide, else one step at a time)."""
    bt, L, dm, n, io, with_z, with_D, with_h0, segs, opts = case
    opts = dict(opts)
    want_rows = opts.pop("_rows", None)
    monkeypatch.setenv("SSS_LOG", "1")
    if segs:
        monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segs))
    seed = zlib.crc32(repr(case).encode()) % 100000
    inp = gen.selective_inputs(bt, L, dm, n, io=io, with_z=with_z, with_D=with_D, h0=with_h0, seed=seed)
    bias = None
    if opts.get("delta_softplus"):
        bias = (0.3 * np.random.default_rng(seed).standard_normal(dm)).astype(np.float32)
    cm = to_channel_major(inp)
    note(f"[channel-major] {case}")
    capfd.readouterr()
    y, hl = run_selective(cm, layout="bdl", delta_bias=bias, **opts)
    seg_len, rows = _rows_logged(capfd.readouterr().err)
    tile, piece = (32, 8) if io == "bf16" else (16, 4)
    rule = ("tile" if n <= 16 and L % tile == 0 and seg_len % tile == 0 else
            "piece" if L % piece == 0 and seg_len % piece == 0 else "step")
    note(f"    rows={rows} seg_len={seg_len}")
    assert rows == rule and (want_rows is None or rows == want_rows)
    yr, hr = oracle_lib.selective_scan(cm["x"], cm["delta"], cm["A"], cm["B"], cm["C"], cm["D"], cm["z"], cm["h0"],
                                       layout="bdl", delta_bias=bias, **opts)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    ey, eh = rel_err(y, yr), rel_err(hl, hr)
    note(f"    err y={ey:.3e} h_last={eh:.3e}")
    assert ey <= tol and eh <= tol


@pytest.mark.timeout(600)
def test_config3_selective_long_channel_major_full(oracle_lib):
    """The long layer (B=1, D=5120, N=16, L=65536, bf16) with channel-major operands, every
    output and the final state against the oracle."""
    cfg, inp = gen.config_inputs(3)
    cm = to_channel_major(inp)
    del inp
    note(f"[channel-major] {cfg['name']} inputs generated")
    y, hl = run_selective(cm, layout="bdl")
    note("    GPU done")
    yr, hlr = oracle_lib.selective_scan(cm["x"], cm["delta"], cm["A"], cm["B"], cm["C"], cm["D"], cm["z"], cm["h0"],
                                        layout="bdl")
    note("    oracle done")
    ey, eh = rel_err(y, yr), rel_err(hl, hlr)
    note(f"    err y={ey:.3e} h_last={eh:.3e}")
    assert ey <= TOL_BF16 and eh <= TOL_BF16


# ---------------------------------------------------------------- backward (gradients)
BWD_CASES = [  # (batch, seqlen, dim, dstate, io, z, D, h0, dh_last, forced segments)
    (1, 1, 1, 1, "f32", False, False, False, False, 0),
    (2, 300, 33, 16, "f32", True, True, True, True, 0),
    (2, 1000, 70, 16, "f32", True, True, True, True, 3),
    (1, 2000, 64, 16, "bf16", True, True, True, True, 0),
    (3, 513, 20, 8, "bf16", False, True, False, True, 7),
    (2, 777, 40, 4, "f32", True, False, True, False, 2),
    (1, 400, 100, 2, "f32", True, True, True, True, 5),
    (2, 300, 24, 32, "f32", True, True, True, True, 3),
    (1, 200, 16, 64, "bf16", True, True, True, True, 2),
    # 16 states keep a checkpoint every four steps: segments whose last two-step sub-chunk is
    # odd-numbered and one step long, and lengths of every residue mod 4
    (1, 665, 40, 16, "bf16", True, True, True, True, 2),
    (2, 1001, 24, 16, "f32", True, False, True, True, 3),
    (1, 7, 70, 16, "f32", True, True, True, True, 0),
    # bf16 with an odd channel count (the last group's lanes past D read channel D-1's 2-byte
    # elements), very short sequences, and a two-state bf16 layer split in segments
    (2, 130, 97, 16, "bf16", True, True, False, True, 2),
    (1, 3, 33, 16, "bf16", True, True, True, True, 0),
    (2, 257, 65, 2, "bf16", True, True, True, True, 4),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}N{c[3]}{c[4]}S{c[9]}" for c in BWD_CASES])
def test_backward(oracle_lib, monkeypatch, case):
    """selective_scan_bwd against the oracle's adjoint gradients (itself pinned by finite
    differences), every gradient tensor, across single- and multi-segment plans."""
    import torch
    import selective_state_space_20_amd as sss
    bt, L, dm, n, io, with_z, with_D, with_h0, with_dhl, segs = case
    if segs:
        monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segs))
    seed = zlib.crc32(repr(case).encode()) % 100000
    inp = gen.selective_inputs(bt, L, dm, n, io=io, with_z=with_z, with_D=with_D, h0=with_h0, seed=seed)
    rng = np.random.default_rng(seed + 7)
    dy = rng.standard_normal((bt, L, dm)).astype(np.float32)
    dhl = rng.standard_normal((bt, dm, n)).astype(np.float32) if with_dhl else None
    note(f"[backward] {case}")
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    g = sss.selective_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                               dy=to_dev(dy, "cuda:0"), dh_last=to_dev(dhl, "cuda:0"))
    torch.cuda.synchronize()
    r = oracle_lib.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                      inp["h0"], dy=dy, dh_last=dhl)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    errs = {}
    for k in ("dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0"):
        if r[k] is None:
            assert g[k] is None
            continue
        errs[k] = rel_err(g[k].cpu().numpy(), r[k])
    note("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= tol for v in errs.values()), errs


BWD_SPECIAL_CASES = [(2, 777, 40, 16, "f32", 5), (1, 1000, 70, 16, "bf16", 4), (2, 513, 33, 8, "f32", 3)]


@pytest.mark.parametrize("case", BWD_SPECIAL_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}N{c[3]}{c[4]}S{c[5]}"
                                                        for c in BWD_SPECIAL_CASES])
def test_backward_special_values(oracle_lib, monkeypatch, case):
    """Gradients where the zero-started checkpoints' correction exp2(A' * S) * h_enter meets its
    limits: states with A = 0 (no decay: the entering state carries unchanged, factor 1), a
    run of zero step sizes across segment boundaries (S = 0 at checkpoints past a segment's
    start, a = 1), and a large initial state (the correction dominates the first segment);
    against the oracle on every gradient element."""
    import torch
    import selective_state_space_20_amd as sss
    bt, L, dm, n, io, segs = case
    monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segs))
    seed = zlib.crc32(repr(case).encode()) % 100000
    inp = gen.selective_inputs(bt, L, dm, n, io=io, with_z=True, with_D=True, h0=True, seed=seed)
    inp["A"][:, : n // 4] = 0.0
    lo, hi = L // 5, L // 5 + L // 4  # zero steps over at least one segment boundary
    inp["delta"][:, lo:hi, :] = 0
    inp["h0"] = (inp["h0"] * 10.0).astype(np.float32)
    rng = np.random.default_rng(seed + 3)
    dy = rng.standard_normal((bt, L, dm)).astype(np.float32)
    dhl = rng.standard_normal((bt, dm, n)).astype(np.float32)
    note(f"[backward special] {case}")
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    g = sss.selective_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                               dy=to_dev(dy, "cuda:0"), dh_last=to_dev(dhl, "cuda:0"))
    torch.cuda.synchronize()
    r = oracle_lib.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                      inp["h0"], dy=dy, dh_last=dhl)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    errs = {k: rel_err(g[k].cpu().numpy(), r[k]) for k in ("dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0")}
    note("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= tol for v in errs.values()), errs


# Gradients through the delta front end (selective_scan_bwd_ex): (batch, seqlen, dim, dstate,
# io, with z, bias, softplus, forced segments).  Single- and multi-segment plans, every state
# count's checkpoint spacing, bf16 with an odd channel count, bias alone and softplus alone.
BWD_FRONT_CASES = [
    (1, 1, 1, 1, "f32", False, True, True, 0),
    (2, 300, 33, 16, "f32", True, True, True, 0),
    (2, 1000, 70, 16, "f32", True, True, True, 3),
    (1, 2000, 64, 16, "bf16", True, True, True, 0),
    (2, 130, 97, 16, "bf16", True, True, True, 2),
    (3, 513, 20, 8, "bf16", False, True, True, 7),
    (2, 777, 40, 4, "f32", True, True, False, 2),
    (1, 400, 100, 2, "f32", True, False, True, 5),
    (2, 300, 24, 32, "f32", True, True, True, 3),
    (1, 200, 16, 64, "bf16", True, True, True, 2),
    (1, 665, 40, 16, "bf16", True, False, True, 2),
]


@pytest.mark.parametrize("case", BWD_FRONT_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}N{c[3]}{c[4]}b{int(c[6])}s{int(c[7])}S{c[8]}"
                                                      for c in BWD_FRONT_CASES])
def test_backward_front_end(oracle_lib, monkeypatch, case):
    """selective_scan_bwd_ex against the oracle's gradients through the front end (step size
    softplus(delta + bias), or delta + bias), every gradient tensor and the bias gradient."""
    import torch
    import selective_state_space_20_amd as sss
    bt, L, dm, n, io, with_z, with_bias, sp, segs = case
    if segs:
        monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segs))
    seed = zlib.crc32(repr(case).encode()) % 100000
    inp = gen.selective_inputs(bt, L, dm, n, io=io, with_z=with_z, with_D=True, h0=True, seed=seed)
    rng = np.random.default_rng(seed + 1)
    if sp:  # raw step sizes before softplus: spread over both tails
        raw = rng.normal(-3.0, 2.5, size=inp["x"].shape).astype(np.float32)
        inp["delta"] = gen.f32_to_bf16_bits(raw) if io == "bf16" else raw
    bias = None
    if with_bias:  # without softplus the step must stay positive
        bias = (0.5 * rng.standard_normal(dm) if sp else 0.01 * np.abs(rng.standard_normal(dm))).astype(np.float32)
    dy = rng.standard_normal((bt, L, dm)).astype(np.float32)
    dhl = rng.standard_normal((bt, dm, n)).astype(np.float32)
    note(f"[backward front end] {case}")
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    g = sss.selective_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                               dy=to_dev(dy, "cuda:0"), dh_last=to_dev(dhl, "cuda:0"),
                               delta_bias=to_dev(bias, "cuda:0"), delta_softplus=sp)
    torch.cuda.synchronize()
    r = oracle_lib.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                      inp["h0"], dy=dy, dh_last=dhl, delta_bias=bias, delta_softplus=sp)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    errs = {}
    for k in ("dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0", "ddelta_bias"):
        if r.get(k) is None:
            assert g.get(k) is None, k
            continue
        errs[k] = rel_err(g[k].cpu().numpy(), r[k])
    note("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= tol for v in errs.values()), errs


def test_backward_front_end_off_is_plain():
    """selective_scan_bwd_ex with no bias and no softplus gives selective_scan_bwd's gradients
    bit for bit (the same kernels)."""
    import torch
    import selective_state_space_20_amd as sss
    from selective_state_space_20_amd import _lib
    bt, L, dm, n = 2, 700, 70, 16
    inp = gen.selective_inputs(bt, L, dm, n, io="bf16", with_z=True, with_D=True, h0=True, seed=77)
    rng = np.random.default_rng(78)
    dy = to_dev(rng.standard_normal((bt, L, dm)).astype(np.float32), "cuda:0")
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    g = sss.selective_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"], dy=dy)
    e = {k: torch.empty_like(v) for k, v in g.items()}
    ws = torch.empty(_lib.selective_scan_bwd_workspace_size(bt, L, dm, n, 0), dtype=torch.uint8, device="cuda:0")
    p = lambda v: 0 if v is None else v.data_ptr()
    rc = _lib.selective_scan_bwd_ex_raw(p(t["x"]), p(t["delta"]), p(t["A"]), p(t["B"]), p(t["C"]), p(t["D"]),
                                        p(t["z"]), p(t["h0"]), p(dy), 0, 0, 0, p(e["dx"]), p(e["ddelta"]), p(e["dA"]),
                                        p(e["dB"]), p(e["dC"]), p(e["dD"]), p(e["dz"]), p(e["dh0"]), 0, bt, L, dm, n,
                                        _lib.SSS_BF16, ws.data_ptr(), ws.numel(),
                                        torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    for k in g:
        assert torch.equal(g[k], e[k]), k


# The saved-states gradients against the recompute path's: fp32 arithmetic on the same
# values in a different order (a checkpoint from the kept state against the state from zero
# plus the decayed entering state), far below the oracle tolerances.
SAVED_TOL = 1e-5

SAVED_CASES = [(2, 1500, 100, 16, "bf16", 5), (1, 777, 70, 8, "f32", 3), (1, 900, 64, 4, "bf16", 0),
               (2, 96, 64, 16, "f32", 1), (1, 700, 20, 64, "bf16", 0)]


@pytest.mark.parametrize("case", SAVED_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}N{c[3]}{c[4]}S{c[5]}" for c in SAVED_CASES])
def test_backward_saved_states(monkeypatch, case):
    """selective_scan_fwd_save gives selective_scan_fwd's outputs bitwise and keeps the segment
    entering states; selective_scan_bwd_saved from them gives selective_scan_bwd's gradients up
    to rounding (its checkpoints start from the kept states, while selective_scan_bwd runs the
    segments from zero and adds the decayed entering state: the same values in different
    order), on two calls in a row; a single-segment plan keeps nothing (size 0, no buffer
    needed) and takes the same kernels, bitwise."""
    import torch
    import selective_state_space_20_amd as sss
    bt, L, dm, n, io, segs = case
    if segs:
        monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segs))
    seed = zlib.crc32(repr(case).encode()) % 100000
    inp = gen.selective_inputs(bt, L, dm, n, io=io, with_z=True, with_D=True, h0=True, seed=seed)
    rng = np.random.default_rng(seed + 5)
    dy = to_dev(rng.standard_normal((bt, L, dm)).astype(np.float32), "cuda:0")
    dhl = to_dev(rng.standard_normal((bt, dm, n)).astype(np.float32), "cuda:0")
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    nbytes = sss.selective_scan_states_size(bt, L, dm, n, 0)
    note(f"[saved states] {case} states {nbytes} bytes")
    if segs == 1:
        assert nbytes == 0
    y_ref, hl_ref = sss.selective_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"])
    g_ref = sss.selective_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"], dy=dy,
                                   dh_last=dhl)
    torch.cuda.synchronize()
    for _ in range(2):
        states = torch.full((max(nbytes // 4, 1),), float("nan"), dtype=torch.float32, device="cuda:0")
        y, hl = sss.selective_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                                       states=states)
        g = sss.selective_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"], dy=dy,
                                   dh_last=dhl, states=states)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(hl, hl_ref)
        for k, v in g_ref.items():
            if v is not None:
                if nbytes == 0:
                    assert torch.equal(g[k], v), k
                else:
                    e = rel_err(g[k].cpu().numpy(), v.cpu().numpy())
                    assert e <= SAVED_TOL, (k, e)


def test_saved_states_errors(monkeypatch):
    """Too small a states buffer, or one overlapping an output, is refused before any work."""
    import torch
    import selective_state_space_20_amd as sss
    monkeypatch.setenv("SSS_FORCE_SEGMENTS", "4")
    inp = gen.selective_inputs(1, 512, 64, 16, io="f32", with_z=False, with_D=False, h0=False, seed=11)
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    nbytes = sss.selective_scan_states_size(1, 512, 64, 16, 0)
    assert nbytes == 4 * 1 * 16 * 64 * 4
    small = torch.empty(nbytes // 4 - 1, dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError):
        sss.selective_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], states=small)
    y = torch.empty((1, 512, 64), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(sss.selective_scan_fwd_workspace_size(1, 512, 64, 16, 0), dtype=torch.uint8, device="cuda:0")
    rc = sss.selective_scan_fwd_save_raw(t["x"].data_ptr(), t["delta"].data_ptr(), t["A"].data_ptr(),
                                         t["B"].data_ptr(), t["C"].data_ptr(), 0, 0, 0, y.data_ptr(), 0,
                                         y.data_ptr(), nbytes, 1, 512, 64, 16, sss.SSS_F32, ws.data_ptr(),
                                         ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == -5  # SSS_ERR_ALIAS: states over y
    rc = sss.selective_scan_fwd_save_raw(t["x"].data_ptr(), t["delta"].data_ptr(), t["A"].data_ptr(),
                                         t["B"].data_ptr(), t["C"].data_ptr(), 0, 0, 0, y.data_ptr(), 0,
                                         small.data_ptr(), small.numel() * 4, 1, 512, 64, 16, sss.SSS_F32,
                                         ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == -4  # SSS_ERR_WORKSPACE: states too small
    torch.cuda.synchronize()


@pytest.mark.timeout(600)
def test_backward_long_layer_full():
    """Gradients of the full-size long layer (B=1, D=5120, N=16, L=65536, bf16, gated, h0,
    dh_last) against the oracle, every element of every gradient tensor; the saved-states
    training pair gives the same gradients up to rounding at this size too."""
    import torch
    import oracle
    import selective_state_space_20_amd as sss
    cfg, inp = gen.config_inputs(3)
    rng = np.random.default_rng(4003)
    dy = rng.standard_normal(inp["x"].shape, dtype=np.float32)
    dhl = rng.standard_normal(inp["h0"].shape, dtype=np.float32)
    note(f"[backward] {cfg['name']} inputs generated")
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    dy_d, dhl_d = to_dev(dy, "cuda:0"), to_dev(dhl, "cuda:0")
    g = sss.selective_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                               dy=dy_d, dh_last=dhl_d)
    # the training pair at full size: the forward keeps its segment entering states and the
    # gradients call starts its checkpoints from them -- the same gradients up to rounding
    b, L, d, n = cfg["batch"], cfg["seqlen"], cfg["dim"], cfg["dstate"]
    states = torch.empty(max(sss.selective_scan_states_size(b, L, d, n), 4) // 4, dtype=torch.float32,
                         device="cuda:0")
    sss.selective_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"], states=states)
    g2 = sss.selective_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                                dy=dy_d, dh_last=dhl_d, states=states)
    torch.cuda.synchronize()
    diff = {k: rel_err(g2[k].cpu().numpy(), g[k].cpu().numpy()) for k in g if g[k] is not None}
    note("    saved-states pair against the recompute path: " + " ".join(f"{k}={v:.1e}" for k, v in diff.items()))
    assert all(v <= SAVED_TOL for v in diff.values()), diff
    del g2, states
    g = {k: (v.cpu().numpy() if v is not None else None) for k, v in g.items()}
    note("    GPU done")
    r = oracle.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["h0"],
                                  dy=dy, dh_last=dhl)
    note("    oracle done")
    errs = {k: rel_err(g[k], r[k]) for k in ("dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0")}
    note("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL_BF16 for v in errs.values()), errs


@pytest.mark.timeout(600)
def test_backward_front_end_long_layer_full():
    """Gradients through the softplus front end (step size softplus(delta + bias)) on the
    full-size long layer (B=1, D=5120, N=16, L=65536, bf16, gated, h0, dh_last), in the plan
    the benchmark times: every element of every gradient tensor and the bias gradient."""
    import torch
    import oracle
    import selective_state_space_20_amd as sss
    cfg, inp = gen.config_inputs(3)
    rng = np.random.default_rng(4004)
    # raw step sizes before softplus, spread over both tails, and a per-channel bias
    inp["delta"] = gen.f32_to_bf16_bits(rng.normal(-3.0, 2.5, size=inp["x"].shape).astype(np.float32))
    bias = (0.5 * rng.standard_normal(cfg["dim"])).astype(np.float32)
    dy = rng.standard_normal(inp["x"].shape, dtype=np.float32)
    dhl = rng.standard_normal(inp["h0"].shape, dtype=np.float32)
    note(f"[backward front end] {cfg['name']} inputs generated")
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    g = sss.selective_scan_bwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["h0"],
                               dy=to_dev(dy, "cuda:0"), dh_last=to_dev(dhl, "cuda:0"),
                               delta_bias=to_dev(bias, "cuda:0"), delta_softplus=True)
    torch.cuda.synchronize()
    g = {k: (v.cpu().numpy() if v is not None else None) for k, v in g.items()}
    del t
    note("    GPU done")
    r = oracle.selective_scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"], inp["h0"],
                                  dy=dy, dh_last=dhl, delta_bias=bias, delta_softplus=True)
    note("    oracle done")
    keys = ("dx", "ddelta", "dA", "dB", "dC", "dD", "dz", "dh0", "ddelta_bias")
    errs = {k: rel_err(g[k], r[k]) for k in keys}
    note("    " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL_BF16 for v in errs.values()), errs


# ---------------------------------------------------------------- causal conv1d front end
CONV_CASES = [  # (batch, seqlen, dim, width, io, silu, bias, forced segments)
    (1, 1, 1, 1, "f32", False, False, 0),
    (2, 100, 64, 4, "bf16", True, True, 0),
    (3, 1000, 37, 4, "f32", True, True, 7),
    (1, 5000, 130, 2, "bf16", False, True, 13),
    (2, 333, 70, 3, "f32", False, False, 3),
    (2, 2000, 200, 8, "bf16", True, False, 5),
    (1, 700, 16, 5, "f32", True, True, 0),
    (2, 640, 96, 6, "bf16", True, True, 4),
    (1, 900, 65, 7, "f32", False, True, 2),
    (1, 40, 4, 4, "bf16", True, True, 3),       # one lane of 4 channels, 61 mirrored lanes
    (2, 300, 2, 3, "f32", True, True, 0),       # one lane of 2 channels
    (1, 3000, 5120, 4, "bf16", True, True, 0),  # the long layer's width, 4 channels per lane
    (2, 1500, 1538, 4, "f32", True, True, 5),   # 2 channels per lane, ragged last wave
]


@pytest.mark.parametrize("case", CONV_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}W{c[3]}{c[4]}s{int(c[5])}S{c[7]}"
                                                  for c in CONV_CASES])
def test_conv1d(oracle_lib, monkeypatch, case):
    """causal_conv1d_fwd against the oracle; forced segment counts put segment boundaries
    (where the window is reloaded from the previous segment) inside the sequence."""
    import torch
    import selective_state_space_20_amd as sss
    bt, L, dm, width, io, silu, with_bias, segs = case
    if segs:
        monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segs))
    rng = np.random.default_rng(zlib.crc32(repr(case).encode()) % 100000)
    x = rng.standard_normal((bt, L, dm)).astype(np.float32)
    if io == "bf16":
        x = gen.f32_to_bf16_bits(x)
    w = rng.standard_normal((dm, width)).astype(np.float32)
    bias = rng.standard_normal(dm).astype(np.float32) if with_bias else None
    note(f"[conv1d] {case}")
    xd = to_dev(x, "cuda:0")
    out = torch.full(xd.shape, float("nan"), dtype=xd.dtype, device="cuda:0")
    sss.causal_conv1d_fwd(xd, to_dev(w, "cuda:0"), to_dev(bias, "cuda:0"), silu=silu, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref = oracle_lib.causal_conv1d(x, w, bias, silu=silu)
    _conv_check(got, ref, io)


def _conv_check(got, ref, io):
    if io == "f32":
        err = rel_err(got, ref)
        note(f"    err {err:.3e}")
        assert err <= TOL_F32
    else:
        # a bf16 output is a rounding decision: every element must be one of the two bf16
        # neighbours of the exact value, i.e. within one bf16 ulp of it (plus fp32 noise)
        assert np.all(np.isfinite(got))
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
        excess = np.abs(got - ref) - ulp - TOL_F32 * np.max(np.abs(ref))
        note(f"    max |err| / ulp = {np.max(np.abs(got - ref) / ulp):.3f}")
        assert np.all(excess <= 0)


@pytest.mark.timeout(600)
def test_conv1d_long_layer_full(oracle_lib):
    """The front end at the long layer's full size (1 x 65536 x 5120 bf16, width 4, bias,
    silu) in the launch configuration the benchmark times, every output element."""
    import torch
    import selective_state_space_20_amd as sss
    rng = np.random.default_rng(4100)
    x = gen.f32_to_bf16_bits(rng.standard_normal((1, 65536, 5120), dtype=np.float32))
    w = (0.5 * rng.standard_normal((5120, 4))).astype(np.float32)
    bias = rng.standard_normal(5120).astype(np.float32)
    note("[conv1d] long layer inputs generated")
    xd = to_dev(x, "cuda:0")
    out = torch.empty(xd.shape, dtype=xd.dtype, device="cuda:0")
    sss.causal_conv1d_fwd(xd, to_dev(w, "cuda:0"), to_dev(bias, "cuda:0"), silu=True, out=out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    del out, xd
    ref = oracle_lib.causal_conv1d(x, w, bias, silu=True)
    _conv_check(got, ref, "bf16")


# ---------------------------------------------------------------- decode step
UPD_CASES = [  # (batch, dim, dstate, io, D, z)
    (1, 1, 1, "f32", False, False),
    (3, 37, 2, "bf16", True, True),
    (2, 100, 4, "f32", True, False),
    (5, 33, 8, "bf16", False, True),
    (4, 5120, 16, "bf16", True, True),
    (3, 77, 16, "f32", True, True),
    (2, 65, 32, "f32", True, True),
    (3, 21, 64, "bf16", True, True),
]


@pytest.mark.parametrize("case", UPD_CASES, ids=[f"B{c[0]}D{c[1]}N{c[2]}{c[3]}" for c in UPD_CASES])
def test_update_random_shapes(oracle_lib, case):
    bt, dm, n, io, with_D, with_z = case
    inp = gen.selective_inputs(bt, 1, dm, n, io=io, with_D=with_D, with_z=with_z, h0=True, h0_std=1.0,
                               seed=zlib.crc32(repr(case).encode()) % 100000)
    x, dl = inp["x"][:, 0], inp["delta"][:, 0]
    z = inp["z"][:, 0] if inp["z"] is not None else None
    state = inp["h0"]
    note(f"[update] B={bt} D={dm} N={n} io={io}")
    y, st = run_update(x, dl, inp["A"], inp["B"][:, 0], inp["C"][:, 0], inp["D"], z, state)
    yr, str_ = oracle_lib.selective_state_update(x, dl, inp["A"], inp["B"][:, 0], inp["C"][:, 0], inp["D"], z, state)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    ey, es = rel_err(y, yr), rel_err(st, str_)
    note(f"    err y={ey:.3e} state={es:.3e}")
    assert ey <= tol and es <= tol


def test_update_continues_a_prefill(oracle_lib):
    """Prefill 300 steps with selective_scan_fwd, then decode 40 tokens one at a time from its
    h_last: outputs and final state match the oracle's scan over all 340 steps."""
    import torch
    import selective_state_space_20_amd as sss
    bt, L0, K, dm, n = 2, 300, 40, 96, 16
    inp = gen.selective_inputs(bt, L0 + K, dm, n, io="bf16", with_D=True, with_z=True, h0=True, seed=91)
    yr, hr = oracle_lib.selective_scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                       inp["h0"])
    pre = {k: (v[:, :L0] if isinstance(v, np.ndarray) and v.ndim == 3 and v.shape[1] == L0 + K else v)
           for k, v in inp.items()}
    y0, h = run_selective(pre)
    t = {k: to_dev(v, "cuda:0") for k, v in inp.items() if k != "io"}
    state = torch.from_numpy(h).cuda()
    ys = []
    for k in range(K):
        s = L0 + k
        c = lambda a: a[:, s].contiguous()
        ys.append(sss.selective_state_update(c(t["x"]), c(t["delta"]), t["A"], c(t["B"]), c(t["C"]), t["D"], c(t["z"]),
                                             state=state))
    torch.cuda.synchronize()
    yk = torch.stack(ys, dim=1).cpu().numpy()
    ey = rel_err(np.concatenate([y0, yk], axis=1), yr)
    eh = rel_err(state.cpu().numpy(), hr)
    note(f"[update] prefill+decode err y={ey:.3e} state={eh:.3e}")
    assert ey <= TOL_BF16 and eh <= TOL_BF16


def test_update_guard_bands():
    """The update writes exactly the state and y: canaries around both survive."""
    import torch
    import selective_state_space_20_amd as sss
    bt, dm, n = 3, 45, 16
    inp = gen.selective_inputs(bt, 1, dm, n, io="f32", with_D=True, with_z=True, h0=True, seed=92)
    pad = 1024
    sbuf = torch.full((bt * dm * n + 2 * pad,), 12345.0, device="cuda:0")
    ybuf = torch.full((bt * dm + 2 * pad,), 12345.0, device="cuda:0")
    st = sbuf[pad:pad + bt * dm * n].view(bt, dm, n)
    st.copy_(torch.from_numpy(inp["h0"]))
    y = ybuf[pad:pad + bt * dm].view(bt, dm)
    d = lambda a: to_dev(np.ascontiguousarray(a), "cuda:0")
    sss.selective_state_update(d(inp["x"][:, 0]), d(inp["delta"][:, 0]), d(inp["A"]), d(inp["B"][:, 0]),
                               d(inp["C"][:, 0]), d(inp["D"]), d(inp["z"][:, 0]), state=st, out=y)
    torch.cuda.synchronize()
    for buf in (sbuf, ybuf):
        assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[-pad:] == 12345.0)
    assert torch.all(torch.isfinite(y)) and torch.all(torch.isfinite(st))


# ---------------------------------------------------------------- elementwise
def _check_ew(oracle_lib, inp, tag):
    note(f"[elementwise] {tag} x{inp['x'].shape}")
    y, hl = run_elementwise(inp)
    yr, hlr = oracle_lib.elementwise_scan(inp["x"], inp["A"], inp["B"], inp["C"], inp["h0"])
    ey, eh = rel_err(y, yr), rel_err(hl, hlr)
    note(f"    err y={ey:.3e} h_last={eh:.3e}")
    assert ey <= TOL_F32 and eh <= TOL_F32, (ey, eh)


EW_CASES = [(1, 1, 1, False), (2, 6, 4, False), (2, 64, 4, False), (3, 1000, 65, True), (1, 5000, 3, True),
            (4, 333, 130, True), (2, 777, 200, True), (1, 3000, 4096, True), (3, 129, 1028, False)]


@pytest.mark.parametrize("case", EW_CASES, ids=[f"B{c[0]}L{c[1]}D{c[2]}" for c in EW_CASES])
def test_elementwise_random_shapes(oracle_lib, case):
    bt, L, dm, h0 = case
    _check_ew(oracle_lib, gen.elementwise_inputs(bt, L, dm, h0=h0, seed=zlib.crc32(repr(case).encode()) % 100000), "random")


@pytest.mark.parametrize("segments", [2, 5, 64])
def test_elementwise_two_pass_forced(oracle_lib, monkeypatch, segments):
    monkeypatch.setenv("SSS_FORCE_SEGMENTS", str(segments))
    _check_ew(oracle_lib, gen.elementwise_inputs(2, 3001, 7, h0=True, seed=70 + segments), f"S={segments}")
    _check_ew(oracle_lib, gen.elementwise_inputs(2, 3001, 520, h0=True, seed=90 + segments), f"S={segments} D=520")


def test_elementwise_hand_worked_and_zero_decay(oracle_lib):
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked_elementwise.json")))
    f = lambda k: np.asarray(g[k], dtype=np.float32)
    y, hl = run_elementwise(dict(x=f("x"), A=f("A"), B=f("B"), C=f("C"), h0=f("h0")))
    assert np.array_equal(y, np.asarray(g["y"], dtype=np.float32))
    assert np.array_equal(hl, np.asarray(g["h_last"], dtype=np.float32))
    inp = gen.elementwise_inputs(2, 500, 9, h0=True, seed=71)
    inp["A"][:] = 0.0
    y, _ = run_elementwise(inp)
    assert np.array_equal(y, (inp["C"] * (inp["B"] * inp["x"])).astype(np.float32))


# ---------------------------------------------------------------- the configurations
def test_config0_elementwise_small(oracle_lib):
    cfg, inp = gen.config_inputs(0)
    _check_ew(oracle_lib, inp, cfg["name"])


def test_config1_selective_fp32(oracle_lib):
    cfg, inp = gen.config_inputs(1)
    _check_sel(oracle_lib, inp, cfg["name"])


def test_config2_selective_bf16_full(oracle_lib):
    cfg, inp = gen.config_inputs(2)
    _check_sel(oracle_lib, inp, cfg["name"])


@pytest.mark.timeout(600)
def test_config3_selective_long_full(oracle_lib):
    """Full-size long-sequence layer (B=1, D=5120, N=16, L=65536, bf16) in the launch
    configuration the benchmark times: every output and the final state against the oracle
    (all channels, all steps; the oracle runs the whole layer on the host threads)."""
    cfg, inp = gen.config_inputs(3)
    note(f"[selective] {cfg['name']} inputs generated")
    y, hl = run_selective(inp)
    note("    GPU done")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hl))
    yr, hlr = oracle_lib.selective_scan(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["D"], inp["z"],
                                        inp["h0"])
    note("    oracle done")
    ey, eh = rel_err(y, yr), rel_err(hl, hlr)
    note(f"    err y={ey:.3e} h_last={eh:.3e}")
    assert ey <= TOL_BF16 and eh <= TOL_BF16


@pytest.mark.timeout(900)
def test_config4_elementwise_large_full(oracle_lib):
    """Full-size elementwise scan (8 x 32768 x 4096, fp32): every output against the oracle,
    which runs the whole scan on the host threads."""
    cfg, inp = gen.config_inputs(4)
    note(f"[elementwise] {cfg['name']} inputs generated")
    y, hl = run_elementwise(inp)
    note("    GPU done")
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(hl))
    yr, hlr = oracle_lib.elementwise_scan(inp["x"], inp["A"], inp["B"], inp["C"], inp["h0"])
    note("    oracle done")
    ey, eh = rel_err(y, yr), rel_err(hl, hlr)
    note(f"    err y={ey:.3e} h_last={eh:.3e}")
    assert ey <= TOL_F32 and eh <= TOL_F32