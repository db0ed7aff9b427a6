"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Bar: dequantised weights bit-exact (fp32 of the oracle's exact fp64 weight,
NaN == NaN); GEMV outputs |y - y_ref| <= 1e-3 * sum_i |x_i w_i| + 1e-5 per row.
Inputs come from the seeded generators only.  Shapes span several K-chunks
and row groups with ragged tails, the full Llama-8B decode shapes, and the
degenerate cases (one row, one block, empty).
"""
import numpy as np
import pytest
import torch

import oracle
from dequant_gemv_amd import synth

pytestmark = pytest.mark.gpu

RTOL = 1e-3
ATOL = 1e-5
DEV = "cuda:0"


@pytest.fixture(scope="module")
def q():
    from dequant_gemv_amd import qgemv

    return qgemv


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _x_dev(x):
    return torch.from_numpy(x.view(np.int16).copy()).to(DEV)


def _run_gemv(q, fmt, w, x, n, k, stream=None):
    wd, xd = _dev(w), _x_dev(x)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    q.GEMV[fmt](wd, xd, y, n, k, stream)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def _assert_close(fmt, n, k, y, yr, ar, rows=None):
    err = np.abs(y - yr)
    bound = RTOL * ar + ATOL
    bad = np.flatnonzero(~(err <= bound))
    assert bad.size == 0, (
        f"{fmt} {n}x{k}: {bad.size} rows out of tolerance, e.g. row "
        f"{(rows[bad[0]] if rows is not None else bad[0])}: gpu {y[bad[0]]!r} ref {yr[bad[0]]!r} bound {bound[bad[0]]!r}")


def _check_gemv(q, fmt, n, k, seed, sample=None):
    w = synth.weights(fmt, n, k, synth.W_SEED + seed)
    x = synth.activations(fmt, k, synth.X_SEED + seed)
    y = _run_gemv(q, fmt, w, x, n, k)
    rows = None
    if sample is not None and sample < n:
        rng = np.random.default_rng(seed)
        rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, sample)]))
        yr, ar = oracle.gemv(fmt, w, x, n, k, rows=rows)
        y = y[rows]
    else:
        yr, ar = oracle.gemv(fmt, w, x, n, k)
    _assert_close(fmt, n, k, y, yr, ar, rows)
    return y


def _check_dequant(q, fmt, n, k, w):
    out = torch.full((n, k), float("nan"), dtype=torch.float32, device=DEV)
    q.DEQUANT[fmt](_dev(w), out, n, k)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle.dequant(fmt, w, n, k).astype(np.float32)
    gb, wb = got.view(np.uint32), want.view(np.uint32)
    same = (gb == wb) | (np.isnan(got) & np.isnan(want))
    if not same.all():
        i = np.argwhere(~same)[0]
        pytest.fail(f"{fmt} dequant {n}x{k}: {int((~same).sum())} mismatches, first at {tuple(i)}: "
                    f"gpu {got[tuple(i)]!r} oracle {want[tuple(i)]!r}")


# ---- dequantisation: bit-exact ------------------------------------------------

@pytest.mark.parametrize("fmt,n,k", [
    ("q4k", 1, 256), ("q4k", 37, 2304), ("q4k", 300, 4096),
    ("nvfp4", 1, 32), ("nvfp4", 37, 2080), ("nvfp4", 300, 4096),
    ("tq1", 1, 256), ("tq1", 37, 4352), ("tq1", 304, 256),
])
def test_dequant_bit_exact(q, fmt, n, k):
    _check_dequant(q, fmt, n, k, synth.weights(fmt, n, k, 50 + n + k))


def test_dequant_q4k_extreme_bytes(q):
    # every byte of the block random, including d/dmin: subnormal, negative,
    # Inf and NaN fp16 values all occur
    rng = np.random.default_rng(9)
    w = rng.integers(0, 256, (64, 16 * 144), dtype=np.uint8)
    _check_dequant(q, "q4k", 64, 4096, w)


def test_dequant_nvfp4_all_scale_codes(q):
    # every E4M3 code (NaN and negative ones included) and every nibble
    n, k = 16, 512
    rng = np.random.default_rng(10)
    nib = rng.integers(0, 256, n * k // 2, dtype=np.uint8)
    sc = np.arange(n * k // 16, dtype=np.int64).astype(np.uint8)
    _check_dequant(q, "nvfp4", n, k, np.concatenate([nib, sc]))


def test_dequant_tq1_all_bytes_every_position(q):
    # 304 blocks (77,824 elements): every byte value, the 13 non-codes, 0 and
    # 255 included, at every payload position; random fp16 d of both signs
    nblk = 304
    rng = np.random.default_rng(8)
    blk = np.empty((nblk, 54), np.uint8)
    for pos in range(52):
        blk[:, pos] = np.concatenate([np.arange(256), rng.integers(0, 256, nblk - 256)])[rng.permutation(nblk)]
    blk[:, 52:54] = rng.uniform(-5e-2, 5e-2, nblk).astype(np.float16).view(np.uint8).reshape(nblk, 2)
    _check_dequant(q, "tq1", 19, 16 * 256, blk.reshape(19, -1))


# ---- GEMV: tolerance ------------------------------------------------------------

SMALL = [
    # (fmt, n, k): several K-chunks, row groups and ragged tails
    ("q4k", 1, 256), ("q4k", 5, 512), ("q4k", 37, 2304), ("q4k", 129, 4096), ("q4k", 77, 14336),
    ("q4k", 300, 18432), ("q4k", 65, 36864),
    # row-streaming Q4_K: ragged last K-chunk at 7 chunks, 2 / 4 / 8 rows per wave
    ("q4k", 300, 13056), ("q4k", 1500, 14336), ("q4k", 1500, 2304), ("q4k", 3000, 3328), ("q4k", 5000, 4096), ("q4k", 16000, 2560),
    ("nvfp4", 1, 32), ("nvfp4", 3, 96), ("nvfp4", 37, 2080), ("nvfp4", 129, 4096), ("nvfp4", 77, 14336),
    ("nvfp4", 65, 36896),
    ("tq1", 1, 256), ("tq1", 5, 768), ("tq1", 37, 4352), ("tq1", 129, 4096), ("tq1", 77, 14336),
    ("tq1", 33, 41216),
]


@pytest.mark.parametrize("fmt,n,k", SMALL)
def test_gemv_small(q, fmt, n, k):
    _check_gemv(q, fmt, n, k, seed=n + k)


# Every rows-per-wave / waves-per-workgroup choice of the row-streaming
# kernels (the shape decides it), with ragged last workgroups.
ROW_STREAM = [(fmt, n, k) for fmt in ("nvfp4", "tq1") for n, k in (
    (1500, 4096), (3000, 4096), (5000, 4096), (14336, 4096), (16000, 4096))] + [
    ("nvfp4", 1500, 14336), ("nvfp4", 5000, 14336)] + [
    # every K-chunk count up to 8 (K <= 16384), ragged last chunks, and N past
    # one round of workgroups
    ("q4k", 2500, 256), ("q4k", 700, 1280), ("q4k", 20000, 2048), ("q4k", 3000, 5120),
    ("q4k", 1100, 8192), ("q4k", 300, 11008), ("q4k", 2100, 12288), ("q4k", 1500, 16384),
    ("q4k", 5000, 16384), ("q4k", 4500, 10240),
    ("nvfp4", 2100, 96), ("nvfp4", 1100, 1056), ("nvfp4", 3000, 5120), ("nvfp4", 5000, 12288),
    ("nvfp4", 700, 16384), ("nvfp4", 2200, 10272), ("nvfp4", 1500, 6176),
    ("tq1", 700, 2048), ("tq1", 2100, 2048), ("tq1", 3000, 6144), ("tq1", 5000, 8192),
]


@pytest.mark.parametrize("fmt,n,k", ROW_STREAM)
def test_gemv_row_stream_shapes(q, fmt, n, k):
    _check_gemv(q, fmt, n, k, seed=7 * n + k, sample=1500)


FULL = [
    # the decode shapes: Q4_K 4096x4096, Q4_K gate/up 14336x4096 and down
    # 4096x14336, NVFP4 4096x14336, TQ1_0 14336x4096; every row checked
    ("q4k", 4096, 4096, 0), ("q4k", 14336, 4096, 1), ("q4k", 4096, 14336, 1),
    ("nvfp4", 4096, 14336, 2), ("tq1", 14336, 4096, 3),
    # Llama-8B attention K/V projection and lm_head rows
    ("q4k", 1024, 4096, 4), ("nvfp4", 1024, 4096, 4), ("tq1", 1024, 4096, 4),
    # the concatenated Q/K/V and gate/up matrices of the fused decode sweep
    ("q4k", 6144, 4096, 5), ("tq1", 28672, 4096, 5),
]


@pytest.mark.parametrize("fmt,n,k,case", FULL)
def test_gemv_full_shapes(q, fmt, n, k, case):
    _check_gemv(q, fmt, n, k, seed=case)


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1"])
def test_gemv_max_k(q, fmt):
    # the largest K the calls accept (2^24: 16.8 M weights per row, a 32 MB x)
    _check_gemv(q, fmt, 3, 1 << 24, seed=90)


@pytest.mark.parametrize("fmt,k", [("q4k", 256), ("nvfp4", 64), ("tq1", 256)])
def test_gemv_twenty_million_rows(q, fmt, k):
    # M = 20,000,003 (grids past 2^24 rows, a ragged last workgroup): the rows
    # repeat a random block of 4099 rows (a period that no power-of-two index
    # mistake preserves); 3000 sampled rows plus the first and last
    n, period = 20_000_003, 4099
    base = synth.weights(fmt, period, k, synth.W_SEED + 95)
    if fmt == "nvfp4":  # nibbles [M][K/2], then scales [M][K/16]
        nib, sc = base[:period * k // 2].reshape(period, k // 2), base[period * k // 2:].reshape(period, k // 16)
        reps = (n + period - 1) // period
        w = np.concatenate([np.tile(nib, (reps, 1))[:n].ravel(), np.tile(sc, (reps, 1))[:n].ravel()])
    else:
        w = np.tile(base.reshape(period, -1), ((n + period - 1) // period, 1))[:n].ravel()
    x = synth.activations(fmt, k, synth.X_SEED + 95)
    y = _run_gemv(q, fmt, w, x, n, k)
    rng = np.random.default_rng(95)
    rows = np.unique(np.concatenate([[0, 1, (1 << 24) - 1, 1 << 24, n - 2, n - 1], rng.integers(0, n, 3000)]))
    yr, ar = oracle.gemv(fmt, w, x, n, k, rows=rows)
    _assert_close(fmt, n, k, y[rows], yr, ar, rows)


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1"])
def test_gemv_lm_head_sampled(q, fmt):
    # 128256 x 4096: 2,048 sampled rows plus the first and last
    _check_gemv(q, fmt, 128256, 4096, seed=4, sample=2048)


@pytest.mark.parametrize("fmt", ["q4k", "nvfp4", "tq1"])
def test_gemv_deterministic_and_on_side_stream(q, fmt):
    n, k = 1000, 4096
    w = synth.weights(fmt, n, k, 61)
    x = synth.activations(fmt, k, 62)
    y0 = _run_gemv(q, fmt, w, x, n, k)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = _run_gemv(q, fmt, w, x, n, k, stream=s)
    assert np.array_equal(y0.view(np.uint64), y1.view(np.uint64))


def test_gemv_concurrent_host_threads(q):
    # the calls keep no global mutable state: four host threads, each with its
    # own stream, format and buffers, enqueue 20 calls at once
    import threading

    cases = [("q4k", 3000, 4096), ("nvfp4", 2000, 14336), ("tq1", 5000, 4096), ("q4k", 777, 36864)]
    data = []
    for i, (fmt, n, k) in enumerate(cases):
        w = synth.weights(fmt, n, k, synth.W_SEED + 400 + i)
        x = synth.activations(fmt, k, synth.X_SEED + 400 + i)
        ref = _run_gemv(q, fmt, w, x, n, k)  # one call alone, checked against the oracle
        yr, ar = oracle.gemv(fmt, w, x, n, k)
        _assert_close(fmt, n, k, ref, yr, ar)
        data.append((fmt, n, k, _dev(w), _x_dev(x), ref))
    outs = [[] for _ in cases]
    errors = []

    def work(j):
        try:
            fmt, n, k, wd, xd, _ = data[j]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(20):
                    y = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
                    q.GEMV[fmt](wd, xd, y, n, k, s)
                    outs[j].append(y)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(j,)) for j in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for j, (fmt, n, k, _, _, ref) in enumerate(data):
        assert len(outs[j]) == 20
        for y in outs[j]:
            assert np.array_equal(y.cpu().numpy().astype(np.float64), ref), (fmt, n, k)


def test_gemv_empty_is_noop(q):
    y = torch.full((4,), 7.0, device=DEV)
    w = torch.zeros(144, dtype=torch.uint8, device=DEV)
    x = torch.zeros(256, dtype=torch.int16, device=DEV)
    q.qgemv_q4k(w, x, y, 0, 256)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_gemv_writes_only_m_outputs(q):
    n, k = 37, 512
    w = synth.weights("q4k", n, k, 63)
    x = synth.activations("q4k", k, 64)
    y = torch.full((n + 64,), 7.0, device=DEV)
    q.qgemv_q4k(_dev(w), _x_dev(x), y, n, k)
    torch.cuda.synchronize()
    assert torch.all(y[n:] == 7.0)


def test_nvfp4_nan_scale_poisons_only_its_row(q):
    n, k = 9, 4096
    w = synth.weights("nvfp4", n, k, 65)
    x = synth.activations("nvfp4", k, 66)
    w[n * k // 2 + 3 * (k // 16) + 17] = 0x7F  # NaN scale in row 3
    y = _run_gemv(q, "nvfp4", w, x, n, k)
    yr, ar = oracle.gemv("nvfp4", w, x, n, k)
    assert np.isnan(y[3]) and np.isnan(yr[3])
    keep = np.arange(n) != 3
    _assert_close("nvfp4", n, k, y[keep], yr[keep], ar[keep])


# A NaN block scale poisons its own row and no other, through every GEMV
# kernel family: the small-shape kernels, the row-streaming kernels, and for
# TQ1_0 the table-driven one (K = 4096, more than 1024 rows).  fp16 0x7E00
# is a quiet NaN; the byte offsets are the block's d (Q4_K: d at 0, dmin at
# 2; TQ1_0: d at 52).
NAN_D_CASES = [
    ("q4k", 9, 4096, 0), ("q4k", 2100, 4096, 0), ("q4k", 2100, 4096, 2),
    ("tq1", 9, 4096, 52), ("tq1", 2100, 4096, 52), ("tq1", 3001, 8192, 52),
]


@pytest.mark.parametrize("fmt,n,k,field", NAN_D_CASES)
def test_nan_block_scale_poisons_only_its_row(q, fmt, n, k, field):
    w = synth.weights(fmt, n, k, 67 + n % 7)
    x = synth.activations(fmt, k, 68)
    bsz = 144 if fmt == "q4k" else 54
    row, blk = n // 2 + 1, (k // 256) // 2 + 1
    off = (row * (k // 256) + blk) * bsz + field
    flat = w.reshape(-1)  # a view: the rows are contiguous
    flat[off], flat[off + 1] = 0x00, 0x7E
    y = _run_gemv(q, fmt, w, x, n, k)
    yr, ar = oracle.gemv(fmt, w, x, n, k)
    assert np.isnan(y[row]) and np.isnan(yr[row])
    keep = np.arange(n) != row
    _assert_close(fmt, n, k, y[keep], yr[keep], ar[keep])


# TQ1_0 payload bytes drawn uniformly over all 256 values (the encoder only
# makes 243 of them, 81 for qh), so every entry of the table-driven kernel's
# digit table and every byte value of the arithmetic digits is exercised;
# d stays a finite fp16.
@pytest.mark.parametrize("n,k", [(9, 4096), (2100, 4096), (14336, 4096)])
def test_tq1_gemv_every_byte_value(q, n, k):
    rng = np.random.default_rng(69 + n)
    w = rng.integers(0, 256, size=(n, (k // 256) * 54), dtype=np.uint8)
    d = rng.uniform(1e-2, 5e-2, size=(n, k // 256)).astype(np.float16)
    blocks = w.reshape(n, k // 256, 54)
    blocks[:, :, 52:54] = d.view(np.uint8).reshape(n, k // 256, 2)
    x = synth.activations("tq1", k, 70)
    y = _run_gemv(q, "tq1", w, x, n, k)
    yr, ar = oracle.gemv("tq1", w, x, n, k)
    _assert_close("tq1", n, k, y, yr, ar)


def test_read_ceiling_folds_every_byte(q):
    nbytes = 3 * 32768 + 4096  # ragged last workgroup
    rng = np.random.default_rng(12)
    buf = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    sink = torch.zeros(q.qgemv_read_sink_len(nbytes), dtype=torch.float32, device=DEV)
    q.qgemv_read_ceiling(_dev(buf.view(np.uint8)), nbytes, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(buf)


def test_build_id_is_current(q):
    from dequant_gemv_amd import build

    assert q.qgemv_build_id() == build.build_id()
