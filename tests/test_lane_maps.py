"""Lane mappings of the MFMA kernels, checked on a CPU model of the wave.

The forward flash kernel and the one-pass backward kernels move data between
lanes and registers with index expressions that the GPU parity tests exercise
only as a whole. Here each expression is re-stated from the kernel sources
(csrc/mfma_common.h, csrc/flash_common.h, csrc/kernel_bwd.hip) and run on
the model in wave64.py: the swizzled LDS tile fill, the MFMA operand reads,
the probability operand taken straight from the score accumulators, the
transposing V reads, the row statistics passed between lane layouts by
ds_bpermute, the lane-half reductions by v_permlane32_swap, the row dot
products read in the accumulator layout and the staged row stores. Each test
compares with plain matrix arithmetic on the same values.

A final group models forming a per-row dot product of accumulator rows with
operand registers by one lane-half swap (the form a discarded backward
variant used): it shows which result of the swap pairs with which
accumulator registers, and that the opposite pairing is wrong.
"""
import numpy as np
import pytest

import wave64 as w

RNG = np.random.default_rng(11)


# ---------------------------------------------------------------- kernel index expressions
def swz(D, r):
    if D == 128:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


def swoff(D, r, c):
    return r * D * 2 + 16 * (c ^ swz(D, r))


def acc_key(i, h):
    return 8 * (i >> 2) + 4 * h + (i & 3)


def bf16_round(x):
    """Round to bf16 (nearest even) and back, as the kernels' conversions."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def bf16_values(*shape):
    return bf16_round(RNG.standard_normal(shape))


def fill_tile(D, rows):
    """A 64-row swizzled tile filled as FlashOffsets::dma fills it: copy
    instruction i of wave wv moves rows 16 wv + RPI i + lane / CPR; lane l
    fetches global chunk (l % CPR) ^ swz(row) of its row and writes LDS bytes
    tile + (16 wv + RPI i) * ROWB + 16 l."""
    ROWB, CPR = 2 * D, D // 8
    RPI = 1024 // ROWB
    IPW = 64 // 4 // RPI
    lds = w.Lds(64 * ROWB)
    for wv in range(4):
        for i in range(IPW):
            for lane in range(64):
                row = 16 * wv + RPI * i + lane // CPR
                c = (lane % CPR) ^ swz(D, row)
                dst = (16 * wv + RPI * i) * ROWB + 16 * lane
                lds.write16(dst, rows[row, 8 * c: 8 * c + 8])
    return lds


def k_operand(lds, D, ks, t=0):
    """FlashOffsets::k: lane l reads 16 bytes at row r = l % 32 (+32 t), chunk (2 ks + h) ^ swz(r)."""
    out = np.empty((64, 8))
    for lane in range(64):
        r, h = lane & 31, lane >> 5
        off = r * 2 * D + 16 * ((2 * ks + h) ^ swz(D, r)) + t * 32 * 2 * D
        out[lane] = lds.read16(off, 8)
    return out


def qfrag(Q, ks):
    """load_qfrag: lane l holds row l % 32, channels 16 ks + 8 (l / 32) .. +8."""
    return np.stack([Q[lane % 32, 16 * ks + 8 * (lane // 32): 16 * ks + 8 * (lane // 32) + 8] for lane in range(64)])


def v_offsets(D):
    """FlashOffsets::v[mt][sec] (bytes, relative to the tile + 16 st rows)."""
    off = np.empty((D // 32, 2, 64), dtype=np.int64)
    for lane in range(64):
        j, g = lane & 15, lane >> 4
        for mt in range(D // 32):
            for sec in range(2):
                row = 4 * (g >> 1) + (j >> 2) + 8 * sec
                ch = 32 * mt + 16 * (g & 1) + 4 * (j & 3)
                off[mt, sec, lane] = row * 2 * D + 16 * ((ch // 8) ^ swz(D, row)) + (ch % 8) * 2
    return off


def v_operand(lds, D, mt, st):
    off = v_offsets(D) + st * 16 * 2 * D
    lo = w.ds_read_tr16_b64(lds, off[mt, 0])
    hi = w.ds_read_tr16_b64(lds, off[mt, 1])
    return np.concatenate([lo, hi], axis=1)


def p_operand(p, half):
    """p_operand: elements 8 half .. +8 of the accumulators, as a B operand."""
    return bf16_round(p[:, 8 * half: 8 * half + 8])


# ---------------------------------------------------------------- tests
@pytest.mark.parametrize("D", [64, 128])
def test_tile_fill_and_swizzled_reads(D):
    """Every chunk the tile copy writes is where swoff looks for it."""
    rows = bf16_values(64, D)
    lds = fill_tile(D, rows)
    for r in range(64):
        for c in range(D // 8):
            np.testing.assert_array_equal(lds.read16(swoff(D, r, c), 8), rows[r, 8 * c: 8 * c + 8])


@pytest.mark.parametrize("D", [64, 128])
def test_scores_transposed_layout(D):
    """S^T = K Q^T from K operands read out of the tile and Q fragments: register
    i of lane l holds <k_{acc_key(i, l / 32)}, q_{l % 32}> for both 32-key halves."""
    K, Q = bf16_values(64, D), bf16_values(32, D)
    lds = fill_tile(D, K)
    for t in range(2):
        s = np.zeros((64, 16))
        for ks in range(D // 16):
            s = w.mfma_32x32x16(k_operand(lds, D, ks, t), qfrag(Q, ks), s)
        want = K[32 * t: 32 * t + 32] @ Q.T
        for lane in range(64):
            for i in range(16):
                assert s[lane, i] == pytest.approx(want[acc_key(i, lane >> 5), lane & 31], rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("D", [64, 128])
def test_probability_operand_meets_transposed_v(D):
    """O^T = V^T P^T with P^T taken straight from score accumulators (p_operand)
    and V^T gathered by transposing reads (v_operand): the key order inside each
    16-key step is permuted the same way on both sides."""
    V = bf16_values(64, D)
    lds = fill_tile(D, V)
    P = RNG.random((32, 32))                  # [query, key] within one 32-key half
    p_acc = w.matrix_to_acc(P.T)              # accumulators of P^T: rows keys, columns queries
    for mt in range(D // 32):
        o = np.zeros((64, 16))
        for st in range(2):
            o = w.mfma_32x32x16(v_operand(lds, D, mt, st), p_operand(p_acc, st), o)
        want = (bf16_round(P) @ V[:32]).T[32 * mt: 32 * mt + 32]
        np.testing.assert_allclose(w.acc_to_matrix(o), want, rtol=1e-12, atol=1e-12)


def test_halves_reductions():
    """halves_sum / halves_max: the swap of a register with itself gives every
    lane the value of its partner in the other half."""
    x = RNG.standard_normal(64)
    r0, r1 = w.permlane32_swap(x, x)
    partner = x[np.arange(64) ^ 32]
    np.testing.assert_array_equal(r0 + r1, x + partner)
    np.testing.assert_array_equal(np.maximum(r0, r1), np.maximum(x, partner))


def test_bwd_small_statistics_handoff():
    """bwd_small: phase (a) leaves query r's lse and delta in lanes r and r + 32;
    phase (b) needs them per accumulator register i, whose query is
    acc_key(i, h) (S = Q K^T there), through ds_bpermute at 4 acc_key(i, h)."""
    stat = RNG.standard_normal(32)
    q_lse = stat[np.arange(64) & 31]
    # query row of each accumulator register, from the MFMA output layout itself
    query = w.matrix_to_acc(np.repeat(np.arange(32.0)[:, None], 32, axis=1)).astype(int)
    for i in range(16):
        src = np.array([4 * acc_key(i, lane >> 5) for lane in range(64)])
        got = w.ds_bpermute(src, q_lse)
        np.testing.assert_array_equal(got, stat[query[:, i]])


@pytest.mark.parametrize("D", [64, 128])
def test_row_dot_in_accumulator_layout(D):
    """row_dot_acc + halves_sum: lane l's dot product of its row (key l % 32) of
    dV, held as dV^T accumulators, with the same row of V in the swizzled tile."""
    V = bf16_values(64, D)
    lds = fill_tile(D, V)
    dV = RNG.standard_normal((32, D))
    acc = [w.matrix_to_acc(dV.T[32 * mt: 32 * mt + 32]) for mt in range(D // 32)]
    part = np.zeros(64)
    for lane in range(64):
        r, h = lane & 31, lane >> 5
        for mt in range(D // 32):
            for g in range(4):
                wv = lds.read16(r * 2 * D + 16 * ((4 * mt + g) ^ swz(D, r)) + 8 * h, 4)
                for e in range(4):
                    part[lane] += bf16_round(acc[mt][lane, 4 * g + e]) * wv[e]
    r0, r1 = w.permlane32_swap(part, part)
    got = r0 + r1
    want = (bf16_round(dV) * V[:32]).sum(axis=1)
    np.testing.assert_allclose(got, want[np.arange(64) & 31], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("f32", [True, False])
def test_staged_row_stores(D, f32):
    """stage_rows: x^T accumulators written into the dead tiles and read back
    16 bytes per lane come out as row-major rows (fp32: t0 rows 0..15, t1 rows
    16..31, chunk c of row r at c ^ (r % 16); bf16: one tile in the swizzle)."""
    X = RNG.standard_normal((32, D))
    acc = [w.matrix_to_acc(X.T[32 * mt: 32 * mt + 32]) for mt in range(D // 32)]
    out = np.full((32, D), np.nan)
    if f32:
        RB, CH = 4 * D, D // 4
        RPI = 64 // CH
        t = [w.Lds(16 * RB), w.Lds(16 * RB)]
        for lane in range(64):
            r, h = lane & 31, lane >> 5
            rr = r & 15
            for mt in range(D // 32):
                for g in range(4):
                    t[r >= 16].write32(rr * RB + 16 * ((8 * mt + 2 * g + h) ^ rr), acc[mt][lane, 4 * g: 4 * g + 4])
        for i in range(32 // RPI):
            for lane in range(64):
                row, chk = RPI * i + lane // CH, lane % CH
                out[row, 4 * chk: 4 * chk + 4] = t[row >= 16].read32((row & 15) * RB + 16 * (chk ^ (row & 15)), 4)
        np.testing.assert_array_equal(out, X)
    else:
        CPR = D // 8
        RPI = 64 // CPR
        t0 = w.Lds(64 * 2 * D)
        for lane in range(64):
            r, h = lane & 31, lane >> 5
            for mt in range(D // 32):
                for g in range(4):
                    t0.write16(swoff(D, r, 4 * mt + g) + 8 * h, bf16_round(acc[mt][lane, 4 * g: 4 * g + 4]))
        for i in range(32 // RPI):
            for lane in range(64):
                row, chk = RPI * i + lane // CPR, lane % CPR
                out[row, 8 * chk: 8 * chk + 8] = t0.read16(swoff(D, row, chk), 8)
        np.testing.assert_array_equal(out, bf16_round(X))


def test_output_store_channels():
    """store_out: lane l writes, for tile mt and group g, channels
    32 mt + 8 g + 4 h .. +4 of row l % 32 from registers 4 g .. +4."""
    D = 128
    X = RNG.standard_normal((32, D))
    acc = [w.matrix_to_acc(X.T[32 * mt: 32 * mt + 32]) for mt in range(D // 32)]
    out = np.full((32, D), np.nan)
    for lane in range(64):
        h = lane >> 5
        for mt in range(D // 32):
            for g in range(4):
                c0 = 32 * mt + 8 * g + 4 * h
                out[lane & 31, c0: c0 + 4] = acc[mt][lane, 4 * g: 4 * g + 4]
    np.testing.assert_array_equal(out, X)


# ---------------------------------------------------------------- one-swap row dots
def _swap_row_dot(D, pairing):
    """Row dots of dV (as dV^T accumulators, lane = key l % 32) with V held as
    B-operand registers of the same lane (V row l % 32, channels
    16 ks + 8 h + e), the partner half's channels brought over by one
    permlane32_swap per register pair: the swap of (elements e, elements 4 + e)
    of step ks = 2 mt + u yields the channels of accumulator group g = 2 u in
    its first result and g = 2 u + 1 in its second (`pairing` "isa"), or the
    other way round ("reversed")."""
    V = bf16_values(32, D)
    dV = bf16_values(32, D)
    acc = [w.matrix_to_acc(dV.T[32 * mt: 32 * mt + 32]) for mt in range(D // 32)]
    vf = [np.stack([V[lane & 31, 16 * ks + 8 * (lane >> 5): 16 * ks + 8 * (lane >> 5) + 8] for lane in range(64)])
          for ks in range(D // 16)]
    part = np.zeros(64)
    for mt in range(D // 32):
        for u in range(2):
            reg = vf[2 * mt + u]
            for e in range(4):
                first, second = w.permlane32_swap(reg[:, e], reg[:, 4 + e])
                g_first, g_second = (2 * u, 2 * u + 1) if pairing == "isa" else (2 * u + 1, 2 * u)
                part += acc[mt][:, 4 * g_first + e] * first + acc[mt][:, 4 * g_second + e] * second
    r0, r1 = w.permlane32_swap(part, part)
    return r0 + r1, (dV * V).sum(axis=1)[np.arange(64) & 31]


@pytest.mark.parametrize("D", [64, 128])
def test_one_swap_row_dot_pairing(D):
    got, want = _swap_row_dot(D, "isa")
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    bad, want = _swap_row_dot(D, "reversed")
    assert np.linalg.norm(bad - want) > 0.3 * np.linalg.norm(want)
