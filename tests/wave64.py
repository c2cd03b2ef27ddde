"""CPU model of the gfx950 wave64 operations the MFMA kernels build on.

Test infrastructure: the lane-mapping tests drive it with the kernels' own
index expressions (re-stated in Python) and check that the pieces compose to
the intended matrix products and row statistics. Every function states the
definition it models; `tests/hip/lane_probe.hip` runs the same operations on
the GPU so that a GPU test can hold this model against the hardware.

Registers are numpy arrays whose first axis is the lane (64 lanes).
"""
import numpy as np

LANES = 64


def permlane32_swap(vdst, vsrc):
    """V_PERMLANE32_SWAP_B32 (CDNA4 ISA): lanes 32..63 of VDST trade places
    with lanes 0..31 of VSRC0; the other halves stay. Returns the new
    (VDST, VSRC0) pair: the compiler builtin's results 0 and 1, with its first
    argument in VDST and its second in VSRC0."""
    vdst, vsrc = np.asarray(vdst), np.asarray(vsrc)
    d, s = vdst.copy(), vsrc.copy()
    d[32:] = vsrc[:32]
    s[:32] = vdst[32:]
    return d, s


def ds_bpermute(addr, data):
    """DS_BPERMUTE_B32: lane l receives `data` of lane (addr[l] / 4) mod 64
    (addresses in bytes; every lane active)."""
    return np.asarray(data)[(np.asarray(addr, dtype=np.int64) >> 2) & 63]


# ---------------------------------------------------------------- matrix core
def mfma_32x32x16(a, b, c):
    """V_MFMA_F32_32X32X16_BF16 on lane registers (values as float64).

    a, b: [64, 8] operand registers, c: [64, 16] accumulators. Matrix view:
    A[i][k] = a[i + 32 * (k // 8)][k % 8], B[k][j] = b[j + 32 * (k // 8)][k % 8],
    C[r][j] = c[j + 32 * ((r // 4) % 2)][4 * (r // 8) + r % 4]; returns the
    accumulators of D = A B + C in the C layout."""
    A = np.empty((32, 16))
    B = np.empty((16, 32))
    for lane in range(LANES):
        for e in range(8):
            A[lane % 32, 8 * (lane // 32) + e] = a[lane, e]
            B[8 * (lane // 32) + e, lane % 32] = b[lane, e]
    D = A @ B + acc_to_matrix(c)
    return matrix_to_acc(D)


def acc_to_matrix(c):
    """32x32 matrix held by accumulator registers c[64, 16] (C/D layout)."""
    M = np.empty((32, 32))
    for lane in range(LANES):
        for i in range(16):
            M[8 * (i // 4) + 4 * (lane // 32) + i % 4, lane % 32] = c[lane, i]
    return M


def matrix_to_acc(M):
    c = np.empty((LANES, 16))
    for lane in range(LANES):
        for i in range(16):
            c[lane, i] = M[8 * (i // 4) + 4 * (lane // 32) + i % 4, lane % 32]
    return c


# ---------------------------------------------------------------- LDS
class Lds:
    """LDS as 16-bit elements (bf16 values stored as float64 for exact sums)
    plus fp32 views: addresses are bytes, as in the kernels."""

    def __init__(self, nbytes):
        self.h = np.full(nbytes // 2, np.nan)   # 16-bit element slots
        self.w = np.full(nbytes // 4, np.nan)   # 32-bit slots (fp32 staging)

    def write16(self, byte, values):
        assert byte % 2 == 0
        self.h[byte // 2: byte // 2 + len(values)] = values

    def read16(self, byte, n):
        assert byte % 2 == 0
        out = self.h[byte // 2: byte // 2 + n]
        assert len(out) == n
        return out.copy()

    def write32(self, byte, values):
        assert byte % 4 == 0
        self.w[byte // 4: byte // 4 + len(values)] = values

    def read32(self, byte, n):
        assert byte % 4 == 0
        out = self.w[byte // 4: byte // 4 + n]
        assert len(out) == n
        return out.copy()


def ds_read_tr16_b64(lds, addr):
    """DS_READ_B64_TR_B16 with the lane map measured on gfx950 (and held
    against the GPU by tests/hip/lane_probe.hip): inside each group of 16
    lanes, lane i receives, as its element e (e = 0..3), element i % 4 of the
    8-byte segment that lane 4 * e + i // 4 of the group addresses."""
    out = np.empty((LANES, 4))
    for lane in range(LANES):
        g, i = lane // 16, lane % 16
        for e in range(4):
            src = 16 * g + 4 * e + i // 4
            out[lane, e] = lds.read16(int(addr[src]), 4)[i % 4]
    return out
