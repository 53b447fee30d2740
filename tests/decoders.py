"""Test-side readers of the HIP library's outputs (kept apart from the oracle, which only ever
receives the original inputs): FP4 E2M1 code values and the RHT32 + S2F6 decode."""
import numpy as np

# E2M1 magnitudes by code (bit 3 is the sign): the sixteen values the AREX article's section
# "转置打散分组,随机舍入保住期望值" lists
FP4_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def fp4_value(code: int) -> float:
    v = FP4_GRID[code & 7]
    return -v if code & 8 else v


def decode_s2f6_rows(codes, e8m0, mask: int):
    """D H (c 2^(e - 133)) / 32 per 32-chunk with the dense Sylvester matrix, fp64."""
    i = np.arange(32)
    Hm = np.array([[(-1.0) ** bin(a & b).count("1") for b in i] for a in i])
    D = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in i])
    codes = np.asarray(codes)
    R, C = codes.shape
    z = codes.astype(np.float64).reshape(R, C // 32, 32) * 2.0 ** (np.asarray(e8m0, np.float64) - 133)[..., None]
    return ((z @ Hm.T) / 32 * D).reshape(R, C)


def unblock(raw, rows: int, cols: int):
    """Row-major [rows x cols] bytes of a code matrix held in the backward's blocked operand
    layout: 1 KB blocks of 16 rows x 64 bytes, block (rb, kb) at byte (rb * cols/64 + kb) * 1024,
    row r of a block at its bytes 64 r .. 64 r + 63 with the row's 16-byte chunk c at position
    c ^ ((r / 4) % 4)."""
    b = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8)).reshape(rows // 16, cols // 64, 16, 4, 16)
    r = np.arange(16)
    out = np.empty_like(b)
    for c in range(4):
        out[:, :, :, c, :] = b[:, :, r, c ^ ((r >> 2) & 3), :]
    return out.transpose(0, 2, 1, 3, 4).reshape(rows, cols)
