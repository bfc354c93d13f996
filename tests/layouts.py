"""Test-side readers of the library's workspace layouts (numpy only).

The packed operand layout of the bf16 activations (modulated LayerNorm
output h and the attention / SwiGLU concatenation): a row-major [R][K]
matrix is stored as 1-KiB blocks of 8 rows x 64 k-values, block (r // 8,
k // 64) at block index (r // 8) * (K // 64) + k // 64; inside a block row
r % 8 takes 64 values whose 8-value chunks are permuted, chunk c in slot
c ^ ((r // 2) % 8).
"""
import numpy as np


def unpack_rows(p, R, K):
    """Row-major [R][K] view of a packed matrix given as R*K elements."""
    a = np.asarray(p).reshape(R // 8, K // 64, 8, 8, 8)          # rb, kb, r8, slot, e
    b = a.transpose(0, 2, 1, 3, 4).reshape(R, K // 64, 8, 8)      # row, kb, slot, e
    rows = np.arange(R)
    slot = np.arange(8)[None, :] ^ ((rows >> 1) & 7)[:, None]     # slot of chunk c, [R][8]
    out = np.take_along_axis(b, slot[:, None, :, None], axis=2)
    return out.reshape(R, K)


def unpack8_rows(p, R, K):
    """Row-major [R][K] uint8 codes of a packed fp8 matrix given as R*K
    bytes: its bytes sit where a packed bf16 [R][K / 2] matrix's would."""
    pairs = np.ascontiguousarray(np.asarray(p, np.uint8)).view(np.uint16)
    return np.ascontiguousarray(unpack_rows(pairs, R, K // 2)).view(np.uint8).reshape(R, K)


def pack8_rows_loops(x):
    """Packed fp8 layout by explicit loops, from its definition: 1-KiB
    blocks of 8 rows x 128 codes, block (r / 8, k / 128) at index
    (r / 8)(K / 128) + k / 128, row r % 8 at byte 128 (r % 8) of it, 16-byte
    chunk c in slot c ^ ((r / 2) % 8)."""
    R, K = x.shape
    out = np.zeros(R * K, dtype=np.uint8)
    for r in range(R):
        for k in range(K):
            blk = (r // 8) * (K // 128) + k // 128
            c = (k % 128) // 16
            slot = c ^ ((r // 2) % 8)
            out[blk * 1024 + (r % 8) * 128 + slot * 16 + k % 16] = x[r, k]
    return out


def pack_rows_loops(x):
    """Reference packer written with explicit loops (small matrices only)."""
    R, K = x.shape
    out = np.zeros(R * K, dtype=x.dtype)
    for r in range(R):
        for k in range(K):
            blk = (r // 8) * (K // 64) + k // 64
            c = (k % 64) // 8
            slot = c ^ ((r // 2) % 8)
            out[blk * 512 + (r % 8) * 64 + slot * 8 + k % 8] = x[r, k]
    return out
