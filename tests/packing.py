"""Byte-level builders for hand-made cache rows in tests (input construction only)."""

import numpy as np

IDX_ROW = 132
LAT_ROW = 656


def bf16_bits(x) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (inputs here are exact)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((f >> 16) & 1) + 0x7FFF
    return ((f + rounding) >> 16).astype(np.uint16)


def index_pool(num_blocks, block_size):
    return np.zeros((num_blocks, block_size, IDX_ROW), dtype=np.uint8)


def put_index_row(pool, slot, codes: dict, scale: float):
    flat = pool.reshape(-1, IDX_ROW)
    flat[slot, :128] = 0
    for d, c in codes.items():
        flat[slot, int(d)] = int(c, 16) if isinstance(c, str) else int(c)
    flat[slot, 128:132] = np.frombuffer(np.float32(scale).tobytes(), dtype=np.uint8)


def latent_pool(num_blocks, block_size):
    return np.zeros((num_blocks, block_size, LAT_ROW), dtype=np.uint8)


def put_latent_row(pool, slot, codes: dict, scales, rope=None):
    flat = pool.reshape(-1, LAT_ROW)
    flat[slot, :512] = 0
    for d, c in codes.items():
        flat[slot, int(d)] = int(c, 16) if isinstance(c, str) else int(c)
    flat[slot, 512:528] = np.frombuffer(np.asarray(scales, dtype="<f4").tobytes(), dtype=np.uint8)
    r = np.zeros(64, dtype=np.float32) if rope is None else np.asarray(rope, dtype=np.float32)
    flat[slot, 528:656] = np.frombuffer(bf16_bits(r).astype("<u2").tobytes(), dtype=np.uint8)
