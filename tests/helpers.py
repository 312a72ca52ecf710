"""Small input constructors shared by the oracle pins and the GPU parity tests."""
import numpy as np

import synthetic as syn


def set_one_hot(case, j_star, col):
    """Make x_j[col] = 1 for token j_star and 0 for every other referenced token."""
    rows = case.kv_indices
    if case.kv_dtype == syn.KV_BF16:
        case.kv[rows, col] = 0
        case.kv[rows[j_star], col] = 0x3F80  # 1.0
    elif case.kv_dtype == syn.KV_FP8:
        case.kv_scales[0] = 1.0
        case.kv[rows, col] = 0
        case.kv[rows[j_star], col] = 0x38  # 1.0
    else:
        shift = 4 * (col & 1)
        keep = np.uint8(0xF0 >> shift)
        case.kv[rows, col // 2] &= keep
        case.kv[rows[j_star], col // 2] |= np.uint8(0x2 << shift)  # e2m1 1.0
        case.kv_scales[rows[j_star], col // 32] = 127
