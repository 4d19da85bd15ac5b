"""One grouped GEMM over expert segments, in float64 (the group_gemm_same_nk step).

Test infrastructure only (see ``oracle/__init__``).

For expert e and rows p in [offsets[e], offsets[e+1]):  C[p] = A[p] . B[e]^T.
With the SiLU*up epilogue (LlamaFactory PR #10481 write-up, section 1, the
SiLU(fc1_1) * fc1_2 step) B's rows [0, N/2) are gate and [N/2, N) up and
C = silu(gate) * up.  Rows at or past offsets[E] are zero (transformers PR
#45621 write-up, section 3: sentinel outputs must be written).

fp8 operands are block-scaled e4m3 (A: one scale per row and 128 columns,
B: one per 128x128 block); the product is that of the dequantised operands.
With ``out_fp8`` the rows are quantised per 128 columns from their float32
values (codes, scales) and also returned dequantised.
"""

from __future__ import annotations

import numpy as np

from .layer import dequant128, dequant_blocks, quant128, silu


def grouped_gemm(A, B, offsets, epilogue: str = "none", a_scales=None, b_scales=None,
                 out_fp8: bool = False):
    A = np.asarray(A)
    B = np.asarray(B)
    E, N, K = B.shape
    M = A.shape[0]
    fp8 = a_scales is not None
    n_out = N // 2 if epilogue == "silu_mul" else N
    C = np.zeros((M, n_out), dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if a == b:
            continue
        if fp8:
            Ae = dequant128(A[a:b], np.asarray(a_scales)[a:b])
            Be = dequant_blocks(B[e], np.asarray(b_scales)[e])
        else:
            Ae = A[a:b].astype(np.float64)
            Be = B[e].astype(np.float64)
        acc = Ae @ Be.T
        if epilogue == "silu_mul":
            acc = silu(acc[:, :n_out]) * acc[:, n_out:]
        C[a:b] = acc
    if not out_fp8:
        return C
    q, s = quant128(C.astype(np.float32))
    V = int(off[E])
    q[V:] = 0
    s[V:] = 1.0
    return dequant128(q, s), q, s
