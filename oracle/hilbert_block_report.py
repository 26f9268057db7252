"""Empty / partial / full 64x64 blocks of token-level 2D attention patterns in
raster order and in Hilbert order (the claim of "Boosting 2D Local Attention
Efficiency with Hilbert-Guided Sparsity", "The Hilbert Curve Advantage").

CPU only, oracle functions only. Usage: python -m oracle.hilbert_block_report
"""

import numpy as np

from . import hilbert_oracle as H


def main() -> None:
    print("image  pattern            order    empty  partial  full  (64x64 blocks)")
    for side in (64, 128):
        perms = {"raster": np.arange(side * side), "hilbert": H.hilbert_token_order((side, side))}
        patterns = {
            "window 8x8": H.square_window_mask(side, 8),
            "window 16x16": H.square_window_mask(side, 16),
            "neighbourhood 7x7": H.neighborhood_mask(side, 3),
            "neighbourhood 15x15": H.neighborhood_mask(side, 7),
        }
        for name, mask in patterns.items():
            for order, perm in perms.items():
                c = H.block_counts(mask, perm)
                print(f"{side:3d}^2  {name:18s} {order:8s} {c['empty']:6d} {c['partial']:8d} {c['full']:5d}")


if __name__ == "__main__":
    main()
