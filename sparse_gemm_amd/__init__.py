"""MI355X-native hybrid tile-sparse GEMM (PATCH inference hot path).

    from sparse_gemm_amd import patch
    pw = patch.pack(W, tile_map, mask)   # dense W + tile map + 2:4 mask -> blob
    Y = patch.gemm(X, pw)                # Y = X (W o E)^T on the GPU
    Yd = patch.dense_gemm(X, W)          # same-shape dense baseline

``inputs`` draws seeded synthetic data; ``build`` compiles libpatch.so.
"""
