"""CPU oracle for the PATCH hybrid tile-sparse GEMM -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``sparse_gemm_amd``) never imports it and shares no code with
it.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc); this module
only marshals numpy arrays to it.  See ``oracle.c`` for what each function
computes and which passage of the pages it follows.
"""
from .oracle import (  # noqa: F401
    F16, BF16, OracleError, build, lib_path, load, validate, effective_mask, gemm_f64, packed_bytes, pack,
    round_f64, f16_to_double, bf16_to_double, num_threads, silu, swiglu_f64, interleave_gate_up, PATTERN_PAIRS,
    gumbel, gumbel_softmax, sample_mask, exec_map, apply_fine_mask, packed_bytes_q64, pack_q64,
)
