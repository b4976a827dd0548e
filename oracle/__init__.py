"""CPU oracle for the fp16 NT matrix product and the m8n8 fragment copy.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code, header, table or
constant with the HIP library under ``fp16_matrix_core_amd/csrc``; the two meet
only at the seeded input arrays that both consume.

Contents
  gemm   Out = A @ B.T for fp16 A (M,K), B (N,K): the plain definition in
         float64 (products of fp16 values are exact in float64), plus the
         per-element bound sum_k |A[i,k] * B[j,k]| that the parity test scales.
  general  the general product: bfloat16 operands (decoded from their bit
         patterns), operands stored with K indexing their rows, the output's
         previous values as the MMA's C operand, and the acceptance rule for
         float16 / bfloat16 outputs.
  frag   the bit-exact model of the warp-collective 8x8 matrix load/store
         (ldmatrix/stmatrix): shared image <-> per-lane register fragment, for
         num in {1, 2, 4} tiles, row- or column-major shared layouts.
  page1  the lane maps of the single-warp m16n8k16 example, evaluated as
         written, and a fragment-level simulation of that example; used only
         to pin ``gemm`` and ``frag`` to the pages.

Every function cites the passage of the pages it follows ("Warp Matrix
Instructions", "Blackwell Tensor Cores", "copy -> ldstmatrix").
"""

from .gemm import gemm_nt, gemm_nt_loops, gemm_nt_strided, gemm_nt_rows, gemm_nt_batched, within_bound  # noqa: F401
from .general import (  # noqa: F401
    bf16_to_f64, operand_f64, gemm_nt_ex, gemm_ex, gemm_ex_strided, half_ulp, within_bound_out,
)
from .frag import (  # noqa: F401
    register_layout, shared_layout, fit_shared_layout, image_index,
    frag_load, frag_store, frag_roundtrip,
)
