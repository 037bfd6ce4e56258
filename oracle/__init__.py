"""CPU oracle for the quantized matrix-vector product (QMV).

TEST INFRASTRUCTURE ONLY. Nothing in the library's product path imports, calls,
links or executes anything in this package; only the test suite, the smoke
check and the benchmark's CPU-baseline leg may use it.

What it computes, in plain fp64 NumPy and from the definitions on the source
pages (no blocking, fusion or reordering beyond what the definition states):

    y[b, n] = sum_k x[b, k] * dequant(W)[n, k]

Sources (cited by page title and section; every function docstring names the
passage it follows):

* "wh-iron kernel-op coverage audit", section "Quantization precision
  coverage": the Track-1 format table (nvfp4 / mxfp4 / mxfp8_e4m3), the rule
  that sub-byte codes are packed LSB-first, Track 2 (affine w = scale*q + bias),
  the E2M1 codebook of the fp_quantized_nax row and the E4M3 constants of the
  kv_cache row of the op-coverage table, and the "Model-format decode" table
  (NaN sentinel kept explicit; DSv4 mxfp4 = OCP mxfp4).
* "mlx 1.0.0 - quantized_nax.h": `get_pack_factor` / `get_bytes_per_pack`
  (packed geometry), `dequantize` and `qdot` (bit masks of every width and the
  affine dot identity scale*sum(x*q) + bias*sum(x)), `adjust_matrix_offsets`
  (gather semantics: x row from lhs_indices, weight matrix from rhs_indices).
* "ml-explore/mlx pull request 4516": the bias term uses sum(x) with every
  element widened before accumulation; NVFP4 calls carry a global scale.
* "@lgrammel/ds4-provider - moe.metal": `kernel_mul_mv_id` (the routed expert
  of each slot picks the weight matrix; no per-expert host dispatch).
* "ferrum-kernels - primitives.rs" tests: an out-of-range index yields a row
  of zeros rather than a fault.
* The other Track-1 block-scaled formats (``blockfmt.py``): the audit's
  element x block x scale matrix (E5M2 constants from its kv_cache row).
* The fused routed-MoE decode block (``moe.py``): the ds4 moe.metal SwiGLU
  activation and per-token down-projection sum, and the audit's two-dispatch
  description of the block.
* RMSNorm in front of the QMV (``norm.py``): the audit's rms_norm and
  rms_norm_qgemv rows, with the readings its docstring states.
* Quantize-from-float (``quantize.py``): the audit's Track-2 min/max encoder
  and the fp_quantized / kv_cache rows' max-scale element rounding, with the
  readings its docstring states.

Pins that tie this oracle to something other than itself live in
``tests/test_oracle_pins.py`` (run with ``-m "not gpu"``).
"""

from .codes import (
    packed_row_bytes,
    unpack_codes,
    pack_codes,
    storage_to_f64,
    round_f64_to_bf16_bits,
    round_f64_to_f16,
    round_f64_to_f32,
    round_f64_to,
    ulp_of,
)
from .formats import (
    e2m1_value,
    e4m3_value,
    e8m0_value,
    e4m3_encode_nearest,
)
from .quantize import (
    e2m1_encode_nearest,
    floor_log2,
    quantize_affine,
    quantize_mx,
    quantize_nvfp4,
)
from .blockfmt import (
    e5m2_value,
    int_value,
    element_value,
    scale_value,
    implicit_factor,
    dequant_block,
    FORMATS as BLOCK_FORMATS,
    ELEMENTS as BLOCK_ELEMENTS,
)
from .moe import (
    silu,
    swiglu,
    gate_up_projections,
    moe_gate_up_swiglu,
    moe_down_reduce,
)
from .norm import (gamma_stored, rms_factor, rmsnorm, rmsnorm_qmv, rmsnorm_qmv_abs,
                   rmsnorm_stored)
from .qmv import (
    dequant_affine,
    dequant_mxfp4,
    dequant_nvfp4,
    dequant_mxfp8,
    dequant,
    qmv,
    qmv_rows,
    qvm,
    qvm_abs,
    gather_qmv,
    abs_dot,
)

__all__ = [
    "packed_row_bytes", "unpack_codes", "pack_codes", "storage_to_f64",
    "round_f64_to_bf16_bits", "round_f64_to_f16", "round_f64_to_f32",
    "round_f64_to", "ulp_of",
    "e2m1_value", "e4m3_value", "e8m0_value", "e4m3_encode_nearest",
    "dequant_affine", "dequant_mxfp4", "dequant_nvfp4", "dequant_mxfp8",
    "dequant", "qmv", "qmv_rows", "gather_qmv", "abs_dot",
]
