"""CPU oracle for the NVFP4 quantizer and NVFP4 GEMM.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously correct
definition of what the GPU library computes. Only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The GPU library never calls it, and it imports nothing from the GPU
library: the two share no code, tables or constants.

Sources. The method is described on three web pages that summarise NVIDIA's
report "Pretraining Large Language Models with NVFP4" (arXiv 2509.25149):

* gist.science, "Pretraining Large Language Models with NVFP4" -- the lay
  part "Lo esencial" and the "Resumen técnico" with sections 1-5; section 2
  ("Metodología Propuesta") has the sub-headings "Formato NVFP4",
  "Precisión Mixta Selectiva", "Transformadas de Hadamard Aleatorias (RHT)"
  and "Escalado Bidimensional (2D) y Redondeo Estocástico".
* deultimominuto.info, news article on the same report -- sections
  "El desafío de la cuantización", "Cómo funciona NVFP4".
* news.hamidun.com, "NVIDIA desarrolló un método para entrenar redes
  neuronales con precisión de 4-bit" -- section "Cómo Funciona".

The pages give the structure of the format (16-element blocks, E4M3 block
scale, FP32 tensor scale, 4-bit elements with 16 distinct values, a 16x16
Hadamard transform with a fixed random sign vector, 16x16 weight tiles,
stochastic rounding of gradients) but no formula, constant, rounding rule,
random generator or memory layout. Every such detail here is a reading of the
pages; each function says which one it takes.

Parity status of each function (what pins it, in ``tests/test_oracle_*.py``):

* formats.e2m1_*      -- pinned: 16-code closed form, significand rounding
                         via numpy's rint, exhaustive tie neighbourhoods.
* formats.e4m3_*      -- pinned: 256-byte decode by hand-written table rows,
                         torch.float8_e4m3fn cast below 464.
* philox.*            -- pinned: rocRAND's Philox4x32-10 engine (header
                         source compiled for the host) word for word.
* hadamard.*          -- pinned: scipy.linalg.hadamard, H H^T = 16 I,
                         norm preservation, inverse, single spike.
* quantize.*          -- pinned: hand-worked blocks (tests/golden), power-of-
                         two invariance, block-max code invariant, transpose
                         identities, SR counts over all 2^16 random words,
                         SR unbiasedness.
* gemm.*              -- pinned: pure-Python triple loop on tiny inputs,
                         all-ones closed form, unit-row selection.
* mx.*                -- pinned: E8M0 bytes against float32 exponent fields,
                         the [4, 8) scale invariant, a hand-worked block,
                         power-of-two invariance, a triple loop for the GEMM.
* fp8.*               -- pinned: torch.float8_e4m3fn cast below 448 (random
                         values and every midpoint neighbourhood), saturation
                         and signed zero by hand, tensor-scale closed forms,
                         exact E4M3 inputs, power-of-two invariance, a
                         triple loop and an all-ones GEMM.
"""

from .formats import (
    E2M1_MAGNITUDES,
    e2m1_decode,
    e2m1_encode_rn,
    e2m1_encode_sr,
    e4m3_decode,
    e4m3_encode,
)
from .fp8 import FP8_MAX, fp8_dequantize, fp8_encode, fp8_gemm, fp8_quantize, fp8_tensor_scale
from .mx import MX_BLOCK, e8m0_decode, mx_dequantize, mx_gemm, mx_quantize, mx_scale_bytes
from .philox import philox4x32_10, sr_random_u16
from .hadamard import hadamard16, rht_signs, rht
from .quantize import (
    QuantizedTensor,
    tensor_scale,
    quantize_rows,
    quantize,
    quantize_2d,
    rht_quantize,
    dequantize,
    pack_codes,
    unpack_codes,
)
from .gemm import gemm

__all__ = [
    "FP8_MAX",
    "fp8_dequantize",
    "fp8_encode",
    "fp8_gemm",
    "fp8_quantize",
    "fp8_tensor_scale",
    "MX_BLOCK",
    "e8m0_decode",
    "mx_dequantize",
    "mx_gemm",
    "mx_quantize",
    "mx_scale_bytes",
    "E2M1_MAGNITUDES",
    "e2m1_decode",
    "e2m1_encode_rn",
    "e2m1_encode_sr",
    "e4m3_decode",
    "e4m3_encode",
    "philox4x32_10",
    "sr_random_u16",
    "hadamard16",
    "rht_signs",
    "rht",
    "QuantizedTensor",
    "tensor_scale",
    "quantize_rows",
    "quantize",
    "quantize_2d",
    "rht_quantize",
    "dequantize",
    "pack_codes",
    "unpack_codes",
    "gemm",
]
