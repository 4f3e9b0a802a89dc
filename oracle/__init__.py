"""CPU oracle for the packed low-bit weight GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may import
this package.  The product path (the HIP library and its Python binding) never calls
it and shares no code with it.

Every function is a plain, slow, obviously correct restatement of what the pages
define (see each docstring for the passage):

* binary weights  w = scale_g * b,  b in {-1, +1}, one fp16 scale per group of
  consecutive weights  ("bonsai-image-binary-4B-gemlite-1bit" model card, section
  "Binary Weight Representation: 1-bit g128");
* ternary weights {-1, 0, +1} in 2 bits, consumed by a 2-bit quantised matmul
  ("Prism Bonsai ternary 2-bit image path in mlx-vlm" guide, sections
  "运行前提" (prerequisites) and "组件架构" (component architecture));
* weights stored as packed uint32 words plus scales ("backend/ -- FastAPI Mac backend",
  section "Checkpoint layout": transformer-packed-mflux holds uint32 packed weights +
  scales);
* other runtimes' ternary packs: GemLite's int2 weights, uint8 packed over K with a
  transpose, (in_features / 4, out_features) (Bonsai-Image-Demo pull request 20, "CPU
  bring-up"), and MLX's packed uint32 rows (the "Checkpoint layout" section above);
* the 4-bit text encoder: loaded quantised at bits = 4, group_size = 64 (the mlx guide,
  section "组件架构"), dequantised through HQQ on the CPU (pull request 20); its groups are
  read as affine, w = s * q + b (reading R10 of `oracle.lowbit_ref`);
* the reference computation is dequantise-to-dense followed by an ordinary matmul
  (Bonsai-Image-Demo pull request 20, "CPU image bring-up report": the validated CPU
  path runs the unpacked dense transformer).

Readings where the pages are silent (bit encoding, word order, scale form) are listed
in the module docstring of `oracle.lowbit_ref`.

Parity status: every function here is pinned by tests/test_oracle.py (golden words,
brute-force bit strings, math.fsum dot products, closed forms, a library matmul).
"""
from .lowbit_ref import (  # noqa: F401
    TERNARY, BINARY, INT4,
    bf16_bits_to_f64, f64_to_bf16_bits_rne,
    pack, unpack, dequant_f64, gemm_ref_f64, gemm_ref_from_words, gemm_fsum_element,
    silu_f64, swiglu_ref_f64, residual_ref_f64,
    gemlite_u8t_decode, gemlite_u8t_encode, mlx_u32_decode, mlx_u32_encode,
    gemlite_binary_decode, gemlite_binary_encode,
    pack_u4, unpack_u4, dequant_affine_f64, gemm_affine_ref_f64, gemm_affine_fsum_element,
    check_tolerance, REL_FROB_TOL, ELEM_TOL,
)
