"""CPU oracle for the LoRA linear layer over a frozen block-quantized base.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything here.  The product
path (the HIP library and its Python binding) never imports, links or calls
this package, and this package imports nothing from the product path.

What it holds, each written from the definition it cites:

* ``codecs``  -- bf16 / fp16 / OCP E4M3FN encode and decode, value-based
  (round to nearest, ties to even), with no use of library casts.
* ``formats`` -- the NF4 code book (QLoRA paper, "4-bit NormalFloat"
  construction), and pack / dequant of the five base formats
  (Q4_0-style blocks of 32, NF4 blocks of 64, per-tensor FP8 E4M3, MXFP4
  blocks of 32 E2M1 codes with an E8M0 scale, Q8_0-style blocks of 32 int8
  codes with an fp16 scale).
* ``lora``    -- forward and backward of y = x.W^T + (alpha/r).(x.A^T).B^T and
  the per-token two-term E4M3 split of activations for the FP8 base.
* ``adamw``   -- one AdamW step (decoupled weight decay) on the adapters and
  the bf16 copy of the updated parameters.
* ``stacked`` -- forward and backward with frozen lower adapters under one
  trainable top adapter.

Precision: packing decisions (scales, codes) are taken in IEEE fp32, the
precision the GPU packer uses, so codes can be compared bit for bit.  The
matrix products are evaluated in fp64 by default (inputs are exact fp32
values), which makes the oracle strictly more accurate than the fp32
accumulation on the GPU.

Every function is pinned by ``tests/test_oracle_*.py`` against something other
than itself: library codecs, closed forms, invariants, finite differences,
integer-exact data and brute force.
"""

from . import adamw, codecs, formats, lora, stacked  # noqa: F401
