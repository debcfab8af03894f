"""CPU oracle for Four Over Six (4/6) NVFP4 block quantization -- TEST INFRASTRUCTURE.

This package is a plain, slow, deliberately unoptimised NumPy statement of what the
HIP library computes.  It exists only to check that library.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import it; the
product path (``fp4_block_quantization_amd``) never imports or calls it, and the two
share no code, tables or constants.

Sources (pages, by title and section):
  * Four Over Six documentation page (Hugging Face transformers docs), §Four Over
    Six: each NVFP4 block is scaled so that its largest magnitude maps either to 6 or
    to 4, whichever reduces the quantization error; options: random Hadamard
    transform, 2D block scaling, transposed inputs, stochastic rounding; older GPUs
    and CPUs simulate the quantized matmul with an FP32 matrix multiplication.
  * Ultralytics glossary "FP4", opening section: the E2M1 layout and its value set
    {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit.
  * Same page, §How FP4 works: block scaling chooses the scale that maps the block's
    largest magnitude to 6; NVFP4 groups 16 values under one FP8 E4M3 scale plus one
    FP32 per-tensor scale; the worked example of one scale vs 32- vs 16-value blocks.
  * Same page, §FP4 for inference and training: random Hadamard transforms spread
    outliers, stochastic rounding is used for gradients.

Where the pages leave a step open, the modules state the reading they take; the list
of readings is kept with the design notes.  Functions whose result the pages and
mathematics pin are tested against those pins in ``tests/test_oracle_*.py``.
"""

from . import formats, fparith, philox, hadamard, nvfp4, qlinear, mxfp4, page_example  # noqa: F401
