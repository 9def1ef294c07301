"""Float64 CPU oracle for the Mamba-2 SSD scan -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and this
package imports nothing from the product package.

Contents:
  seq      -- the defining sequential recurrence and its hand-derived backward
              (plain C, float64, OpenMP over independent (batch, head) pairs)
  dual     -- the quadratic masked-attention ("dual") form of the same layer
  chunked  -- the chunked evaluation (per-chunk quadratic block + inter-chunk
              state passing) in float64, with its intermediates
  fd       -- central finite differences of the scalar <dy, y>
  dtproc   -- the step preprocessing dt = softplus(dt_raw + dt_bias) and
              its chain rule
  conv     -- the causal depthwise conv1d (+ bias, SiLU) before the scan, and
              its backward
"""
