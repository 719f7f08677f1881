"""fp64 CPU oracle for paged-KV block-sparse-row attention.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the product library never does, and this
package never imports the product library.  It shares no code with the GPU
path.

- ``attn``: exact attention, n-way log-sum-exp merge and the cascade
  composition, backed by ``attn_ref.c`` (plain C, fp64).
- ``plan_ref``: the CPU-side work partition ("plan"), pure Python.
"""
