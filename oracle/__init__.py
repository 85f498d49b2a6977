"""CPU oracle for the DiffusionGemma canvas denoise step — TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 NumPy statement of what one denoise step computes, written from the
pages' description of the method:
  * "DiffusionGemma Technical Report 정리" (juhoplayground.github.io), cited as [TR §section]
  * "Google DiffusionGemma 출시 – 병렬 블록 디코딩" explainer (molayo1419.me), cited as [PBD §section]
  * "DiffusionGemma 완전분석" (cell-devlog.tistory.com), cited as [CA §section]

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of `bench.py` may import,
call or execute anything in this package.  It shares no code with the HIP library and never
imports it: the two meet only through the seeded arrays of `synth/`.

Parity status per function:
  philox.philox4x32_10   pinned to the published Random123 known-answer vectors (Salmon et al.,
                         SC'11) and by statistics (uniformity, bit balance, avalanche)
  model.denoise_layer / denoise_forward
                         pinned by zero-weight reductions to independently written attention and
                         MoE expectations (pre-norm composition, both residual adds)
  selfcond               pinned by closed forms (argmax row at low temperature, mean row at equal
                         logits), an explicit loop, relabelling invariance and the zero-signal loop
  numerics.quant_rows_e4m3 / model.act_quantiser (W8A8 experts)
                         pinned to torch's e4m3 cast, code round trips, hand ties, saturation, the
                         half-step error bound and an exact special case
  everything else        pinned by closed forms, invariants or brute force in tests/test_oracle_*.py
"""
