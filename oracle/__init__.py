"""CPU oracle for the batch-1 decode path -- test infrastructure only.

Plain, slow, obviously-correct numpy code that states what one decode step
of a pre-norm Llama-style (or Mixtral-style MoE) decoder computes, plus an
independent builder of the instruction tensor and a schedule simulator.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the GPU path
(``persistent_megakernel_decode_02_amd``); the two meet only in the seeded
input generators of ``synth``.

Parity status of each function is stated in its module docstring.
"""
