"""CPU oracle for TurboQuant KV-cache encode and decode attention on the packed cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` use it, to check and time the HIP path.

The oracle is plain, slow NumPy/SciPy written from the pages' description of the
method, in float64 unless a step says otherwise.  It shares no code, tables or
constants with the HIP library: it has its own codebook solver, Hadamard matrix,
quantisers, bit packer/unpacker and attention.  Inputs come from the seeded
generators in ``compressed_decode_attention_encode_amd.workloads`` (which hold no
method arithmetic).

Pages cited (by title and section):
  * "vllm-metal TurboQuant" guide (wmrh.cn) -- sections on the quantisation
    principle, choosing a compression ratio, and support limits.
  * "TurboQuant vLLM integration" guide (kwkr.cn) -- section 2 (the five-step
    quantisation pipeline), section 5 (hooks, 128-token buffer), section 6.
  * "TurboQuant-MLX" page (pomoai.com) -- core technique and GPU kernel
    optimisation sections.
  * "TurboQuant benchmark on Apple Silicon" page (zingnex.cn) -- compression
    algorithm details and memory tables.
  * "vLLM, llama.cpp, MLX all follow up" news page (digipub.cc) -- oMLX section.

Every function here is pinned by a CPU test against something other than itself
(closed forms, textbook values, invariants, printed figures, brute force).
"""
