"""fp64 CPU oracle for the sequence-parallel DiT attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports, links or
calls this package; only the test suite, ``smoke()`` in
``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` may use
it.  It shares no code, header,
table or helper with the HIP library: it is written from the source pages'
definitions, in float64, with numpy as the only numerical library.

Sources (cited by page title and section):

* edge-dit.cpp, "Parallel execution" page -- CFG combine formula (CFG
  parallelism section); the attention formula after the sequence-to-head
  redistribution and the Ulysses layouts (Ulysses sequence parallelism
  section); the SPSequenceSplit / SPAllToAll4DLayout state and the packed
  peer-major buffers (SP layout and fused operator sections).
* SGLang Diffusion, "Parallelism Overview" -- the USP shapes ("What happens
  to the shapes"), the ring merge needing the kernel's LSE ("Constraints"),
  the all-to-all being a pure permutation ("The Ulysses transport").
* xLLM, "DiT Architecture and Capability Matrix" -- sequence padding to a
  multiple of lcm(SP, 64) and padding exclusion ("MiniMax-H3 boundaries").
* cache-dit, "Context Parallelism" -- head padding before / after the
  all-to-all ("Any Head Num" under UAA); the padding-free splits of
  arbitrary sequence lengths and head counts (Ulysses Anything Attention).
* cache-dit, "Context Parallelism" (Async FP8 Ulysses Attention) -- Q, V
  and O exchanged as FP8, K kept in 16-bit; the FP8 format (OCP E4M3) and
  the block scaling (32-element blocks with a power-of-two scale, as in the
  OCP Microscaling formats) are readings (see the FP8 section of
  ``reference``).
* diffusers, "Distributed inference" (Ring Anything Attention) -- local K/V
  padded to the longest rank, gathered, then cut back to the real lengths.
* The receive preparation with RoPE on Q and K (edge-dit.cpp "Parallel
  execution", Ulysses section) -- the RoPE convention is not on the pages;
  the RoFormer rotation of adjacent dims with caller-given cos / sin tables
  is the reading taken (see ``reference.rope``).
* The optional F32 -> F16 conversion of the packed QKV operator and the
  direct F16 / BF16 output of the head-to-sequence path (edge-dit.cpp
  "Parallel execution") -- rounding to nearest, ties to even, is the reading
  (see ``reference.round_to_half``).

Modules:
  oracle.reference  -- vectorised numpy fp64 definitions (the oracle proper)
  oracle.brute      -- pure-Python loop versions for tiny inputs (a second,
                       independently written check of the oracle itself)

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(closed forms, invariants, brute force, library cross-checks); none is
"parity unpinned".
"""

from .reference import (  # noqa: F401
    attention,
    attention_kv_len,
    merge,
    ring_attention,
    ring_hop_order,
    a2a_layout,
    pack_seq_to_head,
    unpack_seq_to_head,
    rope,
    unpack_seq_to_head_rope,
    pack_head_to_seq,
    unpack_head_to_seq,
    all_to_all,
    pack_seq_to_head_uneven,
    unpack_seq_to_head_uneven,
    pack_head_to_seq_uneven,
    unpack_head_to_seq_uneven,
    uneven_chunk_sizes,
    all_to_all_uneven,
    ring_anything_pad,
    ring_anything_trim,
    E4M3_MAX,
    FP8_BLOCK,
    e4m3_value,
    e4m3_encode,
    fp8_scale_exp,
    quantize_fp8_blocks,
    dequantize_fp8_blocks,
    bf16_bits_to_f64,
    f64_to_bf16_bits_exact,
    fp8_chunk_sections,
    pack_seq_to_head_fp8,
    unpack_seq_to_head_fp8,
    pack_head_to_seq_fp8,
    unpack_head_to_seq_fp8,
    cfg_combine,
    cfg_combine_f32,
    fmaf,
    HALF_FORMATS,
    half_value,
    half_is_nan,
    round_to_half,
    pack_seq_to_head_convert,
    pack_head_to_seq_convert,
)
