"""Slow, plain float64 CPU oracle for causal packed attention and the MX quantiser.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this
package: only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` use it. It shares no code, constants or helpers with the HIP library in
``causal_flashattention_amd``; the two meet only through the seeded inputs produced by
``causal_flashattention_amd.workloads``.

Sources (web pages; cited by title and section):

* "GPT Kernel Programlama: MatMul, Softmax ve Attention Hesabı" (dehayz.com) -- §2 gives the
  attention equations, §3 the score sum, §4 the causal mask, §5 the max-subtracted softmax,
  §6 the value sum.
* "FlashAttention (HU)" (systems-analysis.info) -- section "A szabványos attention
  problematikája": the softmax(QKᵀ/√d_k)·V definition (its ``\\text`` macros are garbled on the
  page; read as plain softmax(QKᵀ/√d_k)V).
* "FLAMIA: Blackwell Üzerinde Hızlı ve Nedensel Olarak Güvenli Eğitim İçin Flash
  Mikro-Ölçeklemeli Dikkat Mekanizması" (blog.edumints.com) -- section "FLAMIA Mimarisi ve Temel
  Tasarım İlkeleri": MXFP8 path, token-block scaling, leakage safeguards, fwd/bwd consistency,
  document-local scaling over packed layouts.
* "Flash Attention" (ai.ozdemir.be) -- sections "Tanım" and "Gerçek dünyadan örnek": local
  inference reads a quantised K/V cache (8-bit at about half the memory of f16) through flash
  attention.

Modules:

* ``attention``     -- naive two-pass forward with an explicit mask, and its exact gradient.
* ``mx``            -- E4M3 (also E2M1, E2M3, E3M2) / E8M0 block quantiser (along the head dim, or along
  doc-local tokens).
* ``mx_attention``  -- the attention oracle fed with the quantised operand copies.
* ``decode``        -- one query per sequence over a packed (optionally MX-quantised) KV cache.

Every function states the passage it follows; the readings taken where the pages are silent
are listed in the repository's design notes.
"""

from . import attention, decode, mx, mx_attention  # noqa: F401
