"""CPU oracle for layer-streamed LoRA fine-tuning over an NF4 base.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links anything here: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, table,
constant generator or helper with the HIP library; the two meet only at the
seeded input generator (``layer_streamed_qlora_nf4_amd.synth``), which holds
none of the method's arithmetic.

Everything is plain NumPy in float64, written to be checked by eye against its
source.  Citations name a page and a section heading on it:

* LS-docs: "Layer streaming: fine-tune a model that does not fit in your card"
  (trysoup.dev/docs/layer-streaming), with its section headings such as
  "How it works", "Bit-exact is two claims, not one", "Shard cache".
* About: "About Soup" (trysoup.dev/about).

The pages name the stack that supplies NF4, LoRA and the decoder-layer maths
(bitsandbytes, PEFT, transformers: LS-docs "How it works" and "Bit-exact is
two claims, not one") but print none of it.  Where a step is filled from that
stack's published definition the function says which reading it takes.

Modules
-------
bf16    float32 <-> bfloat16 round-to-nearest-even on bit patterns.
nf4     NormalFloat-4 codebook, blockwise absmax quantize / dequantize.
lora    LoRA linear forward and backward (no base-weight gradient).
layer   RMSNorm, rotary embedding, causal GQA attention, SwiGLU and the
        pre-norm decoder layer, forward and hand-derived backward.
model   embedding -> decoder stack -> final norm -> head -> mean next-token
        cross-entropy, forward and backward to every adapter.
sizes   closed-form shard / store sizes.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
(finite differences, closed forms, library special cases, invariants or the
pages' printed sizes).  None is "parity unpinned".
"""
