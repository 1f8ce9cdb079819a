"""fp64 CPU oracle for the DFlash/DSpark draft MLA attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check of the
entry module and the CPU-baseline leg of the bench use it.  It shares no code
with the HIP library or its Python binding, and it never consumes a value the
HIP path produced except as the thing being checked.

What it computes, and the passages it follows:

* ``attention.mla_attention`` -- the plain definition of the draft attention:
  queries from the noise block, keys/values over [context | noise], key =
  [k_nope (per head) | k_rope (head-shared, NoPE)], scale q_head_dim ** -0.5,
  the dense additive mask added unchanged to the scores, softmax over keys,
  weighted sum of v.  NeMo AutoModel pages: "dflash.draft_kimi_k3" --
  KimiK3DFlashAttention (class text and forward: one K/V per query head, no GQA
  repeat; the mask is passed through unchanged) and the module text on NoPE
  (no rotary embedding: the 64 rope channels are one more part of the key, the
  same for every head); "dspark.draft_kimi_k3"
  -- KimiK3DSparkAttention attributes (q_head_dim, scaling) and forward
  (context concatenated before the noise block).
* ``expand.latent_expand`` -- kv_b_proj as a plain Linear: per head a slice of
  qk_nope_head_dim + v_head_dim outputs.  Same class texts; latent width from the
  Kimi K3 model page (MLA context-parallel forward: kv_lora_rank + qk_rope_head_dim
  values per token).
* ``occupancy.tile_classes`` / ``tile_lists`` / ``tile_bits`` -- the integer tile
  classification of an additive mask (all -inf / all zero / only zeros and
  -inf / anything else) and the per-row visibility words of binary tiles
  that the method uses to skip fully masked tiles.  The pages only require
  that the score matrix is never materialised (KimiK3DFlashAttention.forward);
  the classification is defined here by its plain meaning.

* ``backward.mla_attention_backward`` / ``logsumexp_rows`` -- the gradients of
  that attention with respect to q, k_nope, the head-shared k_rope (summed over
  heads) and v, and the per-row log normaliser a forward pass saves for them.
  The draft is trained (DFlash page, KimiK3DFlashDraftModel class text: the
  DFlash trainer; DSpark page, module text: speculative-decoding training).

* ``projection.context_project`` / ``q_project`` / ``kv_project`` / ``rms_norm``
  -- the Linear + RMSNorm chains around the attention: fc and hidden_norm on the
  target context, Q-LoRA (q_a_proj, q_a_layernorm, q_b_proj), and the keys and
  values over [context | noise] (kv_a_proj_with_mqa, kv_a_layernorm on the
  latent part, kv_b_proj).  DFlash page module text (Q-LoRA, compressed KV
  latent, fp32-variance RMSNorm); DSpark page KimiK3DSparkAttention attributes
  and forward, KimiK3DSparkModel._forward_backbone.

* ``gqa.materialize`` / ``forward_block`` / ``gqa_attention`` / ``rope`` /
  ``yarn_inv_freq`` -- the MHA/GQA DFlash draft of the Modular MAX page
  (pipelines.architectures.dflash_kimi_k25): qk-normed, yarn-RoPE keys and the
  values of the context written into a cache once (materialize), then each
  block attends non-causally to that cache plus itself (forward_block).

Readings where the pages are silent (also listed in the design notes):
a row whose every score is -inf returns 0; a mask entry is "masked" only if it
is exactly -inf, any finite value (including large negatives) is added as is.

Pinned by tests/test_oracle_pins.py (closed forms, invariants, brute force,
a library routine) -- nothing here is "parity unpinned".
"""
from .attention import mla_attention, softmax_weights  # noqa: F401
from .backward import logsumexp_rows, mla_attention_backward  # noqa: F401
from .projection import context_project, kv_project, linear, q_project, rms_norm  # noqa: F401
from .gqa import forward_block, gqa_attention, materialize, rope, yarn_inv_freq, yarn_mscale  # noqa: F401
from .expand import latent_expand  # noqa: F401
from .occupancy import tile_bits, tile_classes, tile_lists  # noqa: F401
