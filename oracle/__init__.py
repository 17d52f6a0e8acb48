"""fp64 CPU oracle for chunk-causal multi-head latent attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The product path (``latent_kv_cache_chunk_amd``) never imports
it, and this package imports nothing from the product path: the two share no
code.  The only thing both sides consume is the seeded synthetic inputs, which
the tests hand to each side separately.

Every function is a plain, slow, obviously-correct numpy fp64 implementation
of what the method computes, written in the *non-absorbed* form (per-head K and
V are reconstructed from the latent), so that the absorbed HIP path is checked
against the textbook definition rather than against itself.

Sources (the pages):
  * VideoMLA, arXiv abstract (mlsanity.com paper page, "Abstract (arXiv)"):
    per-head keys and values are replaced by one low-rank content latent
    shared by all heads plus one head-shared, decoupled 3D-RoPE positional
    key; per-token KV memory falls by 92.7% at every cached layer.
  * VideoMLA, atlas.scime.ai AI summary, "Approach" and "Key results":
    head-shared decoupled 3D-RoPE key; 224 cached scalars per token versus
    3072; chunk-causal autoregressive video diffusion on Wan2.1-T2V-1.3B.
  * VideoMLA, mlsanity.com paper page, "Builds on": DeepSeek-V2 (the paper
    that introduced multi-head latent attention); the MLA score and
    up-projection conventions follow it.

Parity status of each function is stated in its docstring ("pinned by ...").
"""

from .mla_oracle import (  # noqa: F401
    BF16_MAX,
    bf16_rne,
    bf16_bits,
    rope3d_angles,
    rope3d,
    latent_rows,
    cache_append,
    attention_probs,
    chunk_attend,
    chunk_attend_rows,
    mha_attend,
    mha_attend_rows,
)
