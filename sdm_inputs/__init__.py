"""Seeded synthetic inputs for the Sparse Delta Memory layer forward.

This module is shared by the tests, the benchmark and the oracle driver.  It
holds no part of the method's arithmetic: it only draws random numbers and lays
them out in the shapes and storage formats the layer consumes.

Workload recipes follow the five configurations the layer is measured on:
tiny, small, 1.4B-shaped, long-context and 8B-shaped.  The 1.4B and 8B shapes
use the memory sizes the SDM blog post (lcabannes.github.io/sdm-blogpost)
states in its "Background" section and in the caption of the figure "The SDM
mechanism, end to end": about 230,400 slots (480 x 480 product keys) with 64
active slots per token, and slot width 3840 stored in bf16 for the 8B model.
The long-context recipe plants a repeated query at token 61 -> T-17, after the
needle-in-a-haystack geometry of the post's "Memory Access Patterns" section
(needle at token 61, query at token 239 of 256).

Distribution notation: N(mu, s) means mean mu and standard deviation s.

Layouts (row-major, innermost last):
  wq, rq   [B, T, H, dk]   in_dtype   (bf16 is carried as raw uint16 bits)
  v        [B, T, H, d]    in_dtype
  alpha    [B, T, H]       float32
  beta     [B, T, H]       float32
  subkeys  [H, 2, S, dk/2] in_dtype
  mem0     [B, H, N, d]    state dtype, N = S*S, slot-major
"""
from .gen import (CONFIGS, Config, config, make_inputs, make_mem0, make_mem0_seqs, make_upstream_grads, make_projection_inputs, bf16_bits_from_f32,
                  f32_from_bf16_bits, normal_f32)

__all__ = ["CONFIGS", "Config", "config", "make_inputs", "make_mem0", "make_mem0_seqs", "make_upstream_grads", "make_projection_inputs", "bf16_bits_from_f32",
           "f32_from_bf16_bits", "normal_f32"]
