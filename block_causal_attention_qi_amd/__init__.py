"""Prefix-reuse block-causal attention for one MI355X (gfx950).

The compute path is the HIP library libqi.so (sources in csrc/, C ABI in include/qi.h);
`qi` is its thin ctypes binding and `synth` draws seeded synthetic inputs.  Importing the
package loads nothing; `from block_causal_attention_qi_amd import qi` loads the library
and fails loudly if it has not been built.
"""
__all__ = ["qi", "synth"]
