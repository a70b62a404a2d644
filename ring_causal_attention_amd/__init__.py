"""MI355X-native blockwise causal (ring) attention: RoPE, packing mask, online softmax.

The compute path is the C-ABI library ``liblwm_attn.so`` (hand-written HIP for gfx950);
``ring_causal_attention_amd.lwm`` is its thin ctypes binding and ``ring_causal_attention_amd.path``
composes its calls into the ring loop and the training step.  Importing this package does not
load the library; the binding loads it on first use and fails loudly if it is missing.
"""
