"""TwELL sparse gated-FFN forward for AMD MI355X (gfx950).

``activation_sparse_feed_gate_amd.tw`` is the binding of the HIP library
(loading it fails loudly when the library is not built);
``activation_sparse_feed_gate_amd.synth`` draws seeded synthetic inputs.
"""
