"""MI355X-native CSR graph-attention hot path.

The compute path is ``libgat.so`` (hand-written HIP for gfx950 behind a C-ABI,
declared in ``include/gat.h``); ``sparse_graph_attention_degree_amd.gat`` is its
ctypes binding.  ``graphs`` holds the seeded synthetic input generators.
"""
__all__ = ["graphs", "gat"]
