"""RelayAttention decode-time attention for AMD Instinct MI355X (gfx950).

``shared_prompt_kv_amd.relay`` is the Python binding of the C-ABI library
``librelay_attn.so`` (built from ``csrc/``).  ``shared_prompt_kv_amd.workloads``
draws the seeded synthetic inputs.  Importing the package loads nothing; the HIP
library is loaded on first use and its absence is an error.
"""
__all__ = ["relay", "workloads"]
