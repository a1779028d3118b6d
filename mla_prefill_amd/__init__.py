"""DSA sparse-MLA prefill attention for AMD Instinct MI355X (gfx950).

The computation lives in ``libdsa_prefill.so`` (hand-written HIP kernels behind
a C ABI, declared in ``include/dsa_prefill.h``).  ``mla_prefill_amd._lib`` is
the ctypes binding with the same function names; ``mla_prefill_amd.routings``
adds torch-side allocation of outputs and workspaces for the three routings.

Importing a binding attribute loads the library and fails loudly when it has
not been built (``python -m mla_prefill_amd.build``).
"""

_BINDING_NAMES = (
    "dsa_abi_version", "dsa_status_string", "dsa_union_pad", "dsa_masked_mha_workspace_bytes",
    "dsa_build_group_union", "dsa_sparse_prefill_grouped", "dsa_sparse_prefill_pertoken",
    "dsa_masked_mha_prefill", "dsa_dense_mha_prefill", "DsaError",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
