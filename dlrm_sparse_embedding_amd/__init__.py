"""MI355X-native pooled embedding lookup, key dedup and sparse optimizer step.

The compute path is the HIP library ``libemb.so`` (C ABI in ``include/emb.h``);
``dlrm_sparse_embedding_amd.emb`` is its thin ctypes binding. Importing this
package loads nothing: the binding loads the library on first use and raises if
it is missing.
"""
__all__ = ["workloads", "emb"]
