"""ring_kv_amd: the speculative-decoding verify step on AMD Instinct MI355X (gfx950).

The work runs in libring_kv (HIP kernels behind the C interface of include/ring_kv.h);
this package is its torch-tensor binding.  Build the library with
``python -m ring_kv_amd.build``.
"""
from .api import (Pager, attn_merge_partials, decode_attn_ref_layout,  # noqa: F401
                  kv_page_in, kv_page_out, ref_layout_to_paged, ref_layout_to_ring,
                  tensor_from_numpy, verify_accept, verify_attn_paged,
                  verify_attn_paged_append_dev, verify_attn_paged_auto_splits,
                  verify_attn_paged_partial, verify_attn_paged_dev, verify_attn_paged_resident,
                  verify_attn_ring, verify_attn_ring_append_dev, verify_attn_ring_dev,
                  verify_kv_append_paged, verify_kv_append_paged_dev,
                  verify_kv_append_ring, verify_kv_append_ring_dev, verify_pos_advance)
from ._lib import LIB_PATH, RkvError, declared_functions, lib  # noqa: F401
