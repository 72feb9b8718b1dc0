"""fp64 CPU oracle of gzip-guided block-sparse causal attention.

Test infrastructure only: imported by tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product library.
"""
from .gsa_oracle import *  # noqa: F401,F403
from .gsa_oracle import (LOCAL, LITERAL, HYBRID, CLASS_NAMES, zlib_runtime_version,  # noqa: F401
                         gzip_member, gzip_length, compressed_lengths, literal_flags,
                         block_mask, block_masks, default_head_counts, head_classes,
                         to_csr, to_csc, token_mask, attn_fwd, attn_fwd_rows, attn_bwd,
                         attn_bwd_qblock, attn_bwd_kblock, kept_keys)
