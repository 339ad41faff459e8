"""fp64 CPU oracle for the attention forward and backward passes, paged decoding, the FP8
forward pass and user score / mask modifications.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check in __graft_entry__ and by the
CPU-baseline leg of bench.py, never by the HIP path.  It shares no code with that path.
"""
from .attention import (MASKS, allowed, allowed_pair_count, attention, attention_blocked,
                        decode_bf16, doc_index, scores)
from .backward import attention_backward, backward_magnitudes, backward_row_dot
from .decode import decode_attention, gather_sequence
from .fp8 import attention_fp8, dequantize_blocks, e4m3_decode, e4m3_encode, quantize_blocks
from .mods import attention_mod, mod_tile_table
from .tiles import tile_class_counts, tile_table

__all__ = ["MASKS", "allowed", "allowed_pair_count", "attention", "attention_backward",
           "attention_fp8", "attention_mod", "mod_tile_table", "dequantize_blocks", "e4m3_decode", "e4m3_encode", "quantize_blocks",
           "attention_blocked", "backward_magnitudes", "backward_row_dot", "decode_attention",
           "decode_bf16", "doc_index", "gather_sequence", "scores",
           "tile_class_counts", "tile_table"]
