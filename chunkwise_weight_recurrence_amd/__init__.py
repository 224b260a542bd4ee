"""MI355X-native chunkwise TTT fast-weight layer (HIP, gfx950) and In-Place TTT update.

The compute lives in ``libttt.so`` (C ABI in ``include/ttt.h``); this package
is its ctypes binding (``binding``), device plumbing (``layer``), seeded
synthetic workloads (``workloads``) and the build script (``build``).
"""
from .binding import (ENTRY_BWD, ENTRY_FWD, EXPORTS, Act, Decay, DType, Loss, Status, TTTDesc,
                      TTTError, TTTMlpDesc, make_mlp_desc, ttt_mlp_bwd_workspace_size, ttt_mlp_chunk_bwd, ttt_mlp_chunk_fwd, ttt_mlp_saved_size,
                      ttt_mlp_workspace_size, inplace_ttt_bwd, inplace_ttt_bwd_workspace_size, inplace_ttt_fwd, inplace_ttt_fwd_guarded,
                      inplace_ttt_guarded_workspace_size,
                      inplace_ttt_workspace_size, lib, make_desc, ttt_chunk_bwd, ttt_chunk_fwd,
                      ttt_last_error, ttt_saved_size, ttt_version, ttt_workspace_size)

__all__ = ["ENTRY_BWD", "ENTRY_FWD", "EXPORTS", "Act", "Decay", "DType", "Loss", "Status", "TTTDesc",
           "TTTError", "TTTMlpDesc", "make_mlp_desc", "ttt_mlp_bwd_workspace_size", "ttt_mlp_chunk_bwd",
           "ttt_mlp_chunk_fwd", "ttt_mlp_saved_size", "ttt_mlp_workspace_size",
           "inplace_ttt_bwd", "inplace_ttt_bwd_workspace_size", "inplace_ttt_fwd", "inplace_ttt_fwd_guarded",
           "inplace_ttt_guarded_workspace_size", "inplace_ttt_workspace_size", "lib", "make_desc", "ttt_chunk_bwd", "ttt_chunk_fwd",
           "ttt_last_error", "ttt_saved_size", "ttt_version", "ttt_workspace_size"]
