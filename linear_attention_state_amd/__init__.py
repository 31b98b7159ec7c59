"""Tail-Replay GDN state rebuild for AMD Instinct MI355X (gfx950).

The compute path is the HIP library libtailreplay.so (C ABI: include/tailreplay.h);
this package is its thin Python binding.  Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""
from .ops import (GroupReplay, gdn_decode, gdn_replay, gdn_replay_noalloc, gdn_replay_workspace_size,  # noqa: F401
                  gdn_transition, gdn_transition_workspace_size,
                  get_gdn_schedule, group_replay, la_layer_inputs, la_output_residual, la_project, rmsnorm,
                  set_gdn_schedule, state_compose, tail_length, tail_seqlens)
from ._lib import LIB_PATH, TailReplayError, lib  # noqa: F401

__all__ = ["gdn_replay", "gdn_replay_noalloc", "gdn_replay_workspace_size", "set_gdn_schedule", "get_gdn_schedule", "gdn_transition", "gdn_transition_workspace_size", "state_compose", "gdn_decode", "group_replay", "GroupReplay", "la_layer_inputs", "la_output_residual", "la_project", "rmsnorm",
           "tail_length", "tail_seqlens", "TailReplayError", "lib", "LIB_PATH"]
