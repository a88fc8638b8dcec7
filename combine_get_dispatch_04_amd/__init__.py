"""MoE token dispatch/combine on one MI355X (gfx950).

`_native` is the ctypes binding of libep.so with the C ABI's names
(ep_get_dispatch_layout and its form for every round of a chunked prefill,
ep_get_dispatch_layout_rounds, ep_dispatch, ep_combine, ep_dispatch_expert_choice,
ep_combine_expert_choice, and one rank's share of the exchange:
ep_pack_by_rank, ep_combine_partial, ep_combine_ranks); `api` is a
torch-tensor front end over it.
`workloads` makes the seeded synthetic inputs.  The library is loaded on
first use and a missing build raises instead of falling back.
"""
from . import _native
from ._native import (EpError, ep_combine, ep_combine_expert_choice, ep_combine_partial,
                      ep_combine_ranks, ep_dispatch, ep_dispatch_expert_choice,
                      ep_ec_workspace_bytes, ep_get_dispatch_layout,
                      ep_get_dispatch_layout_rounds, ep_pack_by_rank, ep_pack_workspace_bytes,
                      ep_workspace_bytes, ep_workspace_bytes_rounds)

__all__ = ["EpError", "ep_get_dispatch_layout", "ep_get_dispatch_layout_rounds", "ep_dispatch",
           "ep_combine", "ep_workspace_bytes_rounds",
           "ep_dispatch_expert_choice", "ep_combine_expert_choice", "ep_pack_by_rank",
           "ep_combine_partial", "ep_combine_ranks", "ep_workspace_bytes",
           "ep_ec_workspace_bytes", "ep_pack_workspace_bytes", "api", "workloads"]


def __getattr__(name):
    if name in ("api", "workloads"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
