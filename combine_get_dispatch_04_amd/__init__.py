"""MoE token dispatch/combine on one MI355X (gfx950).

`_native` is the ctypes binding of libep.so with the C ABI's names
(ep_get_dispatch_layout, ep_dispatch, ep_combine, ep_dispatch_expert_choice,
ep_combine_expert_choice); `api` is a torch-tensor front end over it.
`workloads` makes the seeded synthetic inputs.  The library is loaded on
first use and a missing build raises instead of falling back.
"""
from . import _native
from ._native import (EpError, ep_combine, ep_combine_expert_choice, ep_dispatch,
                      ep_dispatch_expert_choice, ep_ec_workspace_bytes, ep_get_dispatch_layout,
                      ep_workspace_bytes)

__all__ = ["EpError", "ep_get_dispatch_layout", "ep_dispatch", "ep_combine",
           "ep_dispatch_expert_choice", "ep_combine_expert_choice", "ep_workspace_bytes",
           "ep_ec_workspace_bytes", "api", "workloads"]


def __getattr__(name):
    if name in ("api", "workloads"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
