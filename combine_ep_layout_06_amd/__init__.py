"""MI355X-native MoE expert-parallel layout, dispatch and combine for one GPU.

The compute runs in hand-written gfx950 HIP kernels behind a C ABI (``include/ep.h``,
``libep_mi355x.so``). ``binding`` wraps those entry points for torch tensors (device memory
and the current HIP stream only). ``workloads`` draws the seeded synthetic inputs and
``accounting`` counts bytes.
"""
_BINDING_NAMES = ("ep_layout", "ep_dispatch", "ep_dispatch_fp8", "ep_layout_dispatch",
                  "ep_layout_dispatch_fp8", "ep_combine", "ep_version",
                  "ep_error_string", "EpError", "library_path", "load_library")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
