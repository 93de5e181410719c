"""MI355X-native routed MXFP4 mixture-of-experts layer.

The compute path is the HIP library built from csrc/ (libmoe_mi355x.so);
`lib` is its thin ctypes binding.  `workloads` draws the seeded synthetic
inputs."""


def __getattr__(name):
    if name == "lib":
        from . import binding
        return binding
    raise AttributeError(name)
