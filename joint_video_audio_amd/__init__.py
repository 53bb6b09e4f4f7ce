"""MI355X-native forward pass of a MiniMax-H3-style packed DiT block.

The compute path is the HIP library ``libminih3.so`` (kernels for gfx950
behind a C ABI, declared in ``include/minih3.h``); ``joint_video_audio_amd.minih3``
is its thin ctypes binding. ``joint_video_audio_amd.synth`` draws seeded
synthetic workloads. Importing this package loads nothing; the binding loads
the library on first use and raises if it is missing.
"""
