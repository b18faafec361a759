"""MI355X-native masked rotary attention for one sequence-parallel rank's share.

The compute lives in ``libltxa.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/ltxa.h``).  :mod:`video_dit_sequence_amd.ltxa` is the
thin ctypes binding over it; :mod:`video_dit_sequence_amd.workloads` draws the
seeded synthetic inputs.  Importing this package loads nothing; the library is
opened on first use and a missing library is an error.
"""

__version__ = "0.1.0"
