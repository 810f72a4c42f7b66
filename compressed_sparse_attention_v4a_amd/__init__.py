"""MI355X-native hot path of DeepSeek-V4 compressed sparse (CSA) and heavily
compressed (HCA) attention.

The compute lives in libv4a.so (hand-written HIP kernels for gfx950 behind a
C ABI declared in include/v4a.h).  `binding` marshals arguments to it; the
library is loaded on first use and its absence is an error.
"""
