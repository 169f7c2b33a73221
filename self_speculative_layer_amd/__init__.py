"""MI355X-native self-speculative decoding: Python binding of libssd.so.

The binding only marshals arguments: every step of the path (draft, verify,
accept, commit, prefill, AR decode, matchness scoring) runs in the library's
HIP kernels.  PyTorch provides device memory and streams.  Importing the
binding does not load the library; ``binding.lib()`` does, and raises if it
is missing (there is no CPU fallback).
"""
from . import binding  # noqa: F401
