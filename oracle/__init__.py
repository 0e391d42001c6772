"""fp64 CPU oracle for paged GQA attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP
library (``paged_gqa_attention_02_amd``) and never imports it.
"""
from .oracle import (bind, brute_decode, brute_extend, cache_append, decode,  # noqa: F401
                     decode_bf16, decode_e4m3fn, default_threads, encode_e4m3fn, extend,
                     host_cpus,
                     lib, verify)
