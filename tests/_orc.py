"""The oracle as the pin tests see it: one build of pa_oracle.c, swappable so
that the mutation tests can run the same pins against altered builds."""
import oracle


class Oracle:
    def __init__(self, clib=None):
        self.clib = clib or oracle.lib()

    def decode(self, case, num_splits=0, threads=None):
        return oracle.decode(case, num_splits, threads, clib=self.clib)

    def extend(self, case, rows=None, threads=None):
        return oracle.extend(case, rows, threads, clib=self.clib)

    def decode_bf16(self, bits):
        return oracle.decode_bf16(bits, clib=self.clib)

    def decode_e4m3fn(self, bits):
        return oracle.decode_e4m3fn(bits, clib=self.clib)

    def verify(self, case, q, threads=None):
        return oracle.verify(case, q, threads, clib=self.clib)

    def encode_e4m3fn(self, x):
        return oracle.encode_e4m3fn(x, clib=self.clib)

    def cache_append(self, *args, **kw):
        return oracle.cache_append(*args, clib=self.clib, **kw)

    brute_decode = staticmethod(oracle.brute_decode)
    brute_extend = staticmethod(oracle.brute_extend)
