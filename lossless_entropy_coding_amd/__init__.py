"""Lossless BF16 weight codec for MI355X (gfx950).

BF16 words are split into a joint (sign, exponent) symbol coded with a
per-tensor rANS model and a 7-bit fraction coded with a distribution that the
decoded symbol selects; decoding recombines the fields bitwise and copies
non-BF16 spans verbatim [Qwen3.8-27B-BF16-NVLC-Lossless model card, codec
paragraph].  Decoding runs in HIP kernels behind a C ABI (include/bs.h).
"""
