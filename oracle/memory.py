"""Byte accounting of the quantized formats (closed forms).

TEST INFRASTRUCTURE ONLY, like the rest of `oracle/`.

Nominal figures count only the codes; exact figures add the per-block
constants that block-wise quantization stores (one fp32 absmax per block, or,
with nested quantization, one 8-bit code per block plus one fp32 absmax per
group of blocks and one fp32 mean per tensor).
"""


def weight_bytes_per_param(fmt, blocksize=None, nested=False, blocksize2=256):
    """fmt in fp32, fp16, int8, int4.  With a blocksize, the block constants count."""
    base = {"fp32": 4.0, "fp16": 2.0, "int8": 1.0, "int4": 0.5}[fmt]
    if blocksize is None or fmt in ("fp32", "fp16"):
        return base
    if not nested:
        return base + 4.0 / blocksize
    return base + 1.0 / blocksize + 4.0 / (blocksize * blocksize2)


def adam_state_bytes_per_param(bits, blocksize=None):
    """Two moments; 32-bit (4 bytes each) or 8-bit codes (1 byte each) with an
    fp32 absmax per block of each moment."""
    if bits == 32:
        return 8.0
    return 2.0 + (8.0 / blocksize if blocksize else 0.0)


def total_saving(model_fraction, optimizer_fraction):
    """Saving against an FP32 baseline whose model and optimizer bytes are taken
    equal (the assumption under which the pages' savings table adds up)."""
    if optimizer_fraction is None:
        return 1.0 - model_fraction
    return 1.0 - (model_fraction + optimizer_fraction) / 2.0


def nested_saving_bits(blocksize=64, blocksize2=256):
    """Bits per parameter saved by nesting: fp32 absmax per block versus one
    8-bit code per block plus one fp32 absmax per group of blocksize2 blocks."""
    return 32.0 / blocksize - (8.0 / blocksize + 32.0 / (blocksize * blocksize2))
