"""CPU oracle for the fused 3D RoPE (test infrastructure only).

Only tests/, the graft entry point's smoke() and bench.py's cpu_baseline leg
may import this package.  The product library (rope_ltx3drope_amd) never
does: it fails loudly when its HIP library is missing instead of falling
back to the CPU.

Parity pins (all CPU tests, tests/test_oracle_pins.py): closed forms of the
inverse frequencies, tables against an arbitrary-precision evaluation,
unit-vector readback, identity at position 0, norm preservation, a +theta /
-theta round trip, an error bound against the exact complex product, a
brute-force per-element angle recomputation on tiny grids, the bf16 cast
against torch's CPU cast and its closed-form properties.  Every function
here has such pins.  Bit identity with sglang's own tables cannot be
checked: the pages print no table values.

oracle.neox: the rotate-half RoPE with a gathered cos/sin cache (pins in
tests/test_neox_oracle_pins.py).
"""
from . import dit_freqs, neox, patchify  # noqa: F401
from .rope import (  # noqa: F401
    BF16,
    F32,
    apply_rope_tokens,
    axis_tables,
    bf16_bits_to_f32,
    f32_canonical_nan,
    f32_to_bf16_bits,
    from_f32,
    grid_tables,
    inv_freqs,
    rope3d,
    rope3d_qk,
    rope3d_sampled,
    rotate_pairs,
    to_f32,
    token_coords,
    validate,
)
