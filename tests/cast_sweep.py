"""Worker of the exhaustive bf16-cast pin (tests/test_oracle_step.py): one
block of 2^24 consecutive fp32 bit patterns, the oracle's cast against
torch's conversion.  Imported by spawned worker processes, so it holds no
test state."""

import numpy as np

BLOCK = 1 << 24


def check_block(b):
    """(mismatching non-NaN patterns, NaN patterns whose cast is not a NaN of
    the same sign) in block b."""
    import torch
    from oracle import step as S
    torch.set_num_threads(1)
    u = np.arange(b * BLOCK, (b + 1) * BLOCK, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    ours = S.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    bad = int(np.count_nonzero(ours[~nan] != ref[~nan]))
    o = ours[nan].astype(np.uint32) << 16
    bad_nan = int(np.count_nonzero(~np.isnan(o.view(np.float32)))
                  + np.count_nonzero((ours[nan] >> 15) != (u[nan] >> 31)))
    return bad, bad_nan
