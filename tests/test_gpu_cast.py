"""ra_cast_f32_to_bf16 (the finalise step's bf16 cast of out, dQ, dK, dV) against
a round-to-nearest-even reference written here, bit for bit, and the forward's
own bf16 copy of out against that cast.

The reference does not use the kernel's bit trick: for every finite input it
takes the two bf16 neighbours of |x| (truncation and the next value up),
measures both distances exactly in float64 and keeps the nearer one, the one
with an even last mantissa bit on a tie (IEEE 754 roundTiesToEven).  A NaN must
stay a NaN of the same sign with the quiet bit set and its top payload bits
kept, as the header states."""
import numpy as np
import pytest

import synth
from gpu_util import dev, log

pytestmark = pytest.mark.gpu


def rne_reference(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of the float32 array x, round to nearest even."""
    u = x.view(np.uint32).astype(np.uint64)
    sign = (u >> 31) << 15
    mag = u & 0x7FFFFFFF
    lo = mag >> 16                      # bf16 magnitude toward zero
    hi = lo + 1                         # next bf16 magnitude up (0x7f80 is +inf)
    with np.errstate(invalid="ignore"):
        f = np.abs(x.astype(np.float64))

    finite = np.isfinite(x)
    lo = np.where(finite, lo, 0)
    hi = np.where(finite, hi, 1)

    def value(bits):
        v = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
        return np.where(bits == 0x7F80, 2.0 ** 128, v)  # one step past the largest finite bf16

    with np.errstate(invalid="ignore"):
        d_lo = np.where(finite, f, 0.0) - value(lo)
        d_hi = value(hi) - np.where(finite, f, 0.0)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & 1) == 1))
    out = np.where(pick_hi, hi, lo) | sign
    out = np.where(np.isinf(x), 0x7F80 | sign, out)
    out = np.where(np.isnan(x), (u >> 16) | 0x40, out)
    return out.astype(np.uint16)


def _inputs():
    rng = np.random.default_rng(5)
    rand_bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    special = [0x00000000, 0x80000000, 0x7F800000, 0xFF800000,            # +-0, +-inf
               0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF812345, 0x7FBFFFFF,  # NaNs (quiet, signalling, payloads)
               0x00000001, 0x80000001, 0x007FFFFF, 0x00008000, 0x00018000,  # subnormals, incl. ties
               0x00007FFF, 0x00008001, 0x0000FFFF, 0x00010000, 0x00800000,  # around the subnormal/normal edge
               0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x7F7F8001,  # max finite, ties that overflow
               0x3F808000, 0x3F818000, 0x3F808001, 0x3F807FFF,               # ties to even at 1.0
               0x3F800000, 0xBF800000, 0x3EAAAAAB, 0x40490FDB]
    ties = rng.integers(0, 2 ** 16, size=4096, dtype=np.uint64).astype(np.uint32) << 16 | 0x8000
    sub = rng.integers(1, 1 << 23, size=4096, dtype=np.uint64).astype(np.uint32)  # positive subnormals
    bits = np.concatenate([np.array(special, dtype=np.uint32), ties, sub, sub | 0x80000000, rand_bits])
    return bits.view(np.float32)


def test_reference_itself():
    """Spot values of the reference (hand-derived, independent of any code here)."""
    x = np.array([1.0, 1.00390625, 1.01171875, 1.0 + 2 ** -8 + 2 ** -20, 1.0 + 2 ** -9, -0.0, 3.0e38, 3.4e38,
                  -np.inf, 2.0 ** -133, 3 * 2.0 ** -134], dtype=np.float32)
    # 1 + 2^-8 is halfway between 1.0 and 1 + 2^-7: ties to 1.0 (even mantissa);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to 1 + 2^-6 (even);
    # just above the first tie rounds up, a quarter ulp rounds down;
    # 3.0e38 = 1.7632 * 2^127: mantissa 0.7632 * 128 = 97.7 -> 98;
    # 3.4e38 lies past the midpoint above the largest finite bf16, (2 - 2^-7) * 2^127: +inf;
    # subnormals: 2^-133 is bf16 subnormal 0x0001 (its ulp is 2^-133), 3 * 2^-134 ties between 1 and 2 -> 2.
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x3F80, 0x8000, 0x7F62, 0x7F80, 0xFF80, 0x0001, 0x0002],
                    dtype=np.uint16)
    assert np.array_equal(rne_reference(x), want), [hex(v) for v in rne_reference(x)]


@pytest.mark.parametrize("offset,n_cut", [(0, 0), (1, 3), (3, 0), (0, 5)])
def test_cast_bit_exact(offset, n_cut):
    """Aligned (vector path) and misaligned (element path) pointers, lengths with a tail."""
    import torch
    import exact_long_context_ra_amd as ra
    x = _inputs()
    n = x.size - offset - n_cut
    log(f"cast bit-exact offset={offset} n={n}")
    xs = torch.from_numpy(x.copy()).to(dev())
    src = xs[offset:offset + n]
    buf = torch.full((n + 8,), -1, dtype=torch.int16, device=dev())
    dst = buf[offset:offset + n].view(torch.bfloat16)
    ra.lib()
    from exact_long_context_ra_amd._lib import check
    check(ra.lib().ra_cast_f32_to_bf16(src.data_ptr(), dst.data_ptr(), n, torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    got = buf.cpu().numpy().view(np.uint16)
    want = rne_reference(x[offset:offset + n])
    bad = np.nonzero(got[offset:offset + n] != want)[0]
    assert bad.size == 0, (f"{bad.size} mismatches, first at {bad[0]}: x bits {x[offset + bad[0]].view(np.uint32):#010x} "
                           f"got {got[offset + bad[0]]:#06x} want {want[bad[0]]:#06x}")
    # nothing written outside [offset, offset + n)
    assert np.all(got[:offset] == 0xFFFF) and np.all(got[offset + n:] == 0xFFFF)


def test_cast_api_and_empty():
    import torch
    import exact_long_context_ra_amd as ra
    x = torch.from_numpy(_inputs()[:1000].copy()).to(dev())
    y = ra.cast_f32_to_bf16(x)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), rne_reference(x.cpu().numpy()))
    empty = torch.empty(0, device=dev())
    assert ra.cast_f32_to_bf16(empty).numel() == 0


@pytest.mark.parametrize("layout", ["zigzag", "stripe"])
def test_forward_lowp_copy_is_the_rne_cast(layout):
    """The forward's bf16 copy of out (written by the last ring step) equals the
    library cast of its fp32 out, bit for bit."""
    import torch
    import exact_long_context_ra_amd as ra
    from gpu_util import ring_from_global
    S, N, H, D = 2048, 4, 2, 128
    log(f"out_lowp == cast(out) {layout}")
    q, k, v = synth.qkv(S, H, D, torch.bfloat16, seed=9, device="cpu")
    q, k, v = q.to(dev()), k.to(dev()), v.to(dev())
    kr, idx = ring_from_global(k, layout, N)
    vr, _ = ring_from_global(v, layout, N)
    for r in range(N):
        ql = q.index_select(1, idx[r]).contiguous()
        out, _, lowp = ra.ring_fwd(layout, N, r, ql, kr, vr, causal=True, want_lowp=True)
        cast = ra.cast_f32_to_bf16(out)
        torch.cuda.synchronize()
        assert torch.equal(lowp.view(torch.int16), cast.view(torch.int16)), f"rank {r}"
        want = rne_reference(out.cpu().numpy().reshape(-1))
        assert np.array_equal(cast.view(torch.int16).cpu().numpy().reshape(-1).view(np.uint16), want)
