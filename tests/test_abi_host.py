"""CPU-only checks of the C ABI: the library loads, exports every function the
header declares, lays tokens out exactly as the oracle does, and rejects bad
arguments with the right status before touching the GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from oracle_pins import closed_form_pairs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ra.h")


@pytest.fixture(scope="module")
def ra():
    import exact_long_context_ra_amd as pkg
    pkg.lib()
    return pkg


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported(ra):
    names = _declared_functions()
    assert len(names) >= 15
    lib = ra.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"


def test_abi_version_and_strings(ra):
    lib = ra.lib()
    assert lib.ra_abi_version() == 3
    assert lib.ra_status_str(0) == b"RA_OK"
    assert lib.ra_status_str(4) == b"RA_ERR_WORKSPACE"
    assert lib.ra_kernel_name(0) == b"block_fwd"
    assert lib.ra_kernel_name(1) == b"block_bwd_dkdv"
    assert lib.ra_kernel_name(7) == b"block_bwd_dq"
    assert lib.ra_kernel_name(8) == b"block_bwd_dq_ds"


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "stripe"])
@pytest.mark.parametrize("S,N", [(16, 1), (64, 4), (96, 3), (512, 8), (131072, 8)])
def test_positions_match_oracle(ra, layout, S, N):
    for r in range(N):
        got = ra.layout_positions(layout, S, N, r)
        want = oracle.layout_positions(layout, S, N, r)
        assert np.array_equal(got, want), (layout, S, N, r)


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "stripe"])
def test_posmap_segments(ra, layout):
    S, N = 4096, 8
    for r in range(N):
        m = ra.layout_posmap(layout, S, N, r)
        pos = []
        for i in range(m.nseg):
            s = m.seg[i]
            pos.extend(s.begin + s.stride * np.arange(s.len))
        assert np.array_equal(np.array(pos), oracle.layout_positions(layout, S, N, r))


@pytest.mark.parametrize("layout", ["contiguous", "zigzag", "stripe"])
def test_pair_counts_from_library_positions(ra, layout):
    """The benchmark's FLOP accounting counts pairs from library positions; the
    counts must equal the closed forms."""
    S, N = 256, 8
    for r in range(N):
        qpos = ra.layout_positions(layout, S, N, r)
        got = sum(int(np.searchsorted(np.sort(ra.layout_positions(layout, S, N, s)), qpos, side="right").sum())
                  for s in range(N))
        assert got == closed_form_pairs(layout, S, N, r)


@pytest.mark.parametrize("layout", ["zigzag_varlen", "stripe_varlen"])
def test_per_sequence_positions_match_oracle(ra, layout):
    for N, cu in [(1, [0, 6, 24]), (2, [0, 8, 24]), (4, [0, 8, 8, 64, 128]), (8, [0, 16, 16, 4096, 8192])]:
        S = cu[-1]
        for r in range(N):
            got = ra.layout_positions(layout, S, N, r, cu)
            assert np.array_equal(got, oracle.layout_positions(layout, S, N, r, cu)), (layout, N, cu, r)


def test_per_sequence_validation(ra):
    from exact_long_context_ra_amd._lib import RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED
    lib = ra.lib()
    assert _ring_fwd(ra, _problem(ra), layout=3) == RA_ERR_INVALID_ARG  # needs cu_seqlens
    assert b"cu_seqlens" in lib.ra_last_error()
    cu_bad = (C.c_int32 * 3)(0, 20, 64)  # 20 is not a multiple of 2*world = 8
    p = _problem(ra, num_seqs=2, cu_seqlens=4096, cu_seqlens_host=C.cast(cu_bad, C.c_void_p))
    assert _ring_fwd(ra, p, layout=3) == RA_ERR_INVALID_ARG
    assert b"not divisible" in lib.ra_last_error()
    with pytest.raises(ra.RAError):
        ra.layout_posmap("zigzag_varlen", 64, 4, 0)
    assert lib.ra_layout_posmap(3, 64, 4, 0, C.byref(ra.posmap([(0, 1, 16)]))) == RA_ERR_UNSUPPORTED


def _problem(ra, **kw):
    from exact_long_context_ra_amd._lib import ra_problem
    p = ra_problem()
    p.batch, p.heads, p.head_dim, p.dtype = 1, 2, 64, 1
    p.softmax_scale, p.causal, p.seq_len = 0.0, 1, 64
    p.cu_seqlens, p.cu_seqlens_host, p.num_seqs = None, None, 0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _t(ptr=4096, sb=64 * 2 * 64, st=2 * 64, sh=64):
    from exact_long_context_ra_amd._lib import ra_tensor
    return ra_tensor(ptr, sb, st, sh)


def _ring_fwd(ra, p, layout=0, world=4, rank=0, q=None, out=None, lse=4096, srank=16 * 128 * 64):
    lib = ra.lib()
    return lib.ra_ring_fwd(C.byref(p), layout, world, rank, q or _t(), _t(), _t(), srank, out or _t(),
                           lse, _t(ptr=None), None)


def test_validation_errors(ra):
    from exact_long_context_ra_amd._lib import RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED
    lib = ra.lib()
    assert _ring_fwd(ra, _problem(ra, head_dim=96)) == RA_ERR_UNSUPPORTED
    assert b"head_dim" in lib.ra_last_error()
    assert _ring_fwd(ra, _problem(ra), rank=4) == RA_ERR_INVALID_ARG
    assert _ring_fwd(ra, _problem(ra), layout=7) == RA_ERR_INVALID_ARG
    assert _ring_fwd(ra, _problem(ra, seq_len=66)) == RA_ERR_INVALID_ARG       # 66 % 4 != 0
    assert _ring_fwd(ra, _problem(ra, seq_len=68), layout=1) == RA_ERR_INVALID_ARG  # 68 % 8 != 0
    assert _ring_fwd(ra, _problem(ra), q=_t(ptr=4098)) == RA_ERR_INVALID_ARG  # misaligned
    assert _ring_fwd(ra, _problem(ra), q=_t(st=2 * 64 + 1)) == RA_ERR_INVALID_ARG
    assert _ring_fwd(ra, _problem(ra), lse=None) == RA_ERR_INVALID_ARG
    assert _ring_fwd(ra, _problem(ra, batch=0)) == RA_ERR_INVALID_ARG
    assert _ring_fwd(ra, _problem(ra, dtype=5)) == RA_ERR_INVALID_ARG
    # varlen: device pointer required, batch 1, host copy validated
    cu_bad = (C.c_int32 * 3)(0, 40, 60)  # does not end at seq_len=64
    p = _problem(ra, num_seqs=2, cu_seqlens=4096, cu_seqlens_host=C.cast(cu_bad, C.c_void_p))
    assert _ring_fwd(ra, p) == RA_ERR_INVALID_ARG
    assert b"cu_seqlens" in lib.ra_last_error()
    cu_dec = (C.c_int32 * 3)(0, 40, 30)
    p = _problem(ra, num_seqs=2, cu_seqlens=4096, cu_seqlens_host=C.cast(cu_dec, C.c_void_p))
    assert _ring_fwd(ra, p) == RA_ERR_INVALID_ARG
    p = _problem(ra, num_seqs=2, cu_seqlens=None)
    assert _ring_fwd(ra, p) == RA_ERR_INVALID_ARG
    p = _problem(ra, num_seqs=1, cu_seqlens=4096, batch=2)
    assert _ring_fwd(ra, p) == RA_ERR_INVALID_ARG


def test_block_posmap_validation(ra):
    from exact_long_context_ra_amd._lib import RA_ERR_INVALID_ARG
    lib = ra.lib()
    p = _problem(ra)
    good = ra.posmap([(0, 1, 16)])
    dec = ra.posmap([(32, 1, 8), (0, 1, 8)])      # not increasing
    longm = ra.posmap([(60, 1, 16)])              # runs past seq_len
    short = ra.posmap([(0, 1, 15)])               # lengths do not sum to lq
    for bad in (dec, longm, short):
        st = lib.ra_block_attn_fwd(C.byref(p), _t(), 16, bad, _t(), _t(), 16, good, _t(), 4096, None)
        assert st == RA_ERR_INVALID_ARG
        st = lib.ra_block_attn_fwd(C.byref(p), _t(), 16, good, _t(), _t(), 16, bad, _t(), 4096, None)
        assert st == RA_ERR_INVALID_ARG


def test_workspace_validation(ra):
    from exact_long_context_ra_amd._lib import RA_ERR_WORKSPACE
    lib = ra.lib()
    p = _problem(ra)
    need = lib.ra_ring_workspace_min_bytes(C.byref(p), 0, 4)
    assert need == 256  # delta: batch*heads*L*4 = 1*2*16*4 = 128, rounded up to 256
    full = lib.ra_ring_workspace_bytes(C.byref(p), 0, 4)
    assert full == need + 1 * 2 * 128 * 128 * 2  # + bf16 dS^T: b*h*round_up(L, 128)^2
    p32 = _problem(ra, dtype=0)
    assert lib.ra_ring_workspace_bytes(C.byref(p32), 0, 4) == lib.ra_ring_workspace_min_bytes(C.byref(p32), 0, 4)
    st = lib.ra_ring_bwd(C.byref(p), 0, 4, 0, _t(), _t(), _t(), 0, _t(), 4096, _t(), _t(), _t(), _t(), 0,
                         4096, need - 1, None)
    assert st == RA_ERR_WORKSPACE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    import exact_long_context_ra_amd._lib as L
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "libra.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        L.lib()


def test_noalloc_rejects_before_any_gpu_call(ra):
    """The no-allocation backward checks that delta fits its fixed scratch with
    host arithmetic alone: an oversized problem is refused before any HIP call
    (this runs without a GPU) and with a message naming the limit."""
    lib = ra.lib()
    cap = lib.ra_noalloc_scratch_bytes()
    assert cap == 32 << 20
    from exact_long_context_ra_amd._lib import ra_problem, ra_tensor
    p = ra_problem()
    p.batch, p.heads, p.head_dim, p.dtype, p.causal = 1, 64, 128, 1, 1
    p.seq_len = 8 * (cap // 4 // 64 + 128)  # delta of S/8 rows x 64 heads x 4 B > cap
    t = ra_tensor(None, 0, 0, 0)
    st = lib.ra_ring_bwd_noalloc(C.byref(p), 1, 8, 0, t, t, t, 0, t, None, t, t, t, t, 0, None)
    assert st == 4  # RA_ERR_WORKSPACE
    assert b"fixed scratch" in lib.ra_last_error()


def test_default_workspace_chunks_long_blocks(ra):
    """Default backward workspace: the whole block's dS^T while each (b, h) slice
    stays under the 4 GiB a buffer descriptor addresses; beyond, dS^T chunks of
    whole 128-key tiles within 32 GiB (host arithmetic, no GPU)."""
    lib = ra.lib()
    # zigzag, 32 heads, 8 ranks: S/N = 32768 -> slice 32768^2 * 2 B = 2 GiB (whole block)
    p = _problem(ra, heads=32, head_dim=128, seq_len=8 * 32768)
    need = lib.ra_ring_workspace_min_bytes(C.byref(p), 1, 8)
    assert need == 32 * 32768 * 4
    assert lib.ra_ring_workspace_bytes(C.byref(p), 1, 8) == need + 32 * 32768 * 32768 * 2
    # S/N = 65536 -> slice 8 GiB: chunks of 32 GiB / (32 * 65536 * 2 B per key) = 8192 keys
    p = _problem(ra, heads=32, head_dim=128, seq_len=8 * 65536)
    need = lib.ra_ring_workspace_min_bytes(C.byref(p), 1, 8)
    assert lib.ra_ring_workspace_bytes(C.byref(p), 1, 8) == need + 8192 * 32 * 65536 * 2
    # S/N = 262144, 2 heads -> 1 MiB per key, but a slice must stay under 4 GiB: 8064 keys
    p = _problem(ra, heads=2, head_dim=128, seq_len=8 * 262144)
    need = lib.ra_ring_workspace_min_bytes(C.byref(p), 0, 8)
    kc = ((2 ** 32 - 1) // (262144 * 2)) // 128 * 128
    assert kc == 8064
    assert lib.ra_ring_workspace_bytes(C.byref(p), 0, 8) == need + kc * 2 * 262144 * 2


def test_slice_limit_applies_to_descriptor_operands_only(ra):
    """q/k/v/dout are read through buffer descriptors (32-bit offsets): a (batch,
    head) slice of 2 GiB or more is RA_ERR_UNSUPPORTED.  Results and accumulators
    are written through 64-bit addresses: the same slice passes their check (the
    call then stops at the next argument, a NULL lse)."""
    from exact_long_context_ra_amd._lib import RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED
    lib = ra.lib()
    huge = _t(st=1 << 24, sh=64)   # 32 MiB per row (bf16): 16 rows + the 256-row overrun pass 2 GiB
    assert _ring_fwd(ra, _problem(ra), q=huge) == RA_ERR_UNSUPPORTED
    assert b"q_local" in lib.ra_last_error()
    huge_out = _t(st=1 << 23, sh=64)  # 32 MiB per row (fp32)
    assert _ring_fwd(ra, _problem(ra), out=huge_out, lse=None) == RA_ERR_INVALID_ARG
    assert b"lse" in lib.ra_last_error()
