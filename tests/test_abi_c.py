"""The boundary is a C ABI: include/ra.h compiles as strict C99 and a C program
links libra.so and calls it.  Host-only entry points (no GPU needed): version,
status strings, layout positions and posmaps, workspace sizing, and a
validation error reported before anything is enqueued."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "exact_long_context_ra_amd")

C_SOURCE = r"""
#include <stdio.h>
#include <string.h>
#include "ra.h"

int main(void) {
  int64_t zz[8], st[2];
  ra_posmap m;
  ra_problem p;
  ra_tensor t;
  ra_status s;
  int i;
  printf("abi %d %d\n", ra_abi_version(), RA_ABI_VERSION);
  s = ra_layout_positions(RA_LAYOUT_ZIGZAG, 16, 2, 0, zz);
  printf("zigzag %d", (int)s);
  for (i = 0; i < 8; ++i) printf(" %lld", (long long)zz[i]);
  printf("\n");
  s = ra_layout_positions(RA_LAYOUT_STRIPE, 8, 4, 1, st);
  printf("stripe %d %lld %lld\n", (int)s, (long long)st[0], (long long)st[1]);
  s = ra_layout_posmap(RA_LAYOUT_ZIGZAG, 16, 2, 1, &m);
  printf("posmap %d %d %lld %lld %lld %lld %lld %lld\n", (int)s, (int)m.nseg, (long long)m.seg[0].begin,
         (long long)m.seg[0].stride, (long long)m.seg[0].len, (long long)m.seg[1].begin,
         (long long)m.seg[1].stride, (long long)m.seg[1].len);
  memset(&p, 0, sizeof p);
  p.batch = 1;
  p.heads = 32;
  p.head_dim = 128;
  p.dtype = RA_DTYPE_BF16;
  p.causal = 1;
  p.seq_len = 131072;
  printf("workspace %zu %zu\n", ra_ring_workspace_min_bytes(&p, RA_LAYOUT_ZIGZAG, 8),
         ra_ring_workspace_bytes(&p, RA_LAYOUT_ZIGZAG, 8));
  memset(&t, 0, sizeof t);
  s = ra_ring_fwd(&p, RA_LAYOUT_ZIGZAG, 8, 8, t, t, t, 0, t, NULL, t, NULL);
  printf("error %d %s\n", (int)s, ra_status_str(s));
  printf("message %s\n", ra_last_error());
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_c99_and_library_links_from_c(tmp_path):
    lib = os.path.join(PKG, "libra.so")
    if not os.path.exists(lib):
        pytest.skip("libra.so is not built")
    src = tmp_path / "abi.c"
    src.write_text(C_SOURCE)
    exe = tmp_path / "abi"
    cmd = ["gcc", "-std=c99", "-pedantic-errors", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L", PKG, "-l:libra.so", "-Wl,-rpath," + PKG]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    out = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    abi, abi_macro = out["abi"].split()
    assert abi == abi_macro
    # zigzag, 16 tokens on 2 ranks: chunks of 4, rank 0 holds chunks 0 and 3
    assert out["zigzag"].split() == ["0", "0", "1", "2", "3", "12", "13", "14", "15"]
    # stripe, 8 tokens on 4 ranks: rank 1 holds tokens 1 and 5
    assert out["stripe"].split() == ["0", "1", "5"]
    # zigzag rank 1 of 2: chunk 1 (positions 4..7) then chunk 2 (8..11)
    assert out["posmap"].split() == ["0", "2", "4", "1", "4", "8", "1", "4"]
    wmin, wfull = (int(x) for x in out["workspace"].split())
    assert wmin == 4 * 32 * (131072 // 8)          # delta: 4 B per local row and head
    assert wfull > wmin                            # plus the bf16 dS^T of a step
    assert out["error"].split() == ["1", "RA_ERR_INVALID_ARG"]  # rank 8 of a ring of 8
    assert "rank" in out["message"]
