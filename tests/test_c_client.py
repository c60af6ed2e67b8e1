"""The C ABI used from plain C: a C99 program (tests/c_abi/pack_host_check.c)
linked against libpg_attn.so plans the hand-written tiny batch with
pg_pack_host (no GPU) and must reproduce the fixture's position ids, pair
counts and visibility matrix (Pith review of Prefix Grouper, "What carries the
argument"; skillsmp.com "prefix-grouper-grpo", "Step 3")."""
import os
import shutil
import subprocess

import pytest

from tests.golden_io import read_visibility_fixture

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "shared_prefix_grouped_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_plans_golden_batch(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libpg_attn.so")):
        pytest.skip("libpg_attn.so is not built")
    exe = str(tmp_path / "pack_host_check")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D_POSIX_C_SOURCE=200112L",
                    os.path.join(ROOT, "tests", "c_abi", "pack_host_check.c"),
                    "-I", os.path.join(ROOT, "include"), "-L", LIBDIR, "-lpg_attn",
                    "-Wl,-rpath," + LIBDIR, "-o", exe], check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.splitlines()
    groups, positions, pairs, visible = read_visibility_fixture()
    assert groups == [(3, [2, 0, 1]), (0, [2, 1]), (1, [1, 1])]  # the layout the C program plans
    T = len(positions)
    assert out[1] == f"rows {T}"
    assert [int(x) for x in out[2].split(":")[1].split()] == list(positions)
    assert tuple(int(x) for x in out[3].split(":")[1].split()) == pairs
    assert out[4] == "visible:"
    vis = out[5:5 + T]
    assert vis == ["".join(str(int(b)) for b in row) for row in visible]
    # row_hi: the query rows that see key k are exactly [k, row_hi[k])
    row_hi = [int(x) for x in out[5 + T].split(":")[1].split()]
    for k in range(T):
        seen_by = [q for q in range(T) if vis[q][k] == "1"]
        assert seen_by == list(range(k, row_hi[k])), k
    assert out[6 + T].startswith("invalid: 1 ") and len(out[6 + T]) > len("invalid: 1 ")
