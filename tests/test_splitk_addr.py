"""CPU check of the split-K kernel's tile-copy source addresses: the kernel's
own address functions (csrc/splitk_addr.hpp), compiled for the host, are run
over every copy of every tile of items of 1..5 tiles (every tail length,
tiles past the item's end included, contiguous and paged caches, bf16 and
fp8 row layouts). Each 16-byte piece and 4-byte scale must lie in a row of a
token the item covers, within the row's used bytes, and be the token and
chunk the LDS layout expects. Offsets that went negative here once made a
copy read far outside the cache."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "splitk_addr_check")


def test_splitk_copy_addresses_stay_in_the_item():
    exe = EXE
    src = os.path.join(ROOT, "tests", "c", "splitk_addr_check.cpp")
    hdr = os.path.join(ROOT, "compressed_kv_cache_absorbed_amd", "csrc", "splitk_addr.hpp")
    if not os.path.exists(exe) or os.path.getmtime(exe) < max(os.path.getmtime(src), os.path.getmtime(hdr)):
        import __graft_entry__
        exe = __graft_entry__.build_addr_check()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) > 10_000_000
