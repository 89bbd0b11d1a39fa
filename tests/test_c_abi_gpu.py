"""The library from plain C: tests/c_abi/c_abi_demo (built by
__graft_entry__.build()) calls every entry point through the C ABI alone,
with HIP-runtime memory and a stream of its own, on inputs whose results
have a closed form, and checks them on the host."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

DEMO = os.path.join(os.path.dirname(__file__), "c_abi", "c_abi_demo")


def test_plain_c_caller():
    if not os.path.exists(DEMO):
        pytest.fail(f"{DEMO} is not built; run __graft_entry__.build()")
    print("[c abi] running the plain C caller", flush=True)
    r = subprocess.run([DEMO], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi demo ok" in r.stdout
