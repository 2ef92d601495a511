"""The C ABI from a plain C99 program (tests/host/abi_consumer.c), run as a
child process on the GPU: resumed prefill bitwise equal to the uninterrupted
one after a checkpoint restore, in-place and fresh-page decode equal, and an
invalid call rejected with a message."""
import subprocess

import pytest

import abi_consumer_build

pytestmark = pytest.mark.gpu


def test_c_program_drives_the_library(tmp_path):
    exe = abi_consumer_build.build(str(tmp_path / "abi_consumer"))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "abi_consumer: OK" in r.stdout
