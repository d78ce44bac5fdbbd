"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): a sanitizer build of every source's host
pass, loaded with the sanitizer runtime into a child process that runs every
host-side ABI check (tests/test_abi_host.py)."""

import pytest

from sparse_top_kv_head_amd import sanitize as S


@pytest.fixture(scope="module")
def sanitized_lib():
    try:
        S.runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    return S.build_sanitized()


def test_sanitized_library_is_the_one_loaded(sanitized_lib):
    maps = S.loaded_objects()
    assert sanitized_lib in maps
    assert any("libclang_rt.asan" in m for m in maps)


def test_abi_host_checks_pass_under_sanitizers(sanitized_lib):
    r = S.run_host_tests()
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
