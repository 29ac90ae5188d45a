"""Child-process runner for tests/test_sanitizers.py (not collected by pytest).

A library built with AddressSanitizer / UndefinedBehaviorSanitizer needs the
sanitizer runtime loaded before anything else, so the test starts this script
in a fresh interpreter with LD_PRELOAD set and reads its exit status:

    python sanitized_run.py pins <oracle.so>   every oracle pin on that build
    python sanitized_run.py abi <library.so>   tests/test_host_abi.py on that build
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)


def main(mode: str, lib: str) -> int:
    if mode == "pins":
        import oracle
        import pins
        o = oracle.Oracle(lib)
        o.set_threads(2)
        for pin in pins.ALL_PINS:
            pin(o)
            print("pin ok:", pin.__name__, flush=True)
        return 0
    if mode == "abi":
        import pytest
        import dlrm_embedding_interaction_amd as dl
        dl.LIBRARY = lib
        # -s: a sanitizer report goes to fd 2 and must not be held in pytest's capture
        return int(pytest.main(["-q", "-s", "-p", "no:cacheprovider", os.path.join(HERE, "test_host_abi.py")]))
    raise SystemExit(f"unknown mode {mode}")


if __name__ == "__main__":
    sys.exit(main(sys.argv[1], sys.argv[2]))
