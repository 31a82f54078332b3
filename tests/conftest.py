"""Shared pytest setup: the ``gpu`` marker, import paths, oracle build."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    import oracle

    srcs = [oracle._SRC, oracle._SRC_MT, os.path.join(os.path.dirname(oracle._SRC), "cachegen_oracle.h")]
    if not os.path.exists(oracle._LIB_PATH) or max(map(os.path.getmtime, srcs)) > os.path.getmtime(oracle._LIB_PATH):
        oracle.build()
    yield
