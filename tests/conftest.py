"""Shared pytest configuration: the ``gpu`` marker and GPU availability."""

import pytest


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
    except ImportError:
        return False
    return torch.cuda.is_available()


@pytest.fixture(scope="session")
def device():
    if not gpu_available():
        pytest.skip("no GPU in this environment")
    import torch

    return torch.device("cuda:0")
