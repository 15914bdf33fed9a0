"""The package's smoke entry point (one small decode step on cuda:0 against
the oracle) passes."""
import pytest

pytestmark = pytest.mark.gpu


def test_smoke_entry_point():
    import __graft_entry__
    __graft_entry__.smoke()
