import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: GLM-shape case (19 GB of weights)")
    # A planted oracle mistake for the mutation test (tests/test_oracle_mutants.py)
    name = os.environ.get("GLM_ORACLE_MUTANT")
    if name:
        sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
        import oracle_mutants

        oracle_mutants.apply(name)
