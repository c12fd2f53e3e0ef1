"""CPU checks that the committed measurement files still describe this code: the
HBM counters of the 1 GiB message were taken on the current kernel sources (else
the benchmark reports no measured traffic), and every command a profile summary
gives runs committed files with options the benchmark still has."""
import os
import re
import shlex
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")
SUMMARIES = sorted(f for f in os.listdir(PROFILES) if f.endswith(".md"))


@pytest.mark.parametrize("kernel", ["stage1", "owner", "decode"])
def test_headline_counters_match_the_kernel_sources(kernel):
    got = bench.measured_traffic(kernel, bench.workload_tag(True))
    assert got is not None, "profiles/traffic_counters.json was taken on other kernel sources"
    assert got > 0


def _bench_invocations(text):
    """The argument lists that follow `bench.py` in a summary's commands."""
    out = []
    for line in text.splitlines():
        for m in re.finditer(r"bench\.py((?:\s+[^`|>]+)?)", line):
            out.append(shlex.split(m.group(1).strip()) if m.group(1) else [])
    return out


@pytest.mark.parametrize("name", SUMMARIES)
def test_profile_commands_use_existing_options(name):
    with open(os.path.join(PROFILES, name)) as f:
        text = f.read()
    options = {o for a in bench.make_parser()._actions for o in a.option_strings}
    for args in _bench_invocations(text):
        for i, tok in enumerate(args):
            if tok.startswith("--"):
                assert tok in options, f"{name}: bench.py has no option {tok}"
            if tok == "--config":
                assert args[i + 1] in set(bench.REPORTS) | {"all"}, f"{name}: no report {args[i + 1]}"
    for path in re.findall(r"<repo>/([\w./-]+)", text):
        assert os.path.exists(os.path.join(ROOT, path)), f"{name}: {path} is not in the repository"


def test_every_summary_gives_its_command():
    for name in SUMMARIES:
        with open(os.path.join(PROFILES, name)) as f:
            text = f.read()
        assert "Command" in text and "bench.py" in text, name
