"""The committed rocprofv3 summaries under profiles/ (no GPU).

Each summary must state the command that produced it, and that command must run
files of this repository only: `python3 <repo>/<script>` with the script tracked
by git, or a probe binary built here from a tracked source. The summaries are
short text, so a file that grew into raw profiler output is caught too.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _tracked():
    out = subprocess.run(["git", "ls-files"], cwd=ROOT, capture_output=True, text=True)
    if out.returncode != 0:
        pytest.skip("not a git checkout")
    return set(out.stdout.split())


def _summaries():
    return sorted(f for f in os.listdir(PROFILES) if not f.startswith("."))


def test_profiles_are_short_text_summaries():
    names = _summaries()
    assert names, "no profile summaries committed"
    for f in names:
        assert f.endswith((".txt", ".md")), f
        size = os.path.getsize(os.path.join(PROFILES, f))
        assert size < 16 * 1024, f"{f}: {size} bytes is not a short summary"


@pytest.mark.parametrize("name", _summaries())
def test_profile_commands_run_committed_files(name):
    tracked = _tracked()
    text = open(os.path.join(PROFILES, name), encoding="utf-8").read()
    cmds = [line for line in text.splitlines() if "rocprofv3" in line and " -- " in line]
    assert cmds, f"{name} names no rocprofv3 command"
    for line in cmds:
        prog = line.split(" -- ", 1)[1].split()
        if prog[0] == "python3":
            script = prog[1]
            m = re.match(r"/root/repo/(.+)", script)
            assert m, f"{name}: {script} is not a path in the repository"
            assert m.group(1) in tracked, f"{name}: {m.group(1)} is not committed"
        else:
            m = re.match(r"/root/repo/(.+)", prog[0])
            assert m, f"{name}: {prog[0]} is not a path in the repository"
            # a binary built here: its source must be committed beside it
            assert m.group(1) + ".hip" in tracked, f"{name}: no committed source for {m.group(1)}"
