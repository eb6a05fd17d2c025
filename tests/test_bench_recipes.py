"""The profiling recipes that bench.py writes into profiles/ (no GPU needed).

Each recipe must run the program directly after ``--`` (a launcher between
rocprofv3 and the program would re-exec a process that already holds the
GPU), must not combine counter collection with tracing, and must stay within
what one counter pass can collect (8 SQ, 4 TCC, 2 GRBM counters; FETCH_SIZE
takes 3 TCC, WRITE_SIZE 2)."""

import shlex

import pytest

import bench

# derived metrics and the hardware counters they take per block
DERIVED = {
    "FETCH_SIZE": {"TCC": 3},
    "WRITE_SIZE": {"TCC": 2},
    "MfmaUtil": {"SQ": 2, "GRBM": 1},
    "VALUBusy": {"SQ": 1, "GRBM": 1},
    "LdsBankConflict": {"SQ": 2},
}
LIMITS = {"SQ": 8, "TCC": 4, "GRBM": 2}

COMMANDS = bench.profile_commands()


def _split(cmd):
    argv = shlex.split(cmd)
    assert argv[0] == "rocprofv3"
    dash = argv.index("--")
    return argv[1:dash], argv[dash + 1:]


@pytest.mark.parametrize("name", sorted(COMMANDS))
def test_program_follows_the_separator(name):
    _, prog = _split(COMMANDS[name])
    assert prog[:2] == ["python3", "bench.py"], prog
    assert not {"env", "bash", "sh", "taskset", "numactl"} & set(prog)


@pytest.mark.parametrize("name", sorted(COMMANDS))
def test_counters_never_ride_with_traces(name):
    opts, _ = _split(COMMANDS[name])
    if "--pmc" in opts:
        traces = {"-s", "--sys-trace", "-r", "--runtime-trace", "--kernel-trace", "--hip-trace", "--hsa-trace",
                  "--memory-copy-trace", "--scratch-memory-trace", "--marker-trace"}
        assert not traces & set(opts), opts


@pytest.mark.parametrize("name", sorted(n for n in COMMANDS if "--pmc" in COMMANDS[n]))
def test_one_pass_fits_the_counter_blocks(name):
    opts, _ = _split(COMMANDS[name])
    i = opts.index("--pmc") + 1
    counters = []
    while i < len(opts) and not opts[i].startswith("-"):
        counters.append(opts[i])
        i += 1
    assert counters
    use = {"SQ": 0, "TCC": 0, "GRBM": 0}
    for c in counters:
        if c in DERIVED:
            for block, n in DERIVED[c].items():
                use[block] += n
        else:
            block = c.split("_")[0]
            assert block in use, c
            use[block] += 1
    for block, n in use.items():
        assert n <= LIMITS[block], (name, block, n)


def test_every_summary_has_its_recipe():
    """Each trace and traffic summary that bench.py writes names a recipe."""
    for key in bench.TRACES:
        assert f"trace_{key}" in COMMANDS
    for key in bench.TRAFFIC:
        assert f"fetch_{key}" in COMMANDS and f"write_{key}" in COMMANDS
    for p in bench.PREFILL_PMC:
        assert f"pmc_prefill_{p}" in COMMANDS
