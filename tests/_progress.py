"""Progress lines from inside a running test.

pytest captures a test's output at the file-descriptor level, so a line written to
stderr from inside a test body is held until the test ends.  A long test (the
full-size parity cases run for minutes) would then print nothing while it runs.
say() suspends the capture for the one line, so it reaches the real stderr at once.
"""
import sys

_capman = None


def bind(config) -> None:
    """Called once from pytest_configure with the session's config."""
    global _capman
    _capman = config.pluginmanager.getplugin("capturemanager")


def say(line: str) -> None:
    if _capman is None:
        sys.__stderr__.write(line + "\n")
        sys.__stderr__.flush()
        return
    with _capman.global_and_fixture_disabled():
        sys.stderr.write(line + "\n")
        sys.stderr.flush()
