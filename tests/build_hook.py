"""Build step of the test-support native code (run by __graft_entry__.build() as its own
process when the test tree is present): the hardware probe library under tests/hw_probe."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "hw_probe"))

import build as hw_probe_build  # noqa: E402

if __name__ == "__main__":
    print(hw_probe_build.build())
