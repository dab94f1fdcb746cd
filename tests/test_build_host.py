"""The build's commands (no compilation): every HIP source is compiled for
gfx950 with packed fp32 instructions disabled, and only the forward source
gets the memory-clause scheduling strategy."""
import os

from selective_state_space_scan_amd import build as B


def _obj(src):
    return B.object_command("/tmp/x.o", src)


def test_every_source_for_gfx950_without_packed_fp32():
    for src in B.SRCS + [B.PEAKS_SRC]:
        cmd = _obj(src)
        assert "--offload-arch=gfx950" in cmd
        i = cmd.index("-packed-fp32-ops")
        assert cmd[i - 3:i] == ["-Xclang", "-target-feature", "-Xclang"]
        assert "-O3" in cmd and cmd[-4:] == ["-c", src, "-o", "/tmp/x.o"]


def test_scheduling_strategy_only_for_the_forward():
    flag = "-amdgpu-sched-strategy=max-memory-clause"
    fwd = [s for s in B.SRCS if os.path.basename(s) == "ssm_scan.hip"]
    assert len(fwd) == 1 and flag in _obj(fwd[0])
    for src in B.SRCS + [B.PEAKS_SRC]:
        if src not in fwd:
            assert flag not in _obj(src), src


def test_link_command():
    cmd = B.link_command("/tmp/lib.so", ["/tmp/a.o", "/tmp/b.o"])
    assert "-shared" in cmd and "--offload-arch=gfx950" in cmd and cmd[-2:] == ["/tmp/a.o", "/tmp/b.o"]
