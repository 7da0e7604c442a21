"""The host page allocator and planner under AddressSanitizer and
UndefinedBehaviorSanitizer: kvc_host.cpp and a replay driver
(tests/native/host_replay.cpp) built with g++ (host code only, no HIP), then
every step of the five workloads, the degenerate shapes, a scale phase and a
deferred-eviction stream with rollbacks replayed through them, each plan
checked for bounds (image size, unit addresses inside pool and page, unit
slot counts) and page-ID conservation."""
import os
import shutil
import subprocess

import pytest

import kvc_synth as syn
from tests.stream_harness import edge_workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_kvc_amd", "csrc")


def _line(wl, first_frames=1, defer=0, roll_every=0, frames=None):
    frames = wl.frames if frames is None else frames
    return " ".join(str(x) for x in (
        wl.name, wl.num_heads, wl.head_dim, wl.tokens_per_frame, wl.num_special_tokens, wl.row_offset,
        wl.page_size, wl.scale_frames, wl.sliding_window, wl.max_patch_pages, wl.max_special_pages,
        first_frames, defer, roll_every, len(frames), *frames))


def test_host_replay_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    exe = tmp_path / "host_replay"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{CSRC}", os.path.join(ROOT, "tests", "native", "host_replay.cpp"),
           os.path.join(CSRC, "kvc_host.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = [_line(wl) for wl in syn.WORKLOADS.values()]
    lines += [_line(wl, first_frames=64 if name == "steps_of_64" else 1) for name, wl in edge_workloads().items()]
    base = syn.WORKLOADS["base"]
    lines.append(_line(base, first_frames=base.scale_frames))          # scale phase, then single frames
    lines.append(_line(base, defer=1, roll_every=4))                  # deferred eviction with rollbacks
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "replay ok" in r.stdout and ", 0 failures" in r.stdout, r.stdout
