"""Host-side logic of bench.py (no GPU): which launches the timed steps put
events around, and where the traffic figures it reports come from."""
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


class _FakeEvent:
    def __init__(self, log, enable_timing=True):
        self.log = log

    def record(self):
        self.log.append("event")

    def elapsed_time(self, other):
        return 1.0


class _FakeTorch:
    def __init__(self):
        self.log = []
        outer = self

        class _Cuda:
            @staticmethod
            def Event(enable_timing=True):
                return _FakeEvent(outer.log, enable_timing)

        self.cuda = _Cuda()


def test_kernel_timer_brackets_only_the_named_launches():
    t = _FakeTorch()
    tm = bench.KernelTimer(t, only=("logits",))
    for name in ("logits", "xent_fused", "dgrad"):
        tm(name, lambda name=name: t.log.append(name))
    assert t.log == ["event", "logits", "event", "xent_fused", "dgrad"]
    assert tm.ms("logits") == [1.0] and tm.ms("dgrad") == []
    t2 = _FakeTorch()
    every = bench.KernelTimer(t2)
    every("a", lambda: t2.log.append("a"))
    every("b", lambda: t2.log.append("b"))
    assert t2.log == ["event", "a", "event", "event", "b", "event"]
    quiet = bench.KernelTimer(t2, only=())
    assert quiet("a", lambda: 7) == 7 and quiet.ms("a") == []


def test_source_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    csrc = tmp_path / "lm_head_fp32_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("int f() { return 1; } // one\n/* block\n comment */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_code_hash("k.hip")
    (csrc / "k.hip").write_text("int  f()\n{ return 1; }   // another comment\n")
    assert bench.source_code_hash("k.hip") == h
    (csrc / "k.hip").write_text("int f() { return 2; }\n")
    assert bench.source_code_hash("k.hip") != h


def test_traffic_figures_come_from_the_committed_profile():
    """Every source hash bench.py keys a measured traffic figure on is the
    one the committed rocprofv3 summary names, and the figure is the
    calibrated sum that summary's table gives (2 x FETCH_SIZE + WRITE_SIZE)."""
    with open(os.path.join(ROOT, "profiles", "bench_kernel_trace_and_traffic.md")) as f:
        prof = f.read()
    header = re.search(r"whitespace removed\): (.*?)\.\n", prof, flags=re.S).group(1)
    named = dict(re.findall(r"(\w+\.hip) ([0-9a-f]{16})", header))
    for key, t in bench.MEASURED_TRAFFIC.items():
        assert named.get(t["src"]) == t["sha"], key
    table = {m.group(1): int(m.group(2).replace(",", ""))
             for m in re.finditer(r"^\| (\S+?)[< ].*?= ([0-9,]+) \| [0-9.]+ \|$", prof, flags=re.M)}
    want = {"logits_fp32": "gemm_persist", "xent_fwd_bwd_fp32": "xent_fwd_kernel",
            "xent_fused_bf16_1024x32768": "xent_fused_kernel"}
    for key, kname in want.items():
        assert abs(bench.MEASURED_TRAFFIC[key]["bytes"] - table[kname]) <= 1, key


def test_profiles_name_the_current_kernel_sources():
    """Each rocprofv3 summary under profiles/ states the source hash of the
    kernels it measured; those are the sources in the tree (a kernel changed
    since its profile was taken would make the summary describe other code)."""
    pdir = os.path.join(ROOT, "profiles")
    seen = 0
    for fn in sorted(os.listdir(pdir)):
        with open(os.path.join(pdir, fn)) as f:
            text = f.read()
        for name, sha in re.findall(r"(\w+\.hip) ([0-9a-f]{16})", text):
            assert bench.source_code_hash(name) == sha, (fn, name)
            seen += 1
    assert seen >= 3
