"""Runs tests/work_items_check.cpp, the host replay of the attention
launchers' work items (built with g++ on first use; it includes the header
the kernel and the launchers share, so it checks the ranges they use)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "work_items_check.cpp")
HEADER = os.path.join(os.path.dirname(HERE), "fp16_attention_amd", "csrc", "work_items.h")
BIN = os.path.join(HERE, ".bin", "work_items_check")


def build() -> str:
    newest = max(os.path.getmtime(SRC), os.path.getmtime(HEADER))
    if not os.path.exists(BIN) or os.path.getmtime(BIN) < newest:
        os.makedirs(os.path.dirname(BIN), exist_ok=True)
        tmp = BIN + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", "-O1", "-std=c++17", "-Wall", SRC, "-o", tmp])
        os.replace(tmp, BIN)
    return BIN


def run(mode: str, *shape, decode_as=None):
    """Run the replay; returns (exit status, output)."""
    extra = ["--decode-as", decode_as] if decode_as else []
    r = subprocess.run([build(), mode] + [str(int(x)) for x in shape] + extra, capture_output=True, text=True)
    return r.returncode, r.stdout.strip()


def check(mode: str, *shape) -> str:
    """Run the replay; returns its OK line, raises AssertionError on a failed check."""
    r = subprocess.run([build(), mode] + [str(int(x)) for x in shape], capture_output=True, text=True)
    assert r.returncode == 0, f"{mode} {shape}: {r.stdout.strip()} {r.stderr.strip()}"
    return r.stdout.strip()


def items(mode: str, *shape):
    """Every work item of the launch: dicts with b, h, qt, seg, key_begin, key_stop, key_end, list, empty."""
    r = subprocess.run([build(), mode] + [str(int(x)) for x in shape] + ["--list"], capture_output=True, text=True)
    assert r.returncode == 0, f"{mode} {shape}: {r.stdout.strip().splitlines()[-1:]}"
    keys = ("b", "h", "qt", "seg", "key_begin", "key_stop", "key_end", "list", "empty")
    out = []
    for line in r.stdout.splitlines():
        if line.startswith("OK"):
            continue
        out.append(dict(zip(keys, (int(x) for x in line.split()))))
    return out
