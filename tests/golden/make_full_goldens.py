"""Write the float64 oracle's whole-layer search results for the four large synthetic layers.

For each layer it records the oracle's loss at every ratio of the grid, its chosen ratio index,
and the sha256 of the generated activation and weight bytes the values were computed from, in
``full_search_<name>.txt`` beside this script. The GPU parity test at full size regenerates the
same bytes, checks the digests, and compares its losses and its chosen ratio with these.

Calls only the oracle (``oracle.awq_oracle.search_scales_blocked``: msModelSlim "AWQ：激活感知权重
量化算法说明", 缩放因子搜索流程, tokens in blocks) and the seeded generators (``workloads``).
Cost is the oracle's float64 work, 2 * N * d_in * d_out per ratio plus one float reference:
about 1.3 PFLOP for the 70B down_proj stress layer (an hour on an 8-core host).

    python tests/golden/make_full_goldens.py 2 3 4 5
"""
from __future__ import annotations

import argparse
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import awq_oracle as O  # noqa: E402
from workloads import make_w, make_x, to_f32, workload  # noqa: E402


def sha256_of(arr: np.ndarray) -> str:
    h = hashlib.sha256()
    flat = np.ascontiguousarray(arr).reshape(-1).view(np.uint8)
    step = 1 << 28
    for i in range(0, flat.size, step):
        h.update(flat[i:i + step])
    return h.hexdigest()


def widen(arr: np.ndarray, block: int = 4096) -> np.ndarray:
    """float64 copy of generated storage values, converted a row block at a time."""
    out = np.empty(arr.shape, dtype=np.float64)
    for r0 in range(0, arr.shape[0], block):
        out[r0:r0 + block] = to_f32(arr[r0:r0 + block])
    return out


def golden_path(name: str) -> str:
    return os.path.join(HERE, f"full_search_{name}.txt")


def make(config_id: int, block: int) -> str:
    wl = workload(config_id)
    t0 = time.time()
    x_raw, w_raw = make_x(wl), make_w(wl)
    sx, sw = sha256_of(x_raw), sha256_of(w_raw)
    X = widen(x_raw)
    del x_raw
    W = widen(w_raw)
    del w_raw
    print(f"[{wl.name}] generated and widened in {time.time() - t0:.0f} s", flush=True)
    t1 = time.time()
    res = O.search_scales_blocked(X, W, wl.group_size, wl.n_grid, block=block)
    dt = time.time() - t1
    print(f"[{wl.name}] oracle search {dt:.0f} s; k* = {res.best_k}", flush=True)
    lines = [
        f"# Float64 CPU oracle, whole-layer AWQ scale search on the synthetic layer '{wl.name}'.",
        "# Statistic mean|X| (bjdmk.com.cn AWQ article, 显著权重的识别), candidate scales and the",
        "# ratio grid k/n_grid (msModelSlim 'AWQ：激活感知权重量化算法说明', 算法公式), the INT4 group",
        "# quantizer of gsyq.cn section 二, loss = mean over all outputs of (X W^T - X What^T)^2",
        "# (gsyq section 二; bjdmk L(s)), first strict minimum (gsyq section 二).",
        "# Written by tests/golden/make_full_goldens.py (oracle.awq_oracle.search_scales_blocked,",
        f"# token blocks of {block}); values are repr() of float64.",
        f"config_id = {wl.config_id}",
        f"name = {wl.name}",
        f"n_tokens = {wl.n_tokens}",
        f"d_in = {wl.d_in}",
        f"d_out = {wl.d_out}",
        f"group_size = {wl.group_size}",
        f"n_grid = {wl.n_grid}",
        f"sha256_x = {sx}",
        f"sha256_w = {sw}",
        "losses = " + " ".join(repr(float(v)) for v in res.losses),
        f"best_k = {res.best_k}",
        f"oracle_seconds = {dt:.1f}",
    ]
    path = golden_path(wl.name)
    with open(path, "w", encoding="utf-8") as f:
        f.write("\n".join(lines) + "\n")
    print(f"[{wl.name}] wrote {path}", flush=True)
    return path


def read_golden(name: str) -> dict:
    """The key = value lines of a golden file (losses as a float64 array)."""
    kv = {}
    with open(golden_path(name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = [p.strip() for p in line.split("=", 1)]
            kv[k] = v
    kv["losses"] = np.array([float(v) for v in kv["losses"].split()])
    for k in ("config_id", "n_tokens", "d_in", "d_out", "group_size", "n_grid", "best_k"):
        kv[k] = int(kv[k])
    return kv


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("configs", type=int, nargs="+")
    ap.add_argument("--block", type=int, default=4096)
    args = ap.parse_args()
    for cid in args.configs:
        make(cid, args.block)


if __name__ == "__main__":
    main()
