"""Plain device-to-device copies of a known size, for calibrating memory-traffic counters.

Run under a profiler: each copy kernel reads exactly ``--mib`` MiB and writes the same amount, so
the per-dispatch counter values give the scale factor between counter units and bytes.
"""
import argparse

import torch


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=512)
    ap.add_argument("--reps", type=int, default=5)
    a = ap.parse_args()
    n = a.mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {a.mib} MiB x {a.reps}")


if __name__ == "__main__":
    main()
