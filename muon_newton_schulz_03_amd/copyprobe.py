"""A plain device-to-device copy of a known size, used to calibrate the
FETCH_SIZE / WRITE_SIZE hardware counters against bytes actually moved.

    python -m muon_newton_schulz_03_amd.copyprobe --mib 1024
"""
import argparse

import torch


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--mib", type=int, default=1024)
    p.add_argument("--reps", type=int, default=3)
    a = p.parse_args()
    n = a.mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {a.mib} MiB x {a.reps}")


if __name__ == "__main__":
    main()
