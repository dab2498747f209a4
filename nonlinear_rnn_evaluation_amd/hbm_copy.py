"""A plain device copy of known size, used to calibrate hardware byte counters.

    python -m nonlinear_rnn_evaluation_amd.hbm_copy [MiB]

Copies a float32 buffer of MiB mebibytes (default 1024) into another one three times;
the FETCH_SIZE / WRITE_SIZE counters read for this copy, divided by the bytes it must
move, give the factor by which the counters of the Newton kernels are scaled.
"""
import sys

import torch


def main():
    mib = int(sys.argv[1]) if len(sys.argv) > 1 else 1024
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x3")


if __name__ == "__main__":
    main()
