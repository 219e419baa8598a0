"""Plain device-to-device copy of a known size, for calibrating HBM traffic
counters: run under `rocprofv3 --pmc FETCH_SIZE` (then `WRITE_SIZE`) and
compare the counter with the bytes moved.

    python -m video_audio_diffusion_amd.copyprobe [--mib 1024] [--reps 3]
"""
import argparse


def main():
    import torch
    ap = argparse.ArgumentParser()
    ap.add_argument("--mib", type=int, default=1024)
    ap.add_argument("--reps", type=int, default=3)
    a = ap.parse_args()
    n = a.mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {n} bytes x {a.reps}", flush=True)


if __name__ == "__main__":
    main()
