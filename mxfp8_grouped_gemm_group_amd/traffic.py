"""HBM traffic of the fused kernel from rocprofv3 counters.

rocprofv3's derived counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are
read for the fused kernel and for a plain device copy of known size (1 GiB read
+ 1 GiB written per dispatch, ``bench.py --copy-calibration``).  The copy gives
the scale of each counter on this part (bytes the counter reports per byte
actually moved); the kernel's counts are divided by it:

    traffic = FETCH_SIZE(kernel) / (FETCH_SIZE(copy) / 1 GiB)
            + WRITE_SIZE(kernel) / (WRITE_SIZE(copy) / 1 GiB)

Collection (four counter runs, each its own process; see the profiles folder
for the exact commands):

    rocprofv3 --pmc FETCH_SIZE -d DIR/copy_fetch  -o p --output-format csv -- python bench.py --copy-calibration --steps 3 --warmup 1
    rocprofv3 --pmc WRITE_SIZE -d DIR/copy_write  -o p --output-format csv -- python bench.py --copy-calibration --steps 3 --warmup 1
    rocprofv3 --pmc FETCH_SIZE -d DIR/W_fetch     -o p --output-format csv -- python bench.py --workload W --steps 3 --warmup 1 --no-cpu-baseline
    rocprofv3 --pmc WRITE_SIZE -d DIR/W_write     -o p --output-format csv -- python bench.py --workload W --steps 3 --warmup 1 --no-cpu-baseline
    python -m mxfp8_grouped_gemm_group_amd.traffic DIR W

The result goes to ``profiles/traffic_W.json`` together with a hash of the
kernel source it was measured on; ``recorded_traffic`` returns None once the
source has changed.

``python -m mxfp8_grouped_gemm_group_amd.traffic counters DIR W`` summarises
the other counter passes of workload W (one rocprofv3 run each, directories
DIR/W_<pass>; the copy's DIR/copy_rdreq for the request-size cross-check) into
``profiles/counters_W.json``: per-dispatch means (dispatches after the first)
of every counter found, and the figures derived from them (see ``derive``).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
_KERNEL_SRC = os.path.join(_PKG, "csrc", "gfr_kernels.hip")
GIB = 1 << 30


def kernel_hash() -> str:
    with open(_KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def kernel_name(workload: str) -> str:
    """The library kernel a workload's bench run launches."""
    return "gemm1_swiglu_kernel" if workload.startswith("g1_") else "fused_kernel"


def _per_dispatch(run_dir: str, counter: str, name_part: str):
    """Counter value (summed over its dimensions) of every dispatch whose kernel
    name contains name_part, in dispatch order."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter or name_part not in r["Kernel_Name"]:
                    continue
                k = int(r["Dispatch_Id"])
                per[k] = per.get(k, 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def _steady(values):
    """Mean over the dispatches after the first (the first one warms caches)."""
    if not values:
        raise ValueError("no matching dispatches")
    v = values[1:] if len(values) > 1 else values
    return sum(v) / len(v)


def compute(run_dir: str, workload: str) -> dict:
    copy_kernel = "copy"   # torch's device copy kernels carry "copy" in their names
    f_copy = _steady(_per_dispatch(os.path.join(run_dir, "copy_fetch"), "FETCH_SIZE", copy_kernel))
    w_copy = _steady(_per_dispatch(os.path.join(run_dir, "copy_write"), "WRITE_SIZE", copy_kernel))
    kname = kernel_name(workload)
    f_k = _steady(_per_dispatch(os.path.join(run_dir, f"{workload}_fetch"), "FETCH_SIZE", kname))
    w_k = _steady(_per_dispatch(os.path.join(run_dir, f"{workload}_write"), "WRITE_SIZE", kname))
    f_scale = f_copy * 1024 / GIB      # counter bytes per real byte read
    w_scale = w_copy * 1024 / GIB
    read_b = f_k * 1024 / f_scale
    write_b = w_k * 1024 / w_scale
    return {
        "workload": workload,
        "kernel": kname,
        "kernel_source_sha256_16": kernel_hash(),
        "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "kernel_fetch_kib": f_k, "kernel_write_kib": w_k,
        "bytes_read": read_b, "bytes_written": write_b,
        "bytes_per_launch": read_b + write_b,
    }


# Counter passes and their counters (each pass is one rocprofv3 run; the
# block limits of one run: 8 SQ, 4 TCC, 1 GRBM here).
PASSES = {
    "rdreq": ["TCC_EA0_RDREQ", "TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_128B"],
    "l2": ["TCC_HIT", "TCC_MISS", "TCC_ATOMIC", "TCC_EA0_ATOMIC"],
    "sq": ["SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4",
           "SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
           "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"],
    "util": ["MfmaUtil"],
}


def _counters(run_dir: str, name_part: str) -> dict:
    """{counter: steady per-dispatch mean} of every counter in one pass's run."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    names = set()
    for fn in files:
        with open(fn) as f:
            names |= {r["Counter_Name"] for r in csv.DictReader(f)}
    return {n: _steady(_per_dispatch(run_dir, n, name_part)) for n in sorted(names)}


def derive(c: dict, copy_rdreq: Optional[dict]) -> dict:
    """Figures from the raw counter means of one dispatch.

    * read bytes from request counts: 128 * RDREQ_128B + 64 * RDREQ_64B +
      32 * RDREQ_32B (a cross-check of the copy-scaled FETCH_SIZE); for the
      copy the same sum over its 1 GiB read gives the counters' own scale;
    * L2 hit rate TCC_HIT / (TCC_HIT + TCC_MISS);
    * matrix-core work: MOPS counters count 512 operations each, so FLOPs =
      512 * (MOPS_F8 + MOPS_F6F4 + MOPS_I8);
    * MFMA busy fraction: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs)
      -- GRBM_GUI_ACTIVE is summed over the 8 XCDs here, so per XCD it is
      GRBM_GUI_ACTIVE / 8, and 1024 SIMDs (256 CUs x 4);
    * LDS bank conflicts per LDS access cycle.
    """
    d = {}
    if "TCC_EA0_RDREQ_128B" in c:
        rd = 128 * c["TCC_EA0_RDREQ_128B"] + 64 * c.get("TCC_EA0_RDREQ_64B", 0.0) + \
            32 * c.get("TCC_EA0_RDREQ_32B", 0.0)
        d["read_bytes_from_requests"] = rd
        if copy_rdreq and "TCC_EA0_RDREQ_128B" in copy_rdreq:
            crd = 128 * copy_rdreq["TCC_EA0_RDREQ_128B"] + \
                64 * copy_rdreq.get("TCC_EA0_RDREQ_64B", 0.0) + \
                32 * copy_rdreq.get("TCC_EA0_RDREQ_32B", 0.0)
            d["copy_read_bytes_from_requests"] = crd
            d["request_bytes_per_real_byte"] = crd / GIB
            d["read_bytes_from_requests_scaled"] = rd / (crd / GIB)
    if "TCC_HIT" in c and "TCC_MISS" in c and c["TCC_HIT"] + c["TCC_MISS"] > 0:
        d["l2_hit_rate"] = c["TCC_HIT"] / (c["TCC_HIT"] + c["TCC_MISS"])
    mops = sum(c.get(k, 0.0) for k in ("SQ_INSTS_VALU_MFMA_MOPS_F8",
                                       "SQ_INSTS_VALU_MFMA_MOPS_F6F4",
                                       "SQ_INSTS_VALU_MFMA_MOPS_I8"))
    if mops:
        d["mfma_flops"] = 512.0 * mops
    if "SQ_VALU_MFMA_BUSY_CYCLES" in c and c.get("GRBM_GUI_ACTIVE", 0) > 0:
        d["mfma_busy_frac"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / 8 * 1024)
        d["gpu_active_cycles_per_xcd"] = c["GRBM_GUI_ACTIVE"] / 8
    if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_LDS_IDX_ACTIVE", 0) > 0:
        d["lds_bank_conflicts_per_access"] = c["SQ_LDS_BANK_CONFLICT"] / max(
            c["SQ_LDS_IDX_ACTIVE"] - c["SQ_LDS_BANK_CONFLICT"], 1.0)
    return d


def counters(run_dir: str, workload: str) -> dict:
    kname = kernel_name(workload)
    raw = {}
    for p in PASSES:
        pdir = os.path.join(run_dir, f"{workload}_{p}")
        if os.path.isdir(pdir):
            raw.update(_counters(pdir, kname))
    cdir = os.path.join(run_dir, "copy_rdreq")
    copy_rd = _counters(cdir, "copy") if os.path.isdir(cdir) else None
    return {"workload": workload, "kernel": kname, "kernel_source_sha256_16": kernel_hash(),
            "counters_per_dispatch": raw, "copy_rdreq_per_dispatch": copy_rd,
            "derived": derive(raw, copy_rd)}


def recorded_traffic(workload: str) -> Optional[float]:
    fn = os.path.join(_ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        d = json.load(f)
    if d.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return d.get("bytes_per_launch")


def main(argv):
    if len(argv) == 4 and argv[1] == "counters":
        d = counters(argv[2], argv[3])
        out = os.path.join(_ROOT, "profiles", f"counters_{argv[3]}.json")
        with open(out, "w") as f:
            json.dump(d, f, indent=1)
        print(json.dumps(d, indent=1))
        return 0
    if len(argv) != 3:
        print("usage: python -m mxfp8_grouped_gemm_group_amd.traffic RUN_DIR WORKLOAD", file=sys.stderr)
        return 2
    d = compute(argv[1], argv[2])
    out = os.path.join(_ROOT, "profiles", f"traffic_{argv[2]}.json")
    with open(out, "w") as f:
        json.dump(d, f, indent=1)
    print(json.dumps(d, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
