#!/bin/bash
# Build and run the MFMA issue-rate microbenchmark (one MI355X); prints one line per case.
set -e
cd "$(dirname "$0")"
hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops mfma_issue.hip -o /tmp/mfma_issue
timeout -k 10 60 /tmp/mfma_issue
hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops mfma_overlap.hip -o /tmp/mfma_overlap
timeout -k 10 60 /tmp/mfma_overlap
