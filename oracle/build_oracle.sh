#!/bin/sh
# Builds the CPU oracle (test infrastructure) as a shared library for ctypes.
set -e
cd "$(dirname "$0")"
g++ -std=c++17 -O2 -ffp-contract=off -fno-fast-math -Wall -Wextra -shared -fPIC \
    kvc_oracle.cpp -o liboracle.so
