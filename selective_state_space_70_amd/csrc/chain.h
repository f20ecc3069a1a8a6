// XCD-aware placement of chunked work.
//
// A sequence split into chunks forms a chain: chunk k of a chain needs what
// chunks 0..k-1 of the same chain produced in an earlier kernel. MI355X has 8
// XCDs, each with its own L2, and workgroup i of a launch runs on XCD i % 8.
// Placing every chunk of a chain on the same XCD (in both the producing and the
// consuming kernel) keeps that hand-off inside one L2.
#pragma once

#include <hip/hip_runtime.h>

namespace ssm {

constexpr int kXcds = 8;

// (chain, position) of this workgroup on a 1-D grid laid out as
// i = (pos * per_xcd + local) * 8 + xcd with chain = local * 8 + xcd.
struct ChainSlot {
    int chain;
    int pos;
    bool valid;
};

__device__ __forceinline__ ChainSlot chain_slot(int nchains, int npos) {
    const int i = blockIdx.x;
    const int xcd = i % kXcds;
    const int j = i / kXcds;
    const int per_xcd = (nchains + kXcds - 1) / kXcds;
    ChainSlot s;
    s.pos = j / per_xcd;
    s.chain = (j % per_xcd) * kXcds + xcd;
    s.valid = s.chain < nchains && s.pos < npos;
    return s;
}

inline int chain_grid(int nchains, int npos) {
    const int per_xcd = (nchains + kXcds - 1) / kXcds;
    return per_xcd * kXcds * npos;
}

}  // namespace ssm
