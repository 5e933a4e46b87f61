// gram.h -- layout of the per-chunk matrices written by chunk_gram.hip and
// read by chunk_scan_state.hip (see chunk_gram.hip for what they hold).
#pragma once

namespace prism {
namespace gram {

constexpr int kC = 64;                 // chunk length
constexpr int kBlocks = 10;            // 16x16 blocks (i, j), i >= j, of a 64x64 lower-triangular matrix
constexpr int kBlockElems = 256;
constexpr int kMatElems = kBlocks * kBlockElems;
constexpr int kChunkElems = 4 * kMatElems;   // T, A_kkw, A_qkw, -A_qk: 20 KB of bf16
enum { kMatT = 0, kMatAkkw = 1, kMatAqkw = 2, kMatNAqk = 3 };

__host__ __device__ constexpr int blk_index(int i, int j) { return i * (i + 1) / 2 + j; }

// Element (r, c) of a 16x16 block: rows of 16, the two 8-element halves
// swapped in rows 8..15.
__host__ __device__ constexpr int swz(int r, int c)
{
    return r * 16 + ((((c >> 3) ^ (r >> 3)) & 1) << 3) + (c & 7);
}

}  // namespace gram
}  // namespace prism
