// Launch geometry of every kernel of the library: how many workgroups a
// launch gets for its work. Plain C++ (no HIP), so that the arithmetic can be
// compiled and checked on the host alone.
//
// Every kernel loops over its work in grid-stride order, so a grid smaller
// than the work is still correct; the cap only keeps the launch legal. A
// launch's total thread count (workgroups x threads per workgroup) must fit
// in 32 bits, so with 256-thread workgroups the grid is capped at
// floor((2^32 - 1) / 256) = 2^24 - 1 workgroups.
#pragma once

#include <stdint.h>

namespace zs {

constexpr int kBlockThreads = 256;  // threads per workgroup, every kernel
constexpr int64_t kMaxGrid = ((int64_t(1) << 32) - 1) / kBlockThreads;  // 2^24 - 1

// ceil(units / per_block) workgroups, at least 1 and at most kMaxGrid.
inline int64_t grid_blocks(int64_t units, int64_t per_block) {
    int64_t b = units > 0 ? (units + per_block - 1) / per_block : 1;
    if (b > kMaxGrid) b = kMaxGrid;
    return b < 1 ? 1 : b;
}

// Step and reduce kernels, tiled form: one wavefront (64 lanes) per group of
// `tiles` adjacent 512-element tiles, 4 wavefronts per workgroup.
inline int64_t step_tiled_grid(int64_t S, int tiles) {
    return grid_blocks(S / (int64_t(tiles) * 512), kBlockThreads / 64);
}

// Step and reduce kernels, element-at-a-time form: one lane per element.
inline int64_t step_scalar_grid(int64_t S) { return grid_blocks(S, kBlockThreads); }

// Gather of a whole unit in one launch: one lane per 16-byte vector of the
// unit buffer (total_vecs of them).
inline int64_t gather_flat_grid(int64_t total_vecs) {
    return grid_blocks(total_vecs, kBlockThreads);
}

// Gather, one launch per shard (unaligned case): one lane per 16-byte
// vector of the shard, plus one for the head and tail elements.
inline int64_t gather_copy_grid(int64_t S, int es) {
    return grid_blocks((S * es + 15) / 16 + 1, kBlockThreads);
}

// Pack and re-shard: one workgroup per 8 KiB work item of a destination
// shard of S elements of es bytes, D destination shards.
constexpr int64_t kItemBytes = 8192;
inline int64_t items_per_shard(int64_t S, int es) {
    const int64_t per = kItemBytes / es;
    return (S + per - 1) / per;
}
inline int64_t item_grid(int64_t S, int es, int D) {
    return grid_blocks(items_per_shard(S, es) * D, 1);
}

// The stream-ceiling measurement aid: one wavefront per pair of tiles.
inline int64_t streams_grid(int64_t S, int tiles) { return step_tiled_grid(S, tiles); }

// HBM probes over nvec 16-byte vectors: a grid that covers them (reads: two
// vectors per lane) or, per_cu > 0, a persistent grid of per_cu workgroups
// on each of cu_count CUs.
inline int64_t probe_grid(bool read, int64_t nvec, int per_cu, int cu_count) {
    const int64_t lanes = read ? (nvec + 1) / 2 : nvec;
    int64_t b = grid_blocks(lanes, kBlockThreads);
    if (per_cu > 0 && b > int64_t(cu_count) * per_cu) b = int64_t(cu_count) * per_cu;
    return b;
}

}  // namespace zs
