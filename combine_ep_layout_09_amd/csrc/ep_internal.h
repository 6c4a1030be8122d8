// ep_internal.h -- launch helpers behind the libep C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopk = 32;
constexpr int kMaxHidden = 65536;

// Workgroup width (a multiple of 64, at most 1024) and number of column tiles
// that cover a row of nvec 16-byte pieces with vpl pieces per lane.
struct TileShape {
    int threads;
    int tiles;
};
TileShape row_tile_shape(int nvec, int vpl);

// Dispatch launch shape: pieces per lane and the (token, column tile) grid's
// tile width and count.
struct DispatchShape {
    int vpl;
    TileShape tile;
};
DispatchShape dispatch_shape(int nvec, int T, bool fp8);

// Partition of the T*k routing entries into layout blocks.
struct LayoutGeometry {
    int64_t entries;   // T*k
    int32_t chunk;     // entries per block, a multiple of 256
    int32_t blocks;    // >= 1
    bool single_pass;  // one kernel, no workspace traffic
};

LayoutGeometry layout_geometry(const ep_problem& p);
LayoutGeometry layout_geometry_two_pass(const ep_problem& p);
int64_t layout_workspace_bytes(const ep_problem& p);

// Largest layout workspace of any supported problem (E = kMaxExperts): two
// tables of 64 rows by (E + 1) int32, rounded up to 256 bytes.  The
// allocation-free entry point keeps a device array of this size.
constexpr int64_t kMaxLayoutWorkspaceBytes = ((2 * 64 * (kMaxExperts + 1) * 4 + 255) / 256) * 256;

// Small routing tables (T*k entries): ep_layout and ep_layout_dispatch handle
// them in one kernel in which every workgroup reads the whole table, as long
// as the id visits of all workgroups together stay below kFusedMaxVisits.
constexpr int kFusedMaxEntries = 8192;
constexpr int64_t kFusedMaxVisits = int64_t{1} << 23;

// Mid-size tables (kFusedMaxEntries < T*k <= kWholeMaxEntries, LDS for E):
// ep_layout is one kernel in which every workgroup reads the whole table.
constexpr int kWholeMaxEntries = 65536;
constexpr int kWholeMinExperts = 32;
bool layout_whole_fits(const ep_problem& p);
hipError_t launch_layout(const ep_problem& p, const int32_t* topk_idx, const ep_layout_t& out,
                         int32_t* workspace, hipStream_t stream);
// The histogram kernel alone, with the per-block expert prefixes the ranking
// dispatch kernel of ep_layout_dispatch reads (two tables in the workspace);
// also zeroes status[1].
hipError_t launch_layout_tables(const ep_problem& p, const int32_t* topk_idx,
                                const LayoutGeometry& g, int32_t* workspace, int32_t* status,
                                hipStream_t stream);
hipError_t launch_dispatch(const ep_problem& p, const void* x, const int32_t* slot_of,
                           void* recv_x, void* recv_scales, hipStream_t stream);
hipError_t launch_layout_dispatch(const ep_problem& p, const int32_t* topk_idx,
                                  const ep_layout_t& out, void* workspace, const void* x,
                                  void* recv_x, void* recv_scales, hipStream_t stream);
// Prefill-sized tables: layout and dispatch in one launch of one workgroup
// per CU (ncu CUs), each holding its share of the rows in registers.  fits()
// says whether the problem takes that form.
bool layout_dispatch_persistent_fits(const ep_problem& p, int ncu);
hipError_t launch_layout_dispatch_persistent(const ep_problem& p, const int32_t* topk_idx,
                                             const ep_layout_t& out, const void* x, void* recv_x,
                                             void* recv_scales, int ncu, hipStream_t stream);
hipError_t launch_combine(const ep_problem& p, const void* expert_out, const int32_t* slot_of,
                          const float* topk_weights, void* y, hipStream_t stream);
hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream);

}  // namespace ep
