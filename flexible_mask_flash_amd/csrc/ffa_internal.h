// Internal declarations shared by the host planner and the HIP launcher.
//
// The plan is a worklist of fixed-size int32 records uploaded to the device
// once per mask and read by the kernels:
//
//   header  [16]             magic, version, counts, tile shape (see kHdr*)
//   items   [num_items][16]  one main-kernel workgroup each (per batch element)
//   runs    [num_runs][8]    a contiguous range of key tiles of one slice
//   combine [num_combine][8] one split row block to merge
//
// Item:    q0, nrows, h0, run_off, n_runs, slot (-1: final output), tiles, 0,
//          then a copy of its first run record (zeros when n_runs == 0)
//          rows [q0, q0 + nrows) and query heads [h0, h0 + heads_per_item)
//          share one kv head; the item walks runs[run_off .. run_off + n_runs)
//          in order; `tiles` is the total key-tile count of those runs.  The
//          inline first run lets a workgroup issue its first K/V loads as soon
//          as its one item record has arrived (no second dependent load).
// Run:     k0, n_tiles, n_full, k_hi, edge_base, n_lead, lo_base, 0
//          key tile t covers [k0 + t*BN, k0 + (t+1)*BN); row i sees key j iff
//          i + lo_base <= j < min(k_hi, i + edge_base)  (edge_base = ke - qe + 1
//          when bit 0 of the slice type is set, else kNoEdge; lo_base = ks - qs
//          when bit 1 is set, else -kNoEdge); tiles [n_lead, n_lead + n_full)
//          are visible to every row of the item and need no mask, the first
//          n_lead and the last n_tiles - n_lead - n_full tiles do.
// Combine: q0, nrows, h0, n_chunks, slot0, 0, 0, 0
//          chunk c of row (q0 + r), head (h0 + g) is partial slot
//          slot0 + c * kSlotsPerItem + r * heads_per_item + g.
//
// With FFA_PLAN_BACKWARD the same buffer continues (header[kHdrBwd] = offset
// in int32 of this section) with the backward worklists:
//
//   bwd header [8]               n_dq_items, n_dq_runs, n_kv_items, n_kv_runs,
//                                kv_rows_per_item, dq_heads_per_item, 0, 0
//   dq items   [n_dq_items][16]  the forward's items without split (query-major)
//   dq runs    [n_dq_runs][8]
//   kv items   [n_kv_items][16]  key-major: q0/nrows are a key block, h0 is the
//                                kv head; the item walks its runs once per query
//                                head of that kv head
//   kv runs    [n_kv_runs][8]    runs of the transposed slices: k0 / k_hi are
//                                query positions and "row" is the key
// A workgroup (kWaves wavefronts) covers kSlotsPerItem = 128 (row, head) pairs
// that share one kv head: 32 rows x 4 heads, 64 x 2 or 128 x 1.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/ffa.h"

namespace ffa {

constexpr int32_t kMagic = 0x46464131;  // "FFA1"
constexpr int32_t kBlockN = 64;         // keys per tile
constexpr int32_t kWaveRows = 32;       // query rows per wavefront (one 32x32 MFMA block)
constexpr int32_t kWaves = 4;           // wavefronts per workgroup (two workgroups per CU)
constexpr int32_t kSlotsPerItem = kWaveRows * kWaves;  // (row, head) pairs one workgroup covers
constexpr int32_t kNoEdge = 0x3fffffff; // edge_base of a full slice: never limits
constexpr int kRec = 8;                 // int32 per run / combine record
constexpr int kItemRec = 16;            // int32 per item record (item fields + first run)
constexpr int kHdr = 16;                // int32 in the header

enum HeaderField {
  kHdrMagic = 0, kHdrVersion, kHdrItems, kHdrRuns, kHdrCombine, kHdrHeadsPerItem, kHdrRowsPerItem,
  kHdrBlockN, kHdrHeadDim, kHdrHeadsQ, kHdrHeadsKv, kHdrTotalQ, kHdrTotalK, kHdrSlots, kHdrBwd
};
constexpr int kBwdHdr = 8;              // int32 in the backward section's header
constexpr int32_t kKvRowsPerItem = kWaveRows * kWaves;  // keys per key-major backward item

struct Plan {
  int32_t total_q = 0, total_k = 0, heads_q = 0, heads_kv = 0, head_dim = 0;
  int32_t heads_per_item = 1, rows_per_item = 0;
  int32_t num_items = 0, num_runs = 0, num_combine = 0, num_split_items = 0;
  int32_t num_slots = 0, max_item_tiles = 0;
  int64_t visible_pairs = 0, computed_pairs = 0, total_tiles = 0;
  // backward worklists (bwd_off == 0: not planned)
  int32_t bwd_off = 0, num_dq_items = 0, num_dq_runs = 0, num_kv_items = 0, num_kv_runs = 0;
  int64_t dq_tiles = 0, kv_tiles = 0;
  std::vector<int32_t> meta;  // header + items + runs + combine (+ backward section)
  int64_t meta_bytes() const { return (int64_t)meta.size() * 4; }
  int64_t workspace_bytes() const { return (int64_t)num_slots * (head_dim + 1) * 4; }
  // backward: fp32 lse * log2 e and rowsum(dout * out) per (head, row)
  int64_t bwd_workspace_bytes() const { return bwd_off ? (int64_t)2 * heads_q * total_q * 4 : 0; }
  const int32_t* items() const { return meta.data() + kHdr; }
  const int32_t* runs() const { return items() + (size_t)num_items * kItemRec; }
  const int32_t* combine() const { return runs() + (size_t)num_runs * kRec; }
};

// Validates the problem and fills `plan`.  Returns FFA_OK or an error code
// (message in last_error()).  num_cus must be > 0.
ffa_status build_plan(const int32_t* q_ranges, const int32_t* k_ranges, const int32_t* mask_types,
                      int32_t num_slices, int32_t total_q, int32_t total_k, int32_t heads_q,
                      int32_t heads_kv, int32_t head_dim, int32_t split_tiles, int32_t max_splits,
                      int32_t num_cus, uint32_t flags, Plan* plan);

ffa_status set_error(ffa_status st, const std::string& msg);
// Validates the optional sink / softcap arguments (NULL: none).
ffa_status check_extras(const ffa_attn_extras* ex, bool has_rows);
void clear_error();
const char* last_error();

}  // namespace ffa

// The opaque handle of the C ABI.
struct ffa_plan_s {
  ffa::Plan plan;
};
